"""The append kernel's quotient: y = x / d for the 8- and 4-bit codes, computed without a
division per element, gives the same codes as the fp32 IEEE quotient for every input.

The kernel takes r0 = the hardware reciprocal of d (within one ulp of 1 / d), refines it
with one Newton step r = fma(fma(-d, r0, 1), r0, r0), and corrects the quotient x r once
with Markstein's step y = fma(fma(-d, t, x), r, t).  The argument, each premise pinned
below by exact arithmetic on the CPU:

  1. for every positive finite fp16 d (the scale is an fp16 value) and every fp32 r0 within
     one ulp of 1 / d, the Newton step gives exactly r = RN(1 / d) (exhaustive, exact
     rationals);
  2. with that r, the corrected quotient is within 0.5 ulp + 3 * 2^-24 ulp of x / d (first
     quotient within 1.5 ulp, residual rounded at most once, final rounding): checked
     against exact rationals on random inputs;
  3. so the code round_half_away(y), clamped, can differ from the IEEE quotient's code only
     where the two quotients straddle a boundary k + 1/2, i.e. for x within an ulp or so of
     (k + 1/2) d.  For every positive fp16 d and k = 0 .. 127, every x within six ulps of
     (k + 1/2) d (both signs), plus random and subnormal inputs, gives the IEEE quotient bit
     for bit (wherever |x / d| >= 2^-30) and the same 8- and 4-bit codes everywhere: about
     10^8 cases.

The kernel then rounds the quotient half away from zero as trunc(clamp(y + copysign(1/2 -
2^-25, y), -qmax, qmax)); the last test checks that identity for every fp32 y with |y| in
[2^-30, 512) (below, both sides give 0; above, both clamp; the sign is symmetric).

fp32 fma is emulated exactly: the product of two fp32 values is exact in fp64, the fp64 sum
carries its exact rounding error (TwoSum), and the one case where rounding the fp64 sum to
fp32 could differ from rounding the exact sum (the fp64 sum sitting on an fp32 midpoint) is
decided by that error's sign.  The emulation is itself checked against exact rationals.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def rn32(fr: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to fp32 (normal or subnormal)."""
    if fr == 0:
        return np.float32(0.0)
    if fr < 0:
        return -rn32(-fr)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(fr, ulp)
    q = int(q)
    if r > ulp / 2 or (r == ulp / 2 and q % 2 == 1):
        q += 1
    return np.float32(float(q * ulp))


def _rn32_of_sum(s: np.ndarray, err: np.ndarray) -> np.ndarray:
    """RN to fp32 of the exact value s + err, s an fp64 sum and err its exact rounding error."""
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    on_mid_up = (s - r64) == (up.astype(np.float64) - r64) / 2
    on_mid_dn = (r64 - s) == (r64 - dn.astype(np.float64)) / 2
    out = np.where(on_mid_dn & (err < 0), dn, r)
    return np.where(on_mid_up & (err > 0), up, out)


def fma32(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """RN32(a b + c) for fp32 arrays, exactly."""
    p = a.astype(np.float64) * b.astype(np.float64)   # exact: 48 significant bits
    c64 = c.astype(np.float64)
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)                  # TwoSum: s + err == p + c exactly
    return _rn32_of_sum(s, err)


def kernel_quotient(x: np.ndarray, d: np.float32, r: np.float32) -> np.ndarray:
    """The kernel's sequence: a first quotient and one Markstein correction."""
    dd = np.full_like(x, d)
    rr = np.full_like(x, r)
    t = (x.astype(np.float64) * np.float64(r)).astype(np.float32)
    return fma32(fma32(-dd, t, x), rr, t)


def codes(y: np.ndarray, qmax: int) -> np.ndarray:
    """round_half_away, then clamp to [-qmax, qmax] (the stored format)."""
    t = np.trunc(y)
    r = np.where(np.abs(y - t) >= 0.5, t + np.sign(y), t)
    return np.clip(r, -qmax, qmax)


def positive_fp16_scales() -> np.ndarray:
    return np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)


def test_fma_emulation_is_exact():
    rng = np.random.default_rng(5)
    n = 4000
    a = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    b = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    # c close to -a b, so that the sum cancels and its rounding is delicate
    c = (-(a.astype(np.float64) * b) * (1 + rng.standard_normal(n) * 2.0 ** -rng.integers(10, 40, n))).astype(np.float32)
    got = fma32(a, b, c)
    for i in range(n):
        want = rn32(Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i])))
        assert got[i] == want, (a[i], b[i], c[i])


def test_newton_step_gives_the_rounded_reciprocal_of_every_fp16_scale():
    n_cases = 0
    for d in positive_fp16_scales():
        inv = 1 / Fraction(float(d))
        want = rn32(inv)
        ulp = Fraction(float(np.spacing(np.float32(float(inv)))))
        cands = {want}
        lo = hi = want
        for _ in range(2):
            lo = np.nextafter(lo, np.float32(0))
            hi = np.nextafter(hi, np.float32(np.inf))
            cands |= {lo, hi}
        for r0 in cands:
            if abs(Fraction(float(r0)) - inv) > ulp:      # outside the reciprocal's one-ulp bound
                continue
            n_cases += 1
            e = rn32(1 - Fraction(float(d)) * Fraction(float(r0)))
            r = rn32(Fraction(float(r0)) + Fraction(float(e)) * Fraction(float(r0)))
            assert r == want, (d, r0)
    assert n_cases > 2 * 31743 - 100


def test_corrected_quotient_is_within_half_an_ulp_and_a_sliver():
    rng = np.random.default_rng(11)
    ds = positive_fp16_scales()
    for d in ds[rng.integers(0, ds.size, 300)]:
        r = rn32(1 / Fraction(float(d)))
        x = (rng.uniform(-130, 130, 60) * np.float64(d)).astype(np.float32)
        y = kernel_quotient(x, d, r)
        for xi, yi in zip(x, y):
            q = Fraction(float(xi)) / Fraction(float(d))
            if q == 0:
                assert yi == 0
                continue
            ulp = Fraction(float(np.spacing(np.float32(abs(float(q))))))
            assert abs(Fraction(float(yi)) - q) <= ulp / 2 + 3 * ulp / 2 ** 24, (d, xi)


def test_corrected_quotient_equals_the_division_where_it_decides_a_code():
    rng = np.random.default_rng(7)
    ks = np.arange(128, dtype=np.float64) + 0.5
    tiny = np.array([1e-45, -1e-45, 1e-40, 2.0 ** -126, -3e-39], np.float32)
    n_cases = 0
    for d in positive_fp16_scales():
        r = rn32(1 / Fraction(float(d)))
        base = (ks * np.float64(d)).astype(np.float32)
        xs = [base]
        up = dn = base
        for _ in range(6):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
            xs += [up, dn]
        x = np.concatenate(xs)
        x = np.concatenate([x, -x, (rng.uniform(-130, 130, 64) * np.float64(d)).astype(np.float32), tiny])
        y = kernel_quotient(x, d, r)
        want = x / np.full_like(x, d)                 # IEEE fp32 division
        same = y.view(np.uint32) == want.view(np.uint32)
        assert np.all(same | (np.abs(want) < 2.0 ** -30)), d
        for qmax in (127, 7):
            assert np.array_equal(codes(y, qmax), codes(want, qmax)), (d, qmax)
        n_cases += x.size
    assert n_cases > 10 ** 8


def test_code_rounding_identity_for_every_quotient():
    c = np.float32(0.5) - np.float32(2.0 ** -25)
    lo = int(np.float32(2.0 ** -30).view(np.uint32))
    hi = int(np.float32(512.0).view(np.uint32))
    n = 0
    for start in range(lo, hi, 1 << 24):
        y = np.arange(start, min(start + (1 << 24), hi), dtype=np.uint32).view(np.float32)
        y64 = y.astype(np.float64)
        s = y64 + np.float64(c)
        bb = s - y64
        t = _rn32_of_sum(s, (y64 - (s - bb)) + (np.float64(c) - bb))   # RN32(y + c), exactly
        for qmax in (127, 7):
            got = np.trunc(np.minimum(np.maximum(t, np.float32(-qmax)), np.float32(qmax)))
            want = np.clip(np.floor(y64 + 0.5), -qmax, qmax)   # y + 1/2 is exact in fp64 here
            assert np.array_equal(got, want), (start, qmax)
        n += y.size
    assert n == hi - lo
    # the plain addend 1/2 would fail at |y| = 1/2 - 2^-25: the pin has teeth
    y = np.float32(0.5) - np.float32(2.0 ** -25)
    assert np.trunc(y + np.float32(0.5)) == 1.0 and np.trunc(y + c) == 0.0


def test_the_boundary_check_catches_plausible_mistakes():
    """The boundary cases above fail a quotient without the correction step, and one with
    the residual's sign flipped (planted on the CPU, on every 64th fp16 scale)."""
    ks = np.arange(128, dtype=np.float64) + 0.5
    no_corr = flipped = 0
    for d in positive_fp16_scales()[::64]:
        r = rn32(1 / Fraction(float(d)))
        base = (ks * np.float64(d)).astype(np.float32)
        x = np.concatenate([base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))])
        want = codes(x / np.full_like(x, d), 127)
        t = (x.astype(np.float64) * np.float64(r)).astype(np.float32)
        no_corr += int(np.sum(codes(t, 127) != want))
        dd, rr = np.full_like(x, d), np.full_like(x, r)
        flipped += int(np.sum(codes(fma32(fma32(dd, t, x), rr, t), 127) != want))
    assert no_corr > 0 and flipped > 0

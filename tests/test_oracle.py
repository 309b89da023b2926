"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own formula: footprints come from the
page's printed table, scales and codes from exact rational arithmetic and Python's
``struct`` half-precision packing, attention from pure-Python loops, closed forms and
invariants.  A dropped term, a wrong sign, index or rounding mode in the oracle fails
at least one of them.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

import oracle as O
from asymmetric_quantized_kv_amd import inputs as I

GOLD = Path(__file__).parent / "golden"


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------
def f32_nearest(fr: Fraction) -> float:
    """Exact round-to-nearest-even of a non-negative rational to fp32 (normal or subnormal)."""
    if fr == 0:
        return 0.0
    assert fr > 0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    e = max(e, -126)                       # subnormals share the 2^-126 binade spacing
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(fr, ulp)
    q = int(q)
    if r > ulp / 2 or (r == ulp / 2 and q % 2 == 1):
        q += 1
    return float(q * ulp)


def f16_bits_struct(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


def rhaz_exact(fr: Fraction) -> int:
    a = abs(fr)
    n = math.floor(a + Fraction(1, 2))
    return n if fr >= 0 else -n


def ref_block(xs, bits):
    """(d fp16 bits, codes) from exact arithmetic: d = fp16(RN32(amax / qmax)) saturated."""
    qmax = 127 if bits == 8 else 7
    xs32 = [float(np.float32(x)) for x in xs]
    amax = max(abs(x) for x in xs32)
    d32 = min(f32_nearest(Fraction(amax) / qmax), 65504.0)
    dbits = f16_bits_struct(d32)
    d = struct.unpack("<e", struct.pack("<H", dbits))[0]
    if d == 0:
        return dbits, [0] * len(xs32)
    codes = [max(-qmax, min(qmax, rhaz_exact(Fraction(x) / Fraction(d)))) for x in xs32]
    return dbits, codes


def oracle_block(xs, bits):
    x = np.zeros((1, 32), np.float32)
    x[0, :len(xs)] = xs
    q, d = O.quantize_rows(x, bits)
    return int(d.view(np.uint16)[0, 0]), [int(v) for v in q[0]]


# ---------------------------------------------------------------------------
# footprint: the page's printed table
# ---------------------------------------------------------------------------
def _footprint_rows():
    rows, savings = [], []
    for ln in (GOLD / "footprint_kvsplit.txt").read_text().splitlines():
        ln = ln.split("#")[0].strip()
        if not ln:
            continue
        a, b, c = ln.split()
        (savings if a == "saving" else rows).append((a, b, c))
    return rows, savings


@pytest.mark.parametrize("tokens,layout,printed", _footprint_rows()[0])
def test_footprint_matches_printed_table(tokens, layout, printed):
    got = O.layout_footprint_bytes(O.LAYOUT_IDS[layout], 22, 4, 64, int(tokens))
    assert f"{got / 2**20:.2f}" == printed


def test_footprint_savings_percent():
    fp16 = O.layout_footprint_bytes(0, 22, 4, 64, 8192)
    for _, layout, pct in _footprint_rows()[1]:
        got = O.layout_footprint_bytes(O.LAYOUT_IDS[layout], 22, 4, 64, 8192)
        assert round(100 * (1 - got / fp16)) == int(pct)


def test_footprint_context_ratio():
    # "K8V4 saves 59% ... about 2.4 times the context" (KVSplit page, Hacker News section)
    r = O.layout_footprint_bytes(0, 22, 4, 64, 8192) / O.layout_footprint_bytes(2, 22, 4, 64, 8192)
    assert 2.4 <= r < 2.5


def test_cache_object_footprint_and_capacity_granule():
    for layout in range(6):
        c = O.OracleCache(layout, 2, 3, 64, 300)
        assert c.cap == 512
        assert c.footprint_bytes() == O.layout_footprint_bytes(layout, 2, 3, 64, 300)


# ---------------------------------------------------------------------------
# scale and codes: exact arithmetic and Python's half packing
# ---------------------------------------------------------------------------
def test_fp16_cast_matches_struct():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 100,
                        rng.standard_normal(2000).astype(np.float32) * 1e-5])
    # exact fp16 midpoints and their fp32 neighbours
    h = rng.integers(0x0400, 0x7BFF, 2000).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (h + np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)) / 2
    m32 = mid.astype(np.float32)
    x = np.concatenate([x, m32, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))])
    got = O.f32_to_f16(x).view(np.uint16)
    want = np.array([f16_bits_struct(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bits", [8, 4])
def test_block_scale_exact(bits):
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(bits)
    amax = list(np.abs(rng.standard_normal(3000).astype(np.float32)) * np.float32(3.0))
    # amax values whose quotient by qmax lands next to an fp16 rounding midpoint
    h = rng.integers(0x0400, 0x7BFE, 1500).astype(np.uint16).view(np.float16).astype(np.float64)
    nxt = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    for m in (h + nxt) / 2:
        base = np.float32(m * qmax)
        amax += [base, np.nextafter(base, np.float32(0)), np.nextafter(base, np.float32(np.inf))]
    amax += [np.float32(1e7), np.float32(65504 * qmax), np.float32(1e-30), np.float32(0)]
    a = np.array(amax, np.float32)
    got = O.block_scale(a, qmax).view(np.uint16)
    want = [f16_bits_struct(min(f32_nearest(Fraction(float(v)) / qmax), 65504.0)) for v in a]
    assert got.tolist() == want


@pytest.mark.parametrize("bits", [8, 4])
def test_codes_exact_rational(bits):
    rng = np.random.default_rng(100 + bits)
    blocks = [rng.standard_normal(32).astype(np.float32) * s for s in (1, 8, 1e-3, 300)]
    # engineered near-ties: x = (k + 1/2) d and its fp32 neighbours
    for _ in range(40):
        x = rng.standard_normal(32).astype(np.float32)
        dbits, _ = ref_block(x, bits)
        d = np.float32(struct.unpack("<e", struct.pack("<H", dbits))[0])
        qmax = 127 if bits == 8 else 7
        k = rng.integers(0, qmax, 31)
        t = ((k + 0.5) * np.float64(d)).astype(np.float32)
        t = np.where(rng.random(31) < 0.5, t, np.nextafter(t, np.float32(0)))
        y = np.concatenate([[x[np.argmax(np.abs(x))]], t * np.sign(rng.standard_normal(31))]).astype(np.float32)
        blocks.append(y)
    for blk in blocks:
        assert oracle_block(blk, bits) == ref_block(blk, bits)


def _codec_cases():
    out = []
    for ln in (GOLD / "codec_cases.txt").read_text().splitlines():
        if not ln.strip() or ln.startswith("#") or ln.startswith("@"):
            continue
        head, xs, codes = ln.split("|")
        name, bits, dhex = head.split()
        out.append((name, int(bits), int(dhex, 16), [float(v) for v in xs.split()], [int(v) for v in codes.split()]))
    return out


@pytest.mark.parametrize("case", _codec_cases(), ids=lambda c: c[0])
def test_codec_golden_cases(case):
    _, bits, dbits, xs, codes = case
    gd, gc = oracle_block(xs, bits)
    assert gd == dbits
    assert gc[:len(codes)] == codes
    assert all(c == 0 for c in gc[len(xs):])


def _scale_rows():
    out = []
    for ln in (GOLD / "codec_cases.txt").read_text().splitlines():
        if ln.startswith("@scales"):
            head, amaxes, hexbytes = ln.split("|")
            out.append((int(head.split()[1]), [float(v) for v in amaxes.split()], [int(b, 16) for b in hexbytes.split()]))
    return out


@pytest.mark.parametrize("case", _scale_rows(), ids=lambda c: f"{c[0]}-bit")
def test_scale_plane_bytes_golden(case):
    """The stored scale plane of a row: each block's fp16 d, little-endian, in block order."""
    bits, amaxes, want = case
    row = np.zeros((1, 128), np.float32)
    for b, a in enumerate(amaxes):
        row[0, 32 * b] = a
    _, scale_bytes = O.encode_rows(row, bits)
    assert scale_bytes.shape == (1, 8)
    assert scale_bytes[0].tolist() == want


def test_nibble_packing_golden():
    q = np.zeros((1, 32), np.int16)
    q[0, 0], q[0, 1] = 7, -7
    packed = O.pack_codes(q, 4)
    assert packed.shape == (1, 16)
    assert packed[0, 0] == 0x1F and packed[0, 1] == 0x88
    q8 = np.array([[-1, 127, -127, 0] + [0] * 28], np.int16)
    assert O.pack_codes(q8, 8)[0, :4].tolist() == [0xFF, 0x7F, 0x81, 0x00]


@pytest.mark.parametrize("bits", [8, 4])
def test_codec_invariants(bits):
    qmax = 127 if bits == 8 else 7
    k, _, _ = I.workload_small(11, 512, 2, 128, 2, 1, n_outliers=8)
    x = k.reshape(-1, 128)
    q, d = O.quantize_rows(x, bits)
    dd = np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(q) <= qmax)
    normal = dd >= 2.0 ** -14
    assert np.all(np.abs(x - q * dd)[normal] <= dd[normal] / 2)
    packed = O.pack_codes(q, bits)
    if bits == 4:
        assert np.all((packed & 0xF) >= 1) and np.all((packed >> 4) >= 1)
        assert np.all((packed & 0xF) <= 15)
    else:
        assert not np.any(packed.view(np.int8) == -128)
    assert np.array_equal(O.unpack_codes(packed, bits, 128), q)
    z, dz = O.quantize_rows(np.zeros((3, 64), np.float32), bits)
    assert not z.any() and not dz.astype(np.float32).any()


def test_fp16_layout_roundtrip():
    x = I.normal((16, 64), 5)
    c, s = O.encode_rows(x, 16)
    assert s is None
    assert np.array_equal(O.dequant_rows(c, s, 16, 64), x.astype(np.float16).astype(np.float64))


def test_append_is_chunk_invariant():
    k, v, _ = I.workload_small(12, 700, 2, 64, 4, 1)
    for layout in range(6):
        one = O.OracleCache(layout, 1, 2, 64, 700)
        one.append(0, k, v)
        parts = O.OracleCache(layout, 1, 2, 64, 700)
        for a, b in ((0, 1), (1, 300), (300, 333), (333, 700)):
            parts.append(0, k[a:b], v[a:b])
        for name in ("Kc", "Ks", "Vc", "Vs"):
            assert np.array_equal(getattr(one, name), getattr(parts, name))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def brute_attention(q, keys, values, scale):
    """Pure-Python softmax attention of one query vector (math.fsum / math.exp)."""
    s = [scale * math.fsum(qi * ki for qi, ki in zip(q, kr)) for kr in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = math.fsum(w)
    return [math.fsum(wi * vr[j] for wi, vr in zip(w, values)) / tot for j in range(len(values[0]))]


@pytest.mark.parametrize("layout", [0, 2, 3])
def test_decode_matches_bruteforce(layout):
    k, v, q = I.workload_small(21, 5, 2, 32 * 2, 4, 1)
    c = O.OracleCache(layout, 1, 2, 64, 5)
    c.append(0, k, v)
    got = O.attend_decode([c], 0, q, 0.125)
    for h in range(4):
        kv = h // 2
        want = brute_attention(q[0, h].astype(float).tolist(), c.keys(0, kv).tolist(), c.values(0, kv).tolist(), 0.125)
        assert np.max(np.abs(got[0, h] - want)) <= 1e-12


def test_chunk_matches_bruteforce():
    k, v, q = I.workload_small(22, 7, 1, 32, 3, 3)
    c = O.OracleCache(2, 1, 1, 32, 7)
    c.append(0, k, v)
    got = O.attend_chunk(c, 0, q, 3, 0.3)
    kh, vh = c.keys(0, 0).tolist(), c.values(0, 0).tolist()
    for j in range(3):
        pos = 7 - 3 + j
        for h in range(3):
            want = brute_attention(q[j, h].astype(float).tolist(), kh[:pos + 1], vh[:pos + 1], 0.3)
            assert np.max(np.abs(got[j, h] - want)) <= 1e-12


def test_one_token_returns_its_value():
    k, v, q = I.workload_small(23, 1, 2, 64, 4, 1)
    c = O.OracleCache(2, 1, 2, 64, 1)
    c.append(0, k, v)
    out = O.attend_decode([c], 0, q, 0.125)
    for h in range(4):
        assert np.array_equal(out[0, h], c.values(0, h // 2)[0])


def test_equal_keys_or_zero_query_average_values():
    _, v, q = I.workload_small(24, 9, 1, 64, 2, 1)
    k = np.repeat(I.normal((1, 1, 64), 25), 9, axis=0)
    c = O.OracleCache(1, 1, 1, 64, 9)
    c.append(0, k, v)
    mean = c.values(0, 0).mean(axis=0)
    assert np.max(np.abs(O.attend_decode([c], 0, q, 0.125)[0, 0] - mean)) < 1e-13
    c2 = O.OracleCache(4, 1, 1, 64, 9)
    c2.append(0, I.normal((9, 1, 64), 26), v)
    out = O.attend_decode([c2], 0, np.zeros((1, 2, 64), np.float32), 0.125)
    assert np.max(np.abs(out[0, 1] - c2.values(0, 0).mean(axis=0))) < 1e-13


def test_two_token_closed_form():
    # keys along e0 with lengths 2 and -1, query 3 e0, scale 0.5: scores 3 and -1.5
    k = np.zeros((2, 1, 32), np.float32)
    k[0, 0, 0], k[1, 0, 0] = 2.0, -1.0
    v = np.zeros((2, 1, 32), np.float32)
    v[0, 0, :], v[1, 0, :] = 1.0, -2.0
    q = np.zeros((1, 1, 32), np.float32)
    q[0, 0, 0] = 3.0
    c = O.OracleCache(0, 1, 1, 32, 2)
    c.append(0, k, v)
    w1 = math.exp(-4.5)                      # e^(s1 - s0)
    want = (1.0 + w1 * -2.0) / (1.0 + w1)
    out = O.attend_decode([c], 0, q, 0.5)
    assert np.max(np.abs(out[0, 0] - want)) < 1e-14


def test_gqa_group_mapping():
    hkv, g = 4, 3
    k = I.normal((6, hkv, 64), 27)
    v = np.zeros((6, hkv, 64), np.float32)
    for h in range(hkv):
        v[:, h, :] = h + 1
    c = O.OracleCache(0, 1, hkv, 64, 6)
    c.append(0, k, v)
    out = O.attend_decode([c], 0, I.normal((1, hkv * g, 64), 28), 0.125)
    for h in range(hkv * g):
        assert np.allclose(out[0, h], h // g + 1, atol=1e-12)


def test_causal_mask_inclusive():
    # zero queries average the visible values; v_t = t makes that average pos / 2
    n_tok, n_new = 40, 9
    v = np.broadcast_to(np.arange(n_tok, dtype=np.float32)[:, None, None], (n_tok, 1, 32)).copy()
    c = O.OracleCache(0, 1, 1, 32, n_tok)
    c.append(0, I.normal((n_tok, 1, 32), 29), v)
    out = O.attend_chunk(c, 0, np.zeros((n_new, 2, 32), np.float32), n_new, 0.2)
    for j in range(n_new):
        assert np.allclose(out[j], (n_tok - n_new + j) / 2, atol=1e-12)


def test_fp16_layout_equals_unquantized_attention():
    k, v, q = I.workload_small(30, 50, 2, 64, 4, 1)
    k, v = k.astype(np.float16).astype(np.float32), v.astype(np.float16).astype(np.float32)
    c = O.OracleCache(0, 1, 2, 64, 50)
    c.append(0, k, v)
    out = O.attend_decode([c], 0, q, 0.125)
    for kv in range(2):
        assert np.array_equal(c.keys(0, kv), k[:, kv].astype(np.float64))
        assert np.array_equal(c.values(0, kv), v[:, kv].astype(np.float64))
        want = O.attention_exact(q[0, 2 * kv:2 * kv + 2], k[:, kv].astype(np.float64),
                                 v[:, kv].astype(np.float64), 0.125)
        assert np.array_equal(out[0, 2 * kv:2 * kv + 2], want)


@pytest.mark.parametrize("layout", [1, 2, 3, 4])
def test_quantized_attention_within_perturbation_bound(layout):
    k, v, q = I.workload_small(31, 200, 1, 64, 1, 1, n_outliers=4)
    c = O.OracleCache(layout, 1, 1, 64, 200)
    c.append(0, k, v)
    scale = 0.125
    kh, vh = c.keys(0, 0), c.values(0, 0)
    qq = q[0, 0].astype(np.float64)
    delta = scale * np.max(np.abs(kh - k[:, 0]) @ np.abs(qq))
    bound = (math.exp(2 * delta) - 1) * np.max(np.abs(v)) + np.max(np.abs(vh - v[:, 0]))
    exact = O.attention_exact(q[0, :1], k[:, 0].astype(np.float64), v[:, 0].astype(np.float64), scale)
    got = O.attend_decode([c], 0, q, scale)[0, 0]
    assert np.max(np.abs(got - exact[0])) <= bound


def test_reuse_invariant_turn_equals_recompute():
    # keep the cache and process only the new tokens == recompute the whole context
    n_ctx, n_new = 300, 37
    k, v, q = I.workload_small(32, n_ctx + n_new, 2, 64, 8, n_ctx + n_new, n_outliers=4)
    turn = O.OracleCache(2, 1, 2, 64, n_ctx + n_new)
    turn.append(0, k[:n_ctx], v[:n_ctx])
    turn.append(0, k[n_ctx:], v[n_ctx:])
    got = O.attend_chunk(turn, 0, q[n_ctx:], n_new, 0.125)
    full = O.OracleCache(2, 1, 2, 64, n_ctx + n_new)
    full.append(0, k, v)
    want = O.attend_chunk(full, 0, q, n_ctx + n_new, 0.125)[n_ctx:]
    assert np.max(np.abs(got - want)) <= 1e-12
    # and the last row of a turn is the decode of that position
    dec = O.attend_decode([turn], 0, q[-1:], 0.125)
    assert np.max(np.abs(got[-1] - dec[0])) <= 1e-12


def test_sampled_rows_match_full_chunk():
    k, v, q = I.workload_small(33, 150, 2, 64, 4, 60)
    c = O.OracleCache(2, 1, 2, 64, 150)
    c.append(0, k, v)
    full = O.attend_chunk(c, 0, q, 60, 0.125)
    rows = np.array([0, 17, 59])
    assert np.max(np.abs(O.attend_chunk(c, 0, q, 60, 0.125, rows=rows) - full[rows])) <= 1e-13


def test_keys_more_sensitive_than_values():
    # KVSplit page, "Assimetria entre key e value": K4V8 loses more than K8V4 at equal bits
    errs = {}
    n = 1024
    z = I.normal((n, 1, 128), 34)
    sc = np.exp(np.random.default_rng(35).standard_normal((1, 1, 128))).astype(np.float32)
    k, v, q = z * sc, I.normal((n, 1, 128), 36), I.normal((1, 8, 128), 37)
    exact = np.stack([O.attention_exact(q[0, h:h + 1], k[:, 0].astype(np.float64), v[:, 0].astype(np.float64),
                                        128 ** -0.5)[0] for h in range(8)])
    for name in ("K8V4", "K4V8"):
        c = O.OracleCache(O.LAYOUT_IDS[name], 1, 1, 128, n)
        c.append(0, k, v)
        errs[name] = np.sqrt(np.mean((O.attend_decode([c], 0, q, 128 ** -0.5)[0] - exact) ** 2))
    assert errs["K4V8"] > errs["K8V4"]


def test_decode_rejects_empty_cache():
    c = O.OracleCache(2, 1, 1, 64, 10)
    with pytest.raises(ValueError):
        O.attend_decode([c], 0, np.zeros((1, 1, 64), np.float32), 0.125)


# ---------------------------------------------------------------------------
# two-pass attention: split partials and their merge
# ---------------------------------------------------------------------------
def brute_partial(q, keys, values, scale):
    """Python-loop (o, m, l) of one query row over a key range, base-2 scores."""
    if not keys:
        return [0.0] * len(q), -math.inf, 0.0
    xs = [scale * math.log2(math.e) * math.fsum(a * b for a, b in zip(q, k)) for k in keys]
    m = max(xs)
    ws = [2.0 ** (x - m) for x in xs]
    o = [math.fsum(w * v[i] for w, v in zip(ws, values)) for i in range(len(q))]
    return o, m, math.fsum(ws)


def test_split_partial_matches_bruteforce():
    k, v, q = I.workload_small(31, 9, 1, 64, 2, 1)
    c = O.OracleCache(2, 1, 1, 64, 9)
    c.append(0, k, v)
    kh, vh = c.keys(0, 0), c.values(0, 0)
    for a, e in [(0, 9), (2, 5), (8, 9), (4, 4)]:
        o, m, l = O.split_partial(q[0].astype(np.float64), kh[a:e], vh[a:e], 0.2)
        for h in range(2):
            bo, bm, bl = brute_partial(q[0, h].astype(float).tolist(), kh[a:e].tolist(), vh[a:e].tolist(), 0.2)
            assert m[h] == bm if math.isinf(bm) else abs(m[h] - bm) <= 1e-12
            assert abs(l[h] - bl) <= 1e-12 and np.max(np.abs(o[h] - bo)) <= 1e-12


def test_split_partial_closed_forms():
    """One key: o = v, l = 1, m = its score.  Two keys: m = the larger score,
    l = 1 + 2^-|x1 - x2|, o = v_max + 2^-|x1 - x2| v_min.  No key: (0, -inf, 0)."""
    q = np.array([[1.0, -2.0, 0.5, 0.0]])
    k = np.array([[0.5, 0.25, -1.0, 3.0], [2.0, -1.0, 0.0, 1.0]])
    v = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.0, 1.0, 8.0]])
    x = 0.5 * O.LOG2E * (q @ k.T)[0]
    o, m, l = O.split_partial(q, k[:1], v[:1], 0.5)
    assert np.array_equal(o[0], v[0]) and l[0] == 1.0 and abs(m[0] - x[0]) <= 1e-15
    o, m, l = O.split_partial(q, k, v, 0.5)
    hi, lo = (1, 0) if x[1] > x[0] else (0, 1)
    r = 2.0 ** -(abs(x[1] - x[0]))
    assert m[0] == x[hi] and abs(l[0] - (1 + r)) <= 1e-15
    assert np.max(np.abs(o[0] - (v[hi] + r * v[lo]))) <= 1e-14
    o, m, l = O.split_partial(q, k[:0], v[:0], 0.5)
    assert m[0] == -np.inf and l[0] == 0 and not o.any()


@pytest.mark.parametrize("layout", [0, 2, 3])
def test_decode_partials_merge_to_attention(layout):
    """Merging the partials of any cut of the context into ranges gives the attention
    over the whole context (the identity the split kernels rely on); ranges past the
    end are empty and weigh nothing."""
    k, v, q = I.workload_small(32, 300, 2, 64, 8, 2)
    caches = []
    for b in range(2):
        c = O.OracleCache(layout, 1, 2, 64, 300)
        c.append(0, k[: 300 - 77 * b], v[: 300 - 77 * b])      # ragged lengths
        caches.append(c)
    want = O.attend_decode(caches, 0, q, 0.125)
    for n_splits, per in [(1, 512), (3, 128), (5, 64), (7, 64), (2, 1024)]:
        o, m, l = O.decode_partials(caches, 0, q, 0.125, n_splits, per)
        got = O.merge_partials(o, m, l)
        assert np.max(np.abs(got - want)) <= 1e-12, (n_splits, per)
        empty = np.arange(n_splits) * per >= 223
        assert np.all(np.isneginf(m[1][:, empty])) and not l[1][:, empty].any()


def test_chunk_partials_merge_to_chunk_attention():
    k, v, q = I.workload_small(33, 200, 2, 64, 6, 40)
    c = O.OracleCache(2, 1, 2, 64, 200)
    c.append(0, k, v)
    want = O.attend_chunk(c, 0, q, 40, 0.125)
    for n_splits, per in [(1, 256), (4, 64), (16, 64)]:
        o, m, l = O.chunk_partials(c, 0, q, 40, 0.125, n_splits, per)
        assert np.max(np.abs(O.merge_partials(o, m, l) - want)) <= 1e-12
    # token 0 (position 160) sees keys [0, 161): the 4th split of 64 ([192, 256)) is empty for it
    o, m, l = O.chunk_partials(c, 0, q, 40, 0.125, 4, 64, rows=[0, 39])
    assert np.all(np.isneginf(m[0, :, 3])) and np.all(np.isfinite(m[1, :, 3]))


def test_merge_is_invariant_to_the_reference_of_each_split():
    """(o, m, l) and (o 2^c, m - c, l 2^c) describe the same split: the merge agrees."""
    k, v, q = I.workload_small(34, 150, 1, 64, 2, 1)
    c = O.OracleCache(2, 1, 1, 64, 150)
    c.append(0, k, v)
    o, m, l = O.decode_partials([c], 0, q, 0.125, 3, 64)
    shift = np.array([0.0, 3.5, -7.0])
    got = O.merge_partials(o * np.exp2(shift)[..., None], m - shift, l * np.exp2(shift))
    assert np.max(np.abs(got - O.merge_partials(o, m, l))) <= 1e-12


# ---------------------------------------------------------------------------
# layer-specific layouts
# ---------------------------------------------------------------------------
def test_layered_footprint_is_the_mix_of_printed_rows():
    """Half the 22 layers in K8V8 and half in K4V4 take the mean of the two printed
    footprints at 8192 tokens, (93.50 + 49.50) / 2 = 71.50 MiB; FP16 with K8V4 gives
    (176.00 + 71.50) / 2 = 123.75 MiB."""
    mib = 2 ** 20
    mix = [1] * 11 + [4] * 11
    c = O.OracleLayeredCache(mix, 4, 64, 8192)
    assert c.footprint_bytes() == 71.50 * mib
    c2 = O.OracleLayeredCache([0, 2] * 11, 4, 64, 8192)
    assert c2.footprint_bytes() == 123.75 * mib


def test_layered_layers_equal_uniform_caches():
    """Layer l of a layered cache holds exactly the bytes a uniform cache of layouts[l]
    holds after the same appends, and attention over it is the same."""
    layouts = [0, 1, 2, 3, 4]
    lc = O.OracleLayeredCache(layouts, 2, 64, 300)
    for l, lay in enumerate(layouts):
        k, v, q = I.workload_small(60 + l, 50 + 40 * l, 2, 64, 4, 1, n_outliers=2)
        lc.append(l, k, v)
        uc = O.OracleCache(lay, 1, 2, 64, 300)
        uc.append(0, k, v)
        for name in ("Kc", "Ks", "Vc", "Vs"):
            assert np.array_equal(lc.plane(l, name), getattr(uc, name)[0])
        assert np.array_equal(O.attend_decode([lc], l, q, 0.125), O.attend_decode([uc], 0, q, 0.125))
    assert lc.len == [50, 90, 130, 170, 210]


# ---------------------------------------------------------------------------
# fp8 keys (MXFP8 blocks)
# ---------------------------------------------------------------------------
def test_e4m3_table_structure():
    """The code table of the OCP E4M3 definition: zero, subnormals k * 2^-9, normals
    (1 + m/8) 2^(e-7), largest 448, NaN only at S.1111.111, symmetric in the sign bit,
    and strictly increasing over the positive codes."""
    v = O.e4m3_values()
    assert v[0x00] == 0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x3F] == 1.875 and v[0x7E] == 448
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    assert np.all(np.diff(v[0x00:0x7F]) > 0)


def brute_e4m3(y: float) -> int:
    """Nearest finite E4M3 code by exhaustive search: ties to the even code, saturate, +0."""
    v = O.e4m3_values()
    pos = [(c, v[c]) for c in range(0x7F)]
    a = min(abs(y), 448.0)
    best = min(pos, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    c = best[0]
    return (c | 0x80) if (y < 0 and c != 0) else c


def test_e4m3_encode_matches_exhaustive_search():
    rng = np.random.default_rng(11)
    v = O.e4m3_values()
    mids = [(v[c] + v[c + 1]) / 2 for c in range(0x7E)]            # every tie
    ys = list(rng.standard_normal(300) * 40) + list(rng.uniform(-0.02, 0.02, 200)) + mids
    ys += [-m for m in mids] + [0.0, -0.0, 447.9, 448.0, 463.99, 464.0, 500.0, -511.0, 2.0 ** -10, 3 * 2.0 ** -11]
    got = O.e4m3_encode(np.array(ys))
    for y, c in zip(ys, got):
        assert int(c) == brute_e4m3(y), (y, int(c), brute_e4m3(y))


def test_mx_scale_brackets_the_block_maximum():
    """X = 2^e with 256 X <= amax < 512 X (amax / X has exponent 8, E4M3's largest);
    an all-zero block gets e = -127 and zero codes."""
    rng = np.random.default_rng(12)
    amax = np.abs(rng.standard_normal(1000) * np.exp(rng.uniform(-20, 20, 1000))).astype(np.float32)
    e = O.mx_scale_exponent(amax)
    for a, ee in zip(amax.astype(np.float64), e):
        assert Fraction(256) * Fraction(2) ** int(ee) <= Fraction(a) < Fraction(512) * Fraction(2) ** int(ee)
    codes, sc = O.mx_quantize_rows(np.zeros((1, 64), np.float32))
    assert not codes.any() and np.all(sc == 0)


def test_mxfp8_dequant_error_bound():
    """Outside saturation an element is within half an E4M3 spacing of its value: 2^-4 of
    its binade (2^-10 X in the subnormal range); the saturated block maximum is off by at
    most 64 X."""
    x = I.normal((50, 128), 13, 1) * np.float32(3.0)
    x[:, 5] *= 30
    codes, sc = O.mx_quantize_rows(x)
    xh = O.mx_dequant_rows(codes, sc)
    X = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    a = np.abs(x.astype(np.float64)) / X
    err = np.abs(x - xh) / X
    sat = a >= 448
    binade = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))))
    assert np.all(err[~sat] <= binade[~sat] * 2.0 ** -4 + 1e-12)
    assert np.all(err[sat] <= 64)


def test_kf8v4_footprint():
    """fp8 key rows are D code bytes + D/32 exponent bytes; 4-bit value rows as in K8V4."""
    for d in (64, 128):
        per = (d + d // 32) + (d // 2 + 2 * d // 32)
        assert O.layout_footprint_bytes(5, 2, 3, d, 300) == 2 * 3 * 512 * per


def test_fp8_queries_would_miss_the_attention_tolerance():
    """Why the fp8-key chunk path does not round each query to one MX fp8 value for its
    fp8 x fp8 products: that moves attention outputs far past the 5e-3 tolerance on the
    turn's input recipe, while the fp8 keys alone are the cache's content.  The kernel
    therefore splits each bf16 query into two E4M3 parts (next test)."""
    k, v, q = I.workload_small(5, 4000, 1, 128, 8, 64, bf16=True, n_outliers=4)
    oc = O.OracleCache(5, 1, 1, 128, 4000)
    oc.append(0, k, v)
    sm = 128 ** -0.5
    want = O.attend_chunk(oc, 0, q, 64, sm)
    qc, qs = O.mx_quantize_rows(q.reshape(-1, 128))
    q8 = O.mx_dequant_rows(qc, qs).reshape(q.shape).astype(np.float32)
    err = float(np.abs(O.attend_chunk(oc, 0, q8, 64, sm) - want).max())
    assert err > 10 * 5e-3, err


def test_bf16_two_part_e4m3_split():
    """The fp8-key chunk path's query split (OCP MX, two E4M3 parts per element): with
    t = floor(log2 amax) - 7 for the 32-element block, hi = E4M3(x / 2^t) and
    lo = E4M3((x - hi 2^t) / 2^(t-4)) give hi 2^t + lo 2^(t-4) = x exactly for every bf16 x
    of magnitude at least 2^(floor(log2 amax) - 13), and within 2^(t-14) below that.  Checked
    over every bf16 value of the binades from 2^-20 to 2^1 (the block's amax in [1, 2)) and
    for block maxima 2^-90 .. 2^90, with the E4M3 rounding of the oracle."""
    vals = O.e4m3_values()
    for big in (-90, -3, 0, 7, 90):
        # every bf16 bit pattern of [2^(big-20), 2^(big+1)) and its negation
        lo_bits = (127 + big - 20) << 7
        hi_bits = (127 + big + 1) << 7
        pat = np.arange(lo_bits, hi_bits, dtype=np.uint32) << 16
        x = pat.view(np.float32).astype(np.float64)
        x = np.concatenate([x, -x])
        amax_exp = big   # every block holds an element of [2^big, 2^(big+1))
        t = amax_exp - 7
        hi = vals[O.e4m3_encode(x * 2.0 ** -t)] * 2.0 ** t
        assert np.all(np.abs(x) * 2.0 ** -t < 448)
        lo = vals[O.e4m3_encode((x - hi) * 2.0 ** -(t - 4))] * 2.0 ** (t - 4)
        assert np.all(np.abs(x - hi) * 2.0 ** -(t - 4) <= 128)
        err = np.abs(hi + lo - x)
        big_enough = np.abs(x) >= 2.0 ** (amax_exp - 13)
        assert np.all(err[big_enough] == 0)
        assert np.all(err <= 2.0 ** (t - 14))

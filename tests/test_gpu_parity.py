"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Cache planes must match bit for bit; attention outputs within 5e-3 max abs error.
Sizes span several kernel tiles and ragged tails; the oracle finishes in seconds.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import TOL, assert_planes_equal, dev, gpu_cache, host_inputs, log, max_err, torch_mod

pytestmark = pytest.mark.gpu

LAYOUTS = ["FP16", "K8V8", "K8V4", "K4V8", "K4V4", "KF8V4"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# quantize-on-append
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_planes_bit_exact(layout, dtype, d):
    log(f"append {layout} {dtype} D={d}")
    hkv, n = 3, 611
    k, v, _ = I.workload_small(40 + d, n, hkv, d, hkv, 1, bf16=(dtype == "bf16"), n_outliers=4)
    k = np.where(np.arange(n)[:, None, None] % 97 == 5, 0.0, k).astype(np.float32)     # zero blocks
    k = np.where(np.arange(n)[:, None, None] % 89 == 7, k * 1e-30, k).astype(np.float32)  # scale underflow
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 2, hkv, d, n)
    with gpu_cache(layout, 2, hkv, d, n) as h:
        for a, b in ((0, 1), (1, 38), (38, 300), (300, n)):
            kvq.kv_append_quant(h, 1, dev(k[a:b], dtype), dev(v[a:b], dtype))
            oc.append(1, host_inputs(k[a:b], dtype), host_inputs(v[a:b], dtype))
        assert kvq.kv_cache_len(h, 1) == n and kvq.kv_cache_len(h, 0) == 0
        assert kvq.kv_footprint_bytes(h) == oc.footprint_bytes()
        assert_planes_equal(h, oc, 1)


def _golden_rows():
    rows = []
    from test_oracle import _codec_cases
    for _, bits, _, xs, _ in _codec_cases():
        r = np.zeros(64, np.float32)
        r[:len(xs)] = xs
        r[32:32 + len(xs)] = [-x for x in xs]
        rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("layout", ["K8V8", "K8V4", "K4V4"])
def test_append_codec_edge_cases(layout):
    rows = _golden_rows()
    k = rows[:, None, :]
    v = (rows[:, None, :] / np.float32(4.0)).astype(np.float32)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, 1, 64, len(rows))
    oc.append(0, k, v)
    with gpu_cache(layout, 1, 1, 64, len(rows)) as h:
        kvq.kv_append_quant(h, 0, dev(k, "f32"), dev(v, "f32"))
        assert_planes_equal(h, oc, 0)


@pytest.mark.parametrize("layout", ["K8V4", "K4V8"])
def test_append_infinite_elements(layout):
    """Blocks holding +-inf saturate their scale at 65504 and the infinities take the
    clamped code (the block's other elements their quotient by 65504), as in the format;
    the neighbouring blocks of the same row are unaffected."""
    rng = np.random.default_rng(31)
    rows = rng.standard_normal((6, 64)).astype(np.float32) * np.float32(3.0)
    rows[0, 5] = np.inf
    rows[1, 40] = -np.inf
    rows[2, 0], rows[2, 31] = np.inf, -np.inf
    rows[3, 33:40] = np.float32(7e4)           # a finite block whose scale saturates too
    rows[3, 34] = np.inf
    rows[4, :32] = 0.0
    rows[4, 7] = -np.inf
    k = rows[:, None, :]
    v = rows[::-1, None, :].copy()
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, 1, 64, len(rows))
    oc.append(0, k, v)
    with gpu_cache(layout, 1, 1, 64, len(rows)) as h:
        kvq.kv_append_quant(h, 0, dev(k, "f32"), dev(v, "f32"))
        assert_planes_equal(h, oc, 0)


def _mx_edge_rows():
    """Rows of two 32-element blocks, values y * 2^e on E4M3's grid and its midpoints:
    ties to even (normal and subnormal), the 448 saturation, -0, an all-zero block, and
    block maxima at the ends of the exponent range (scale clamp at -127, large scales)."""
    v = O.e4m3_values()
    mids = [(v[c] + v[c + 1]) / 2 for c in range(0x7E)]
    rows = []
    for e, top in ((-3, 256.0), (5, 500.0), (-20, 464.0), (40, 300.0), (-133, 256.0), (92, 511.0)):
        for start in range(0, len(mids), 31):
            blk = [top] + mids[start:start + 31]
            blk += [0.0] * (32 - len(blk))
            b = np.array(blk) * 2.0 ** e
            b[1::3] *= -1
            rows.append(np.concatenate([b, -b[::-1]]))
    z = np.zeros(64)
    z[33] = -0.0
    z[40] = 2.0 ** -100
    rows.append(z)
    return np.array(rows, dtype=np.float32)


def test_append_fp8_key_edge_cases():
    """fp8 key blocks of every rounding case are the oracle's bit for bit."""
    rows = _mx_edge_rows()
    assert np.all(np.isfinite(rows))
    k = rows[:, None, :]
    v = (rows[:, None, :] * np.float32(2.0 ** -60)).astype(np.float32)
    oc = O.OracleCache(O.LAYOUT_IDS["KF8V4"], 1, 1, 64, len(rows))
    oc.append(0, k, v)
    with gpu_cache("KF8V4", 1, 1, 64, len(rows)) as h:
        kvq.kv_append_quant(h, 0, dev(k, "f32"), dev(v, "f32"))
        assert_planes_equal(h, oc, 0)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
DECODE_CASES = [
    # layout, D, group, dtype, session lengths
    ("K8V4", 64, 8, "f32", [128]),
    ("K8V4", 128, 4, "bf16", [1, 129, 700, 2500]),
    ("K4V8", 128, 4, "bf16", [300, 1, 4097]),
    ("K8V8", 64, 8, "f32", [513, 2048]),
    ("K4V4", 64, 8, "f16", [77, 1000]),
    ("FP16", 128, 4, "bf16", [640, 3]),
    ("FP16", 64, 8, "f32", [1500]),
    ("K8V4", 128, 1, "bf16", [900, 200]),
    ("K8V4", 128, 2, "f32", [1025]),
    ("K4V8", 64, 3, "f32", [333, 700]),
    ("K8V8", 128, 5, "bf16", [1200]),
    ("K4V4", 128, 8, "bf16", [2000, 31]),
    ("K8V4", 64, 16, "f32", [600]),
    ("K4V8", 128, 16, "bf16", [257]),
    ("FP16", 64, 2, "f16", [64, 5000]),
    ("K8V4", 64, 2, "bf16", [700, 2049]),     # two value steps per chunk: short prefetch
    ("K4V4", 64, 1, "f32", [900]),
    ("KF8V4", 128, 8, "bf16", [1, 129, 3000]),
    ("KF8V4", 64, 4, "f32", [700, 2049]),
    ("KF8V4", 128, 3, "f16", [513]),
    ("KF8V4", 128, 16, "f32", [1000]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[2]}-{c[3]}-{len(c[4])}s")
def test_decode_matches_oracle(case):
    layout, d, g, dtype, lens = case
    log(f"decode {case}")
    hkv = 2
    hq = hkv * g
    lid = O.LAYOUT_IDS[layout]
    sessions, ocs = [], []
    q = I.normal((len(lens), hq, d), 500 + d + g, 9)
    if dtype == "bf16":
        q = I.bf16_round(q)
    try:
        for i, n in enumerate(lens):
            k, v, _ = I.workload_small(600 + 7 * i + g, n, hkv, d, hq, 1, bf16=(dtype == "bf16"), n_outliers=4)
            h = kvq.kv_cache_create(layout, 2, hkv, d, n + 50)
            sessions.append(h)
            kvq.kv_append_quant(h, 1, dev(k, dtype), dev(v, dtype))
            oc = O.OracleCache(lid, 2, hkv, d, n + 50)
            oc.append(1, host_inputs(k, dtype), host_inputs(v, dtype))
            ocs.append(oc)
        scale = d ** -0.5
        out = kvq.kv_attend_decode(sessions, 1, dev(q, dtype), scale)
        want = O.attend_decode(ocs, 1, host_inputs(q, dtype), scale)
        err = max_err(out, want)
        log(f"  max err {err:.3e}")
        assert err <= TOL
    finally:
        torch_mod().cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)


def test_decode_more_sessions_than_one_launch():
    log("decode 70 sessions")
    d, hkv, g, n_s = 64, 1, 4, 70
    sessions, ocs = [], []
    q = I.normal((n_s, hkv * g, d), 77)
    try:
        for i in range(n_s):
            n = 1 + (i * 37) % 300
            k, v, _ = I.workload_small(700 + i, n, hkv, d, hkv * g, 1)
            h = kvq.kv_cache_create("K8V4", 1, hkv, d, 400)
            kvq.kv_append_quant(h, 0, dev(k, "f32"), dev(v, "f32"))
            oc = O.OracleCache(2, 1, hkv, d, 400)
            oc.append(0, k, v)
            sessions.append(h)
            ocs.append(oc)
        out = kvq.kv_attend_decode(sessions, 0, dev(q, "f32"), 0.125)
        assert max_err(out, O.attend_decode(ocs, 0, q, 0.125)) <= TOL
    finally:
        torch_mod().cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)


@pytest.mark.parametrize("layout", ["K8V4", "K4V8", "K8V8", "FP16", "KF8V4"])
@pytest.mark.parametrize("vscale", [1e-2, 1e-4])
@pytest.mark.parametrize("shape", ["peaked", "flat"])
def test_decode_small_values(layout, vscale, shape):
    """Values scaled by 1e-2 and 1e-4 (small value scales: p times the scale then falls among
    fp16's subnormals for many tokens), under an attention peaked on a few of 32,768 tokens
    or spread over all of them, judged by the error relative to the output's magnitude."""
    log(f"decode small values, {shape} {layout} x{vscale}")
    d, hkv, g, n = 128, 2, 4, 32768
    k, v, _ = I.workload_small(4700, n, hkv, d, hkv * g, 1, bf16=True)
    v = I.bf16_round(v * np.float32(vscale) + np.float32(vscale))   # a nonzero mean: a flat
    rng = np.random.default_rng(47)                                   # attention's output
    q = np.empty((1, hkv * g, d), np.float32)
    for h in range(hkv * g):
        if shape == "peaked":   # each head aligned with three tokens' keys
            q[0, h] = k[rng.choice(n, 3, replace=False), h // g].sum(0) * np.float32(1.2)
        else:                   # logits within +-0.1 of each other
            q[0, h] = rng.standard_normal(d).astype(np.float32) * np.float32(0.01)
    q = I.bf16_round(q)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    oc.append(0, k, v)
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, "bf16"), dev(v, "bf16"))
        out = kvq.kv_attend_decode([h], 0, dev(q, "bf16"), d ** -0.5)
        want = O.attend_decode([oc], 0, q, d ** -0.5)
        got = out.detach().cpu().numpy().astype(np.float64)
        rel = float(np.max(np.abs(got - want)) / np.max(np.abs(want)))
        log(f"  max err relative to max |out|: {rel:.3e}")
        assert rel <= TOL


def test_decode_same_cache_twice_in_one_call():
    """A cache listed twice in one call (two queries over the same context) next to another
    cache: each row must match the oracle, and a second call must too (the split merge's
    per-head state is back at rest)."""
    log("decode with a repeated cache")
    d, hkv, g = 128, 2, 4
    lens = [3000, 1500]
    hs, ocs = [], []
    try:
        for i, n in enumerate(lens):
            k, v, _ = I.workload_small(820 + i, n, hkv, d, hkv * g, 1, bf16=True, n_outliers=4)
            h = kvq.kv_cache_create("K8V4", 1, hkv, d, n)
            kvq.kv_append_quant(h, 0, dev(k, "bf16"), dev(v, "bf16"))
            oc = O.OracleCache(O.LAYOUT_IDS["K8V4"], 1, hkv, d, n)
            oc.append(0, host_inputs(k, "bf16"), host_inputs(v, "bf16"))
            hs.append(h)
            ocs.append(oc)
        order = [0, 1, 0]
        for rep in range(2):
            q = I.bf16_round(I.normal((len(order), hkv * g, d), 830 + rep, 9))
            out = kvq.kv_attend_decode([hs[i] for i in order], 0, dev(q, "bf16"), d ** -0.5)
            want = O.attend_decode([ocs[i] for i in order], 0, host_inputs(q, "bf16"), d ** -0.5)
            err = max_err(out, want)
            log(f"  call {rep}: max err {err:.3e}")
            assert err <= TOL
    finally:
        torch_mod().cuda.synchronize()
        for h in hs:
            kvq.kv_cache_destroy(h)


def test_decode_128_tokens_exact_workload():
    log("decode 128 tokens")
    c = I.decode_128_tokens()
    oc = O.OracleCache(2, 1, 4, 64, 128)
    oc.append(0, c["k"], c["v"])
    with gpu_cache("K8V4", 1, 4, 64, 128) as h:
        kvq.kv_append_quant(h, 0, dev(c["k"], "f32"), dev(c["v"], "f32"))
        assert_planes_equal(h, oc, 0)
        out = kvq.kv_attend_decode([h], 0, dev(c["q"], "f32"), 64 ** -0.5)
        err = max_err(out, O.attend_decode([oc], 0, c["q"], 64 ** -0.5))
        log(f"  decode 128 tokens max err {err:.3e}")
        assert tuple(out.shape) == (1, 32, 64) and err <= TOL


# ---------------------------------------------------------------------------
# chunk prefill
# ---------------------------------------------------------------------------
CHUNK_CASES = [
    # layout, D, group, dtype, cached before the turn, new tokens
    ("K8V4", 128, 8, "bf16", 0, 1),
    ("K8V4", 128, 8, "bf16", 700, 37),
    ("K8V4", 128, 8, "bf16", 3000, 200),
    ("K4V8", 128, 5, "bf16", 1500, 64),
    ("K8V8", 64, 4, "f32", 100, 300),
    ("K4V4", 64, 1, "f16", 2100, 129),
    ("FP16", 128, 4, "bf16", 50, 50),
    ("FP16", 64, 8, "f32", 4000, 16),
    ("K8V4", 64, 2, "f32", 0, 700),
    ("K4V8", 128, 16, "bf16", 333, 3),
    ("KF8V4", 128, 8, "bf16", 3000, 200),
    ("KF8V4", 64, 2, "f32", 0, 700),
    ("KF8V4", 128, 5, "f16", 1500, 64),
    # bf16 queries on fp8 keys take the MX fp8 products, at both head_dims and every group size
    ("KF8V4", 64, 8, "bf16", 1200, 150),
    ("KF8V4", 64, 16, "bf16", 0, 333),
    ("KF8V4", 64, 1, "bf16", 2500, 9),
    ("KF8V4", 128, 16, "bf16", 257, 45),
    ("KF8V4", 128, 1, "bf16", 90, 70),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[2]}-{c[3]}-{c[4]}+{c[5]}")
def test_chunk_matches_oracle(case):
    layout, d, g, dtype, n_ctx, n_new = case
    log(f"chunk {case}")
    hkv = 2
    hq = hkv * g
    n = n_ctx + n_new
    k, v, q = I.workload_small(900 + g + d, n, hkv, d, hq, n_new, bf16=(dtype == "bf16"), n_outliers=4)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    with gpu_cache(layout, 1, hkv, d, n) as h:
        if n_ctx:
            kvq.kv_append_quant(h, 0, dev(k[:n_ctx], dtype), dev(v[:n_ctx], dtype))
            oc.append(0, host_inputs(k[:n_ctx], dtype), host_inputs(v[:n_ctx], dtype))
        kvq.kv_append_quant(h, 0, dev(k[n_ctx:], dtype), dev(v[n_ctx:], dtype))
        oc.append(0, host_inputs(k[n_ctx:], dtype), host_inputs(v[n_ctx:], dtype))
        scale = d ** -0.5
        out = kvq.kv_attend_chunk(h, 0, dev(q, dtype), n_new, scale)
        want = O.attend_chunk(oc, 0, host_inputs(q, dtype), n_new, scale)
        err = max_err(out, want)
        log(f"  max err {err:.3e}")
        assert err <= TOL


def _outlier_queries(shape, seed, factor, top=None):
    """N(0, 1) queries whose four channels per query head are `factor` times larger (the
    same channels in every row), optionally one channel raised to +-`top`: the shape of the
    activation outliers of trained models, and a magnitude past fp16's range."""
    q = I.normal(shape, seed, 9)
    rng = np.random.default_rng(seed)
    d = shape[-1]
    for h in range(shape[1]):
        ch = rng.choice(d, 4, replace=False)
        q[:, h, ch] *= np.float32(factor)
        if top is not None:
            q[:, h, ch[0]] = np.float32(top) * np.sign(q[:, h, ch[0]] + 1e-30)
    return q.astype(np.float32)


QUERY_OUTLIER_LAYOUTS = ["K8V4", "K4V8", "K8V8", "K4V4", "FP16", "KF8V4"]


@pytest.mark.parametrize("layout", QUERY_OUTLIER_LAYOUTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_decode_query_outlier_channels(layout, dtype):
    """Queries with 4 channels per head 64 times the rest: the query's per-head scale then
    spans the outliers, and the other channels must keep their precision."""
    log(f"decode outlier queries {layout} {dtype}")
    d, hkv, g = 128, 2, 4
    lens = [900, 2100]
    q = _outlier_queries((len(lens), hkv * g, d), 41, 64.0) * np.float32(0.25)
    if dtype == "bf16":
        q = I.bf16_round(q)
    hs, ocs = [], []
    try:
        for i, n in enumerate(lens):
            k, v, _ = I.workload_small(4400 + i, n, hkv, d, hkv * g, 1, bf16=(dtype == "bf16"))
            h = kvq.kv_cache_create(layout, 1, hkv, d, n)
            kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
            oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
            oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
            hs.append(h)
            ocs.append(oc)
        out = kvq.kv_attend_decode(hs, 0, dev(q, dtype), d ** -0.5)
        err = max_err(out, O.attend_decode(ocs, 0, host_inputs(q, dtype), d ** -0.5))
        log(f"  max err {err:.3e}")
        assert err <= TOL
    finally:
        torch_mod().cuda.synchronize()
        for h in hs:
            kvq.kv_cache_destroy(h)


@pytest.mark.parametrize("layout", ["K8V4", "FP16", "KF8V4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_queries_beyond_fp16_range(layout, dtype):
    """A query channel at +-2^17 (past fp16's 65504) with the others ~1e-2: decode and chunk
    must scale the query into range rather than overflow it."""
    log(f"queries beyond fp16 {layout} {dtype}")
    d, hkv, g, n_ctx, n_new = 128, 2, 4, 500, 40
    n = n_ctx + n_new
    k, v, _ = I.workload_small(4500, n, hkv, d, hkv * g, 1, bf16=(dtype == "bf16"))
    k = (k * np.float32(1e-4)).astype(np.float32)     # keep the logits moderate
    if dtype == "bf16":
        k = I.bf16_round(k)
    q = _outlier_queries((n_new, hkv * g, d), 45, 0.01, top=2.0 ** 17) * np.float32(0.01)
    q[np.abs(q) > 1] *= np.float32(100.0)            # the top channel back at +-2^17
    if dtype == "bf16":
        q = I.bf16_round(q)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
        qd = dev(q, dtype)
        out_c = kvq.kv_attend_chunk(h, 0, qd, n_new, d ** -0.5)
        err_c = max_err(out_c, O.attend_chunk(oc, 0, host_inputs(q, dtype), n_new, d ** -0.5))
        out_d = kvq.kv_attend_decode([h], 0, dev(q[-1:], dtype), d ** -0.5)
        err_d = max_err(out_d, O.attend_decode([oc], 0, host_inputs(q[-1:], dtype), d ** -0.5))
        log(f"  chunk max err {err_c:.3e}, decode max err {err_d:.3e}")
        assert err_c <= TOL and err_d <= TOL


@pytest.mark.parametrize("layout", ["KF8V4", "K8V4", "FP16"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [128, 64])
def test_queries_with_zero_and_tiny_blocks(layout, dtype, d):
    """Query 32-element blocks that are all zero or sit near the bottom of the format's range
    (a zero query row too): every per-block query scale of the chunk path must stay a usable
    power of two, and decode's per-head scale too."""
    log(f"zero and tiny query blocks {layout} D{d} {dtype}")
    hkv, g, n_ctx, n_new = 2, 4, 300, 70
    n = n_ctx + n_new
    k, v, _ = I.workload_small(4600, n, hkv, d, hkv * g, 1, bf16=(dtype == "bf16"))
    if dtype == "bf16":
        k = I.bf16_round(k)
    q = I.normal((n_new, hkv * g, d), 47, 9)
    tiny = 2.0 ** -120 if dtype == "bf16" else 2.0 ** -14   # bf16: below 2^-115; fp16: its smallest normal
    q[:, 0, 32:64] = 0.0                       # one zero block per row
    q[:, 1, d // 2:d // 2 + 32] *= np.float32(tiny)   # a block at the bottom of the range
    q[:, 2, :] = 0.0                           # a zero query head
    q[:, 3, d - 32:] *= np.float32(tiny)       # a tiny block beside ordinary ones
    q[::7, 4, :] *= np.float32(tiny)           # every seventh row of a head tiny throughout
    q = q.astype(np.float32)
    if dtype == "bf16":
        q = I.bf16_round(q)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
        out_c = kvq.kv_attend_chunk(h, 0, dev(q, dtype), n_new, d ** -0.5)
        out_d = kvq.kv_attend_decode([h], 0, dev(q[-1:], dtype), d ** -0.5)
        err_c = max_err(out_c, O.attend_chunk(oc, 0, host_inputs(q, dtype), n_new, d ** -0.5))
        err_d = max_err(out_d, O.attend_decode([oc], 0, host_inputs(q[-1:], dtype), d ** -0.5))
        log(f"  chunk max err {err_c:.3e}, decode max err {err_d:.3e}")
        assert err_c <= TOL and err_d <= TOL


@pytest.mark.parametrize("layout", ["K8V4", "K4V8", "FP16", "KF8V4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_query_outlier_channels(layout, dtype):
    log(f"chunk outlier queries {layout} {dtype}")
    d, hkv, g, n_ctx, n_new = 128, 2, 4, 1500, 100
    n = n_ctx + n_new
    k, v, _ = I.workload_small(4600, n, hkv, d, hkv * g, 1, bf16=(dtype == "bf16"))
    q = _outlier_queries((n_new, hkv * g, d), 47, 64.0) * np.float32(0.25)
    if dtype == "bf16":
        q = I.bf16_round(q)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
        out = kvq.kv_attend_chunk(h, 0, dev(q, dtype), n_new, d ** -0.5)
        err = max_err(out, O.attend_chunk(oc, 0, host_inputs(q, dtype), n_new, d ** -0.5))
        log(f"  max err {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("layout,d,dtype", [("K8V4", 128, "bf16"), ("K4V4", 128, "f16"), ("K8V8", 64, "bf16"),
                                            ("K4V8", 128, "f32")])
def test_chunk_keys_spanning_five_decades(layout, d, dtype):
    """Key rows scaled by 10^u, u uniform in [-4, 1) per (token, KV head): the fp16 scales of
    the key blocks take exponents over most of fp16's range, and the low part of every block
    (fp6 at head_dim 128 with 16-bit queries, fp8 otherwise) is scaled from its own."""
    log(f"chunk wide key range {layout} D{d} {dtype}")
    hkv, g, n_ctx, n_new = 2, 4, 1200, 130
    hq = hkv * g
    n = n_ctx + n_new
    k, v, q = I.workload_small(960 + d, n, hkv, d, hq, n_new, n_outliers=4)
    k = k * I.log10_uniform((n, hkv, 1), -4.0, 1.0, 961 + d)
    if dtype == "bf16":
        k, v, q = I.bf16_round(k), I.bf16_round(v), I.bf16_round(q)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
        oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
        assert_planes_equal(h, oc, 0)
        scale = d ** -0.5
        out = kvq.kv_attend_chunk(h, 0, dev(q, dtype), n_new, scale)
        want = O.attend_chunk(oc, 0, host_inputs(q, dtype), n_new, scale)
        err = max_err(out, want)
        log(f"  max err {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("layout,d,dtype", [("K8V4", 128, "bf16"), ("K4V8", 64, "f32"), ("KF8V4", 128, "f16"),
                                            ("KF8V4", 64, "f16"), ("KF8V4", 128, "bf16"), ("KF8V4", 64, "bf16")])
def test_chunk_running_max_moves_along_the_keys(layout, d, dtype):
    """Key rows scaled by 1 + 3 t / 64 at position t: the scores grow along the keys, so each
    32-key half of a row brings a larger maximum than the last. Depending on the row the half's
    weights then fit the running max's headroom (no tile max), exceed the headroom test without
    moving the max, or move it (rescale, weights formed again): every branch of the chunk
    kernel's online softmax runs, on rows that are checked against the oracle."""
    log(f"chunk growing keys {layout} D{d} {dtype}")
    hkv, g, n_ctx, n_new = 2, 4, 1400, 100
    hq, n = hkv * g, n_ctx + n_new
    k, v, q = I.workload_small(970 + d, n, hkv, d, hq, n_new, n_outliers=0)
    k = k * (1.0 + 3.0 * np.arange(n, dtype=np.float32) / 64.0)[:, None, None]
    if dtype == "bf16":
        k, v, q = I.bf16_round(k), I.bf16_round(v), I.bf16_round(q)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
        oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
        scale = d ** -0.5
        out = kvq.kv_attend_chunk(h, 0, dev(q, dtype), n_new, scale)
        want = O.attend_chunk(oc, 0, host_inputs(q, dtype), n_new, scale)
        err = max_err(out, want)
        log(f"  max err {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("layout,d,dtype", [("K8V4", 128, "bf16"), ("K8V8", 64, "f32")])
def test_chunk_score_jump_past_fp32_range(layout, d, dtype):
    """One key row 2^9 times larger than the rest, past the first tiles: for the rows it
    attends to, its score exceeds the running max by hundreds of log2 units, so the weights
    formed against the old max overflow to infinity before the tile max is taken and the max
    moves.  (Several such keys competing at scores in the hundreds would test the precision of
    the keys' low part instead: its error grows with the key's magnitude.)"""
    log(f"chunk score jump {layout} D{d} {dtype}")
    hkv, g, n_ctx, n_new = 2, 4, 900, 60
    hq, n = hkv * g, n_ctx + n_new
    k, v, q = I.workload_small(980 + d, n, hkv, d, hq, n_new, n_outliers=0)
    k[700] *= np.float32(512.0)
    if dtype == "bf16":
        k, v, q = I.bf16_round(k), I.bf16_round(v), I.bf16_round(q)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
        oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
        scale = d ** -0.5
        out = kvq.kv_attend_chunk(h, 0, dev(q, dtype), n_new, scale)
        want = O.attend_chunk(oc, 0, host_inputs(q, dtype), n_new, scale)
        err = max_err(out, want)
        log(f"  max err {err:.3e}")
        assert np.all(np.isfinite(out.cpu().numpy())) and err <= TOL


def _causal_rms_with_fp16_keys(oc, q, n_new, scale, want):
    """RMS distance from `want` of causal attention over the same cache with every key
    rounded to fp16 (what the chunk path would return without the keys' low part)."""
    hkv, n = oc.Hkv, oc.len[0]
    g = q.shape[1] // hkv
    out = np.zeros_like(want)
    for h in range(hkv):
        kh = oc.keys(0, h).astype(np.float16).astype(np.float64)
        vh = oc.values(0, h)
        for j in range(n_new):
            pos = n - n_new + j
            out[j, h * g:(h + 1) * g] = O.attention_exact(q[j, h * g:(h + 1) * g], kh[:pos + 1], vh[:pos + 1], scale)
    return float(np.sqrt(np.mean((out - want) ** 2)))


@pytest.mark.parametrize("layout,d,dtype", [("K8V4", 128, "bf16"), ("K4V4", 128, "f16"), ("K8V8", 64, "bf16"),
                                            ("K8V4", 128, "f32"), ("K4V8", 64, "f32")])
def test_chunk_key_low_part_is_applied(layout, d, dtype):
    """The chunk path carries a quantized key as its fp16 rounding plus a low part on the
    block-scaled MFMA (fp6 or fp8).  Without the low part the outputs would sit at the error of
    fp16-rounded keys, which stays inside the 5e-3 gate; this checks that the GPU's RMS error is
    well below that (fp16 weights and values alone give about 0.3 of it on these inputs)."""
    log(f"chunk key low part {layout} D{d} {dtype}")
    hkv, g, n_ctx, n_new = 2, 8, 3000, 200
    hq, n = hkv * g, n_ctx + n_new
    k, v, q = I.workload_small(4000 + g + d, n, hkv, d, hq, n_new, bf16=(dtype == "bf16"), n_outliers=4 * d // 64)
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
    with gpu_cache(layout, 1, hkv, d, n) as h:
        kvq.kv_append_quant(h, 0, dev(k, dtype), dev(v, dtype))
        oc.append(0, host_inputs(k, dtype), host_inputs(v, dtype))
        scale = d ** -0.5
        qh = host_inputs(q, dtype)
        out = kvq.kv_attend_chunk(h, 0, dev(q, dtype), n_new, scale).cpu().numpy().astype(np.float64)
        want = O.attend_chunk(oc, 0, qh, n_new, scale)
        rms = float(np.sqrt(np.mean((out - want) ** 2)))
        rms16 = _causal_rms_with_fp16_keys(oc, qh, n_new, scale, want)
        log(f"  rms err {rms:.3e}, with fp16-rounded keys {rms16:.3e} (ratio {rms / rms16:.2f}), "
            f"max err {np.abs(out - want).max():.3e}")
        assert np.abs(out - want).max() <= TOL
        assert rms <= 0.6 * rms16


# ---------------------------------------------------------------------------
# determinism and device-side error paths
# ---------------------------------------------------------------------------
def test_outputs_are_run_to_run_deterministic():
    torch = torch_mod()
    k, v, q = I.workload_small(950, 3000, 2, 128, 8, 100, bf16=True, n_outliers=4)
    with gpu_cache("K8V4", 1, 2, 128, 3000) as h:
        kvq.kv_append_quant(h, 0, dev(k, "bf16"), dev(v, "bf16"))
        qd = dev(q[-1:], "bf16")
        a = kvq.kv_attend_decode([h], 0, qd, 0.088)
        b = kvq.kv_attend_decode([h], 0, qd, 0.088)
        assert torch.equal(a, b)
        qc = dev(q, "bf16")
        c1 = kvq.kv_attend_chunk(h, 0, qc, 100, 0.088)
        c2 = kvq.kv_attend_chunk(h, 0, qc, 100, 0.088)
        assert torch.equal(c1, c2)


def test_device_error_paths():
    torch = torch_mod()
    with gpu_cache("K8V4", 1, 2, 64, 100) as h, gpu_cache("K4V8", 1, 2, 64, 100) as other:
        q = torch.zeros((1, 4, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_attend_decode([h], 0, q, 0.1)
        assert e.value.code == kvq.KV_EEMPTY
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_attend_chunk(h, 0, q, 1, 0.1)
        assert e.value.code == kvq.KV_EEMPTY
        x = torch.zeros((101, 2, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_append_quant(h, 0, x, x)
        assert e.value.code == kvq.KV_ECAPACITY and kvq.kv_cache_len(h, 0) == 0
        kvq.kv_append_quant(h, 0, x[:10], x[:10])
        kvq.kv_append_quant(other, 0, x[:10], x[:10])
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_attend_decode([h, other], 0, torch.zeros((2, 4, 64), device="cuda"), 0.1)
        assert e.value.code == kvq.KV_EINVAL
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_attend_chunk(h, 0, torch.zeros((11, 4, 64), device="cuda"), 11, 0.1)
        assert e.value.code == kvq.KV_EINVAL
        # n_q_heads not a multiple of n_kv_heads: the binding refuses it before the call, and the
        # library does too when called directly
        with pytest.raises(ValueError):
            kvq.kv_attend_decode([h], 0, torch.zeros((1, 3, 64), device="cuda"), 0.1)
        q3 = torch.zeros((1, 3, 64), device="cuda")
        o3 = torch.empty_like(q3)
        arr = (ctypes.c_void_p * 1)(h)
        rc = kvq.lib().kv_attend_decode(arr, 1, 0, q3.data_ptr(), kvq.KV_F32, 3, 0.1, o3.data_ptr(), None, 0,
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == kvq.KV_EINVAL and "n_q_heads" in kvq.kv_last_error()
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_append_quant(h, 1, x[:1], x[:1])
        assert e.value.code == kvq.KV_EINVAL
        raw = torch.zeros(4 * 64 + 1, dtype=torch.float32, device="cuda")[1:].view(1, 4, 64)
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_attend_decode([h], 0, raw, 0.1)
        assert e.value.code == kvq.KV_EINVAL and "aligned" in str(e.value)
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_cache_truncate(h, 0, 11)
        assert e.value.code == kvq.KV_EINVAL
        kvq.kv_cache_truncate(h, 0, 4)
        assert kvq.kv_cache_len(h, 0) == 4
        kvq.kv_cache_reset(h)
        assert kvq.kv_cache_len(h, 0) == 0
        # sizes that would overflow the host's range arithmetic are refused, not wrapped
        big = (1 << 63) - 1
        assert kvq.lib().kv_append_quant(h, 0, x.data_ptr(), x.data_ptr(), kvq.KV_F32, big, None) == kvq.KV_ECAPACITY
        assert kvq.kv_cache_len(h, 0) == 0
        buf = torch.empty(64, dtype=torch.uint8, device="cuda")
        assert kvq.lib().kv_cache_copy_plane(h, 0, 0, kvq.KV_PLANE_KC, 1 << 62, 1 << 62, buf.data_ptr(),
                                             None) == kvq.KV_EINVAL

"""GPU parity of the two passes on their own: the split partial kernels (decode and
chunk) and the log-sum-exp merge, through kv_attend_*_partial and kv_merge_partials.

A split's (o, m, l) is unique only up to the common rescale (o, l) * 2^c, m - c (the
chunk kernel moves its running max lazily), so the comparison is on what is unique:
the split's normalized output o / l (tolerance 5e-3, as every attention output) and
its log-sum-exp m + log2(l) in base-2 units (tolerance LSE_TOL).  A split that sees
no key must come back exactly as m = -inf, l = 0, o = 0.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import TOL, dev, host_inputs, log, max_err, torch_mod

pytestmark = pytest.mark.gpu

# An error e in a split's log-sum-exp scales its weight in the merge by 2^e; at
# e = 5e-3 that is 0.35 %, which moves a merged output of magnitude <= 4 by < 5e-3.
LSE_TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.lib()
    yield
    torch.cuda.synchronize()


def compare_partials(p_gpu, o, m, l, what: str):
    """GPU partials [..., n_splits, D + 2] against oracle (o, m, l)."""
    p = p_gpu.detach().cpu().numpy().astype(np.float64)
    d = o.shape[-1]
    go, gm, gl = p[..., :d], p[..., d], p[..., d + 1]
    empty = np.isneginf(m)
    assert np.array_equal(np.isneginf(gm), empty), f"{what}: empty splits differ"
    assert np.all(gl[empty] == 0) and np.all(go[empty] == 0), f"{what}: empty split not zero"
    full = ~empty
    assert np.all(np.isfinite(p[full])), f"{what}: non-finite partials"
    err_o = float(np.max(np.abs(go[full] / gl[full][:, None] - o[full] / l[full][:, None]))) if full.any() else 0.0
    err_lse = float(np.max(np.abs((gm[full] + np.log2(gl[full])) - (m[full] + np.log2(l[full]))))) if full.any() else 0.0
    log(f"  {what}: split output err {err_o:.3e}, log-sum-exp err {err_lse:.3e}, "
        f"{int(empty.sum())} empty of {empty.size}")
    assert err_o <= TOL and err_lse <= LSE_TOL


DECODE_CASES = [
    # layout, head_dim, group, lengths, [(n_splits, tokens_per_split)]
    ("K8V4", 128, 4, [1, 700, 1500, 2053], [(1, 2560), (3, 1024), (6, 512)]),
    ("K4V8", 128, 4, [1300, 64], [(2, 1024), (4, 512)]),
    ("FP16", 64, 8, [513, 1024], [(2, 512), (5, 512)]),
    ("K4V4", 64, 1, [900], [(1, 1024), (2, 512)]),
    ("KF8V4", 128, 8, [2000, 33], [(1, 2048), (4, 512)]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"{c[0]}-D{c[1]}-G{c[2]}" for c in DECODE_CASES])
def test_decode_partials_and_merge(case):
    layout, d, g, lens, plans = case
    log(f"decode partials {layout} D={d} G={g} lens={lens}")
    hkv = 2
    hq = hkv * g
    lid = O.LAYOUT_IDS[layout]
    torch = torch_mod()
    q = I.bf16_round(I.normal((len(lens), hq, d), 900 + d + g, 9))
    sessions, ocs = [], []
    try:
        for i, n in enumerate(lens):
            k, v, _ = I.workload_small(910 + 3 * i + g, n, hkv, d, hq, 1, bf16=True, n_outliers=4)
            h = kvq.kv_cache_create(layout, 1, hkv, d, n)
            sessions.append(h)
            kvq.kv_append_quant(h, 0, dev(k, "bf16"), dev(v, "bf16"))
            oc = O.OracleCache(lid, 1, hkv, d, n)
            oc.append(0, k, v)
            ocs.append(oc)
        scale = d ** -0.5
        qd = dev(q, "bf16")
        want = O.attend_decode(ocs, 0, q, scale)
        for n_splits, per in plans:
            p = kvq.kv_attend_decode_partial(sessions, 0, qd, scale, n_splits, per)
            o, m, l = O.decode_partials(ocs, 0, q, scale, n_splits, per)
            compare_partials(p, o, m, l, f"{n_splits} x {per}")
            err = max_err(kvq.kv_merge_partials(p), want)
            log(f"  merged err {err:.3e}")
            assert err <= TOL
        # the one-call path is these two passes under its own plan (uneven sessions may take a
        # streamed launch instead, whose ranges the partial call cannot express: there the
        # oracle alone is the check)
        n_splits, per = kvq.kv_decode_plan(sessions, 0, hq)
        assert n_splits >= 1 and per % 512 == 0 and n_splits * per >= max(lens)
        full = kvq.kv_attend_decode(sessions, 0, qd, scale)
        assert max_err(full, want) <= TOL
        if n_splits > 1 and kvq.kv_decode_launch_kind(sessions, 0, hq) == 0:
            two = kvq.kv_merge_partials(kvq.kv_attend_decode_partial(sessions, 0, qd, scale, n_splits, per))
            assert torch.equal(full, two)
    finally:
        torch.cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)


@pytest.mark.parametrize("layout,d,g,n_ctx,n_new,plans", [
    ("K8V4", 128, 8, 1200, 300, [(1, 1536), (4, 384), (8, 192)]),
    ("K4V8", 64, 5, 100, 77, [(3, 64), (1, 192)]),
    ("KF8V4", 128, 8, 900, 120, [(1, 1024), (5, 256)]),
])
def test_chunk_partials_and_merge(layout, d, g, n_ctx, n_new, plans):
    log(f"chunk partials {layout} D={d} G={g} {n_ctx}+{n_new}")
    hkv = 2
    hq = hkv * g
    total = n_ctx + n_new
    torch = torch_mod()
    k, v, _ = I.workload_small(950 + d, total, hkv, d, hq, 1, bf16=True, n_outliers=4)
    q = I.bf16_round(I.normal((n_new, hq, d), 951 + d, 3))
    oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, total)
    oc.append(0, k, v)
    h = kvq.kv_cache_create(layout, 1, hkv, d, total)
    try:
        kvq.kv_append_quant(h, 0, dev(k, "bf16"), dev(v, "bf16"))
        scale = d ** -0.5
        qd = dev(q, "bf16")
        want = O.attend_chunk(oc, 0, q, n_new, scale)
        for n_splits, per in plans:
            p = kvq.kv_attend_chunk_partial(h, 0, qd, n_new, scale, n_splits, per)
            o, m, l = O.chunk_partials(oc, 0, q, n_new, scale, n_splits, per)
            compare_partials(p, o, m, l, f"{n_splits} x {per}")
            err = max_err(kvq.kv_merge_partials(p), want)
            log(f"  merged err {err:.3e}")
            assert err <= TOL
        n_splits, per = kvq.kv_chunk_plan(h, 0, hq, n_new)
        assert n_splits >= 1 and per % 64 == 0 and n_splits * per >= total
        full = kvq.kv_attend_chunk(h, 0, qd, n_new, scale)
        assert max_err(full, want) <= TOL
        if n_splits > 1:
            two = kvq.kv_merge_partials(kvq.kv_attend_chunk_partial(h, 0, qd, n_new, scale, n_splits, per))
            assert torch.equal(full, two)
    finally:
        torch.cuda.synchronize()
        kvq.kv_cache_destroy(h)


def test_merge_alone_on_oracle_partials():
    """a3 by itself: partials made by the oracle (then rounded to fp32), with splits whose
    references sit far apart and rows where only one split saw a key."""
    log("merge on oracle partials")
    torch = torch_mod()
    k, v, q = I.workload_small(960, 700, 1, 128, 4, 3)
    c = O.OracleCache(2, 1, 1, 128, 700)
    c.append(0, k, v)
    caches = [c, c, c]
    o, m, l = O.decode_partials(caches, 0, q, 128 ** -0.5, 6, 128)
    # move each split's reference by up to ~2^±24 (o and l stay well inside fp32's normal range)
    shift = I.normal((3, 4, 6), 961).astype(np.float64) * 8.0
    o, m, l = o * np.exp2(shift)[..., None], m - shift, l * np.exp2(shift)
    m[2, :, 1:], l[2, :, 1:], o[2, :, 1:] = -np.inf, 0.0, 0.0            # session 2: one split only
    p = np.concatenate([o, m[..., None], l[..., None]], axis=-1).astype(np.float32)
    o32, m32, l32 = (p[..., :128].astype(np.float64), p[..., 128].astype(np.float64),
                     p[..., 129].astype(np.float64))
    want = O.merge_partials(o32, m32, l32)
    got = kvq.kv_merge_partials(torch.from_numpy(p).cuda())
    err = max_err(got, want)
    log(f"  merge err {err:.3e}")
    assert err <= 1e-5          # fp32 merge of fp32 inputs; outputs are O(1)
    assert kvq.kv_merge_partials(torch.empty((0, 2, 130), dtype=torch.float32, device="cuda")).shape == (0, 128)


def test_partial_entry_points_reject_bad_splits():
    log("partial entry point errors")
    torch = torch_mod()
    h = kvq.kv_cache_create("K8V4", 1, 2, 64, 2000)
    try:
        k, v, q = I.workload_small(970, 1500, 2, 64, 4, 1, bf16=True)
        kvq.kv_append_quant(h, 0, dev(k, "bf16"), dev(v, "bf16"))
        qd = dev(q, "bf16")
        for n_splits, per in [(2, 500), (2, 512), (0, 2048), (1, 0), (70000, 512)]:   # not a multiple / too short / bad count
            with pytest.raises(kvq.KVError) as e:
                kvq.kv_attend_decode_partial([h], 0, qd, 0.125, n_splits, per)
            assert e.value.code == kvq.KV_EINVAL
        small = torch.empty((1, 4, 3, 66), dtype=torch.float32, device="cuda")
        with pytest.raises(ValueError):   # the binding checks the shape first
            kvq.kv_attend_decode_partial([h], 0, qd, 0.125, 4, 512, partials=small)
        arr = (ctypes.c_void_p * 1)(h)     # the library checks the byte count itself
        rc = kvq.lib().kv_attend_decode_partial(arr, 1, 0, qd.data_ptr(), kvq.KV_BF16, 4, 0.125, 4, 512,
                                                small.data_ptr(), small.numel() * 4,
                                                torch.cuda.current_stream().cuda_stream)
        assert rc == kvq.KV_EINVAL and "smaller" in kvq.kv_last_error()
        qc = dev(q.repeat(10, axis=0), "bf16")
        for n_splits, per in [(2, 700), (1, 1024), (70000, 64)]:
            with pytest.raises(kvq.KVError) as e:
                kvq.kv_attend_chunk_partial(h, 0, qc, 10, 0.125, n_splits, per)
            assert e.value.code in (kvq.KV_EINVAL, kvq.KV_EUNSUPPORTED)
        assert kvq.kv_cache_len(h, 0) == 1500
    finally:
        torch.cuda.synchronize()
        kvq.kv_cache_destroy(h)


def test_ragged_batch_spreads_the_long_session():
    """Lengths that differ by four orders of magnitude: the plan cuts the long session into
    many splits (the short ones keep one busy split each), and the result still matches the
    oracle, pass by pass.  The one-call path launches only the busy splits and its merge
    reads no other partial: a workspace full of NaN gives the same output.  The partial
    pass writes every split, the empty ones as (-inf, 0, 0)."""
    log("ragged batch plan")
    torch = torch_mod()
    lens = [20000, 300, 50, 4096, 1, 700]
    hkv, g, d = 2, 4, 128
    hq = hkv * g
    q = I.bf16_round(I.normal((len(lens), hq, d), 980, 9))
    sessions, ocs = [], []
    try:
        for i, n in enumerate(lens):
            k, v, _ = I.workload_small(981 + i, n, hkv, d, hq, 1, bf16=True, n_outliers=4)
            h = kvq.kv_cache_create("K8V4", 1, hkv, d, n)
            sessions.append(h)
            kvq.kv_append_quant(h, 0, dev(k, "bf16"), dev(v, "bf16"))
            oc = O.OracleCache(O.LAYOUT_IDS["K8V4"], 1, hkv, d, n)
            oc.append(0, k, v)
            ocs.append(oc)
        scale = d ** -0.5
        qd = dev(q, "bf16")
        n_splits, per = kvq.kv_decode_plan(sessions, 0, hq)
        log(f"  plan {n_splits} x {per}")
        assert n_splits > 4 and n_splits * per >= max(lens)
        want = O.attend_decode(ocs, 0, q, scale)
        err = max_err(kvq.kv_attend_decode(sessions, 0, qd, scale), want)
        log(f"  one call err {err:.3e}")
        assert err <= TOL
        nb = kvq.kv_decode_workspace_bytes(sessions, 0, hq)
        ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=qd.device)   # every float NaN
        err = max_err(kvq.kv_attend_decode(sessions, 0, qd, scale, workspace=ws), want)
        log(f"  one call over a NaN-filled workspace err {err:.3e}")
        assert err <= TOL
        p = kvq.kv_attend_decode_partial(sessions, 0, qd, scale, n_splits, per)
        o, m, l = O.decode_partials(ocs, 0, q, scale, n_splits, per)
        compare_partials(p, o, m, l, f"{n_splits} x {per}")
    finally:
        torch.cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)

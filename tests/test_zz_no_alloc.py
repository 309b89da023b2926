"""kv_attend_decode_static: the decode entry point that allocates nothing (its split partials
live in the library's static device scratch) gives exactly kv_attend_decode's output, on two
calls in a row (the second smaller), and rejects a plan whose partials exceed the scratch."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import TOL, dev, log, max_err, torch_mod

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


def _batch(lens, hkv, d, hq, seed):
    torch = torch_mod()
    hs, ocs = [], []
    q = I.normal((len(lens), hq, d), seed, 99)
    for i, n in enumerate(lens):
        k, v, _ = I.workload_small(seed + i, n, hkv, d, hq, 1, n_outliers=4)
        h = kvq.kv_cache_create("K8V4", 1, hkv, d, n)
        kvq.kv_append_quant(h, 0, dev(k, "f32"), dev(v, "f32"))
        oc = O.OracleCache(O.LAYOUT_IDS["K8V4"], 1, hkv, d, n)
        oc.append(0, k, v)
        hs.append(h)
        ocs.append(oc)
    torch.cuda.synchronize()
    return hs, ocs, q


def _compare(hs, ocs, q, d):
    torch = torch_mod()
    hq = q.shape[1]
    n_splits, tps = kvq.kv_decode_plan(hs, 0, hq)
    qd = dev(q, "f32")
    want = kvq.kv_attend_decode(hs, 0, qd, d ** -0.5)
    out = torch.full_like(want, float("nan"))
    kvq.kv_attend_decode_static(hs, 0, qd, d ** -0.5, out)
    torch.cuda.synchronize()
    err = max_err(out, O.attend_decode(ocs, 0, q, d ** -0.5))
    log(f"  plan {n_splits} x {tps}: static == workspace call: {bool(torch.equal(out, want))}, "
        f"max err vs oracle {err:.3e}")
    assert torch.equal(out, want)
    assert err <= TOL
    return n_splits


def test_static_decode_equals_the_workspace_call_twice():
    torch = torch_mod()
    d = 128
    first = ([20000, 300, 4096, 1, 700], 2, 16)     # (lengths, Hkv, Hq)
    second = ([2500, 64], 2, 8)                     # smaller: fewer sessions, rows and tokens
    hs, ocs, q = _batch(*first[:2], d, first[2], 7100)
    try:
        log("static decode, call 1")
        assert _compare(hs, ocs, q, d) > 1        # the scratch holds split partials
    finally:
        torch.cuda.synchronize()
        for h in hs:
            kvq.kv_cache_destroy(h)
    hs, ocs, q = _batch(*second[:2], d, second[2], 7200)
    try:
        log("static decode, call 2 (smaller)")
        _compare(hs, ocs, q, d)
    finally:
        torch.cuda.synchronize()
        for h in hs:
            kvq.kv_cache_destroy(h)


def test_static_decode_rejects_a_plan_beyond_the_scratch():
    """64 sessions, one of them long: the plan spreads the long one over many splits, and
    n_splits x 2048 rows x 130 floats of partials exceed 16 MiB."""
    torch = torch_mod()
    d, hkv, hq = 128, 8, 32
    lens = [65536] + [256] * 63
    hs = []
    try:
        for i, n in enumerate(lens):
            h = kvq.kv_cache_create("K8V4", 1, hkv, d, n)
            k = torch.zeros((n, hkv, d), dtype=torch.bfloat16, device="cuda")
            kvq.kv_append_quant(h, 0, k, k)
            hs.append(h)
        n_splits, _ = kvq.kv_decode_plan(hs, 0, hq)
        need = n_splits * len(lens) * hq * (d + 2) * 4 if n_splits > 1 else 0
        log(f"  plan {n_splits} splits: {need} bytes of partials")
        q = torch.zeros((len(lens), hq, d), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((len(lens), hq, d), dtype=torch.float32, device="cuda")
        if need <= SCRATCH_BYTES:
            pytest.skip(f"this device's plan ({n_splits} splits) fits the scratch")
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_attend_decode_static(hs, 0, q, d ** -0.5, out)
        assert e.value.code == kvq.KV_EINVAL and "static scratch" in str(e.value)
    finally:
        torch.cuda.synchronize()
        for h in hs:
            kvq.kv_cache_destroy(h)

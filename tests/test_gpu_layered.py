"""Caches with a layout per layer (layer-specific quantization): every layer's planes are
the oracle's bit for bit, attention per layer matches the oracle, and sessions and
multi-session decode follow each layer's own layout."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import TOL, dev, log, max_err, torch_mod
from test_gpu_session import PLANES, parse_saved

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


def layered_pair(layouts, hkv=2, d=128, cap=700, seed=1000):
    lids = [O.LAYOUT_IDS[x] for x in layouts]
    h = kvq.kv_cache_create_layered(layouts, hkv, d, cap)
    oc = O.OracleLayeredCache(lids, hkv, d, cap)
    for l in range(len(layouts)):
        n = 100 + 120 * l
        k, v, _ = I.workload_small(seed + l, n, hkv, d, hkv, 1, bf16=True, n_outliers=4)
        kvq.kv_append_quant(h, l, dev(k, "bf16"), dev(v, "bf16"))
        oc.append(l, k, v)
    return h, oc


def test_layered_cache_matches_oracle():
    log("layered cache parity")
    torch = torch_mod()
    h, oc = layered_pair(LAYOUTS)
    try:
        assert kvq.kv_footprint_bytes(h) == oc.footprint_bytes()
        assert [kvq.kv_cache_layout(h, l) for l in range(len(LAYOUTS))] == [O.LAYOUT_IDS[x] for x in LAYOUTS]
        for l in range(len(LAYOUTS)):
            n = oc.len[l]
            for hh in range(2):
                for name, p in PLANES:
                    want = oc.plane(l, name)[hh, :n]
                    assert np.array_equal(kvq.read_plane(h, l, hh, p, 0, n), want), (l, hh, name)
            q = I.bf16_round(I.normal((1, 8, 128), 1010 + l))
            err_d = max_err(kvq.kv_attend_decode([h], l, dev(q, "bf16"), 128 ** -0.5),
                            O.attend_decode([oc], l, q, 128 ** -0.5))
            qc = I.bf16_round(I.normal((37, 8, 128), 1020 + l))
            err_c = max_err(kvq.kv_attend_chunk(h, l, dev(qc, "bf16"), 37, 128 ** -0.5),
                            O.attend_chunk(oc, l, qc, 37, 128 ** -0.5))
            log(f"  layer {l} {LAYOUTS[l]}: decode err {err_d:.3e}, chunk err {err_c:.3e}")
            assert err_d <= TOL and err_c <= TOL
    finally:
        torch.cuda.synchronize()
        kvq.kv_cache_destroy(h)


def test_decode_batch_needs_the_layer_layout_to_agree():
    log("layered multi-session decode")
    torch = torch_mod()
    a, oa = layered_pair(["K8V4", "K4V4"], seed=1030)
    b, ob = layered_pair(["K8V4", "K8V8"], seed=1040)
    try:
        q = I.bf16_round(I.normal((2, 8, 128), 1050))
        out = kvq.kv_attend_decode([a, b], 0, dev(q, "bf16"), 128 ** -0.5)
        assert max_err(out, O.attend_decode([oa, ob], 0, q, 128 ** -0.5)) <= TOL
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_attend_decode([a, b], 1, dev(q, "bf16"), 128 ** -0.5)
        assert e.value.code == kvq.KV_EINVAL and "layout" in str(e.value)
    finally:
        torch.cuda.synchronize()
        kvq.kv_cache_destroy(a)
        kvq.kv_cache_destroy(b)


def test_layered_session_round_trip():
    log("layered session round trip")
    torch = torch_mod()
    layouts = ["K8V4", "FP16", "K4V4"]
    h, oc = layered_pair(layouts, hkv=3, d=64, cap=500, seed=1060)
    h2 = kvq.kv_cache_create_layered(layouts, 3, 64, 500)
    h3 = kvq.kv_cache_create_layered(["K8V4", "FP16", "K4V8"], 3, 64, 500)
    try:
        buf = torch.empty(kvq.kv_session_bytes(h), dtype=torch.uint8, pin_memory=True)
        kvq.kv_session_save(h, buf)
        torch.cuda.synchronize()
        hdr, lens, lids, planes, end = parse_saved(buf.numpy(), oc)
        assert hdr[1:] == (2, -1, 3, 3, 64) and lids == [O.LAYOUT_IDS[x] for x in layouts]
        assert lens == oc.len and end == buf.numel()
        for (l, hh, name), rows in planes.items():
            assert np.array_equal(rows, oc.plane(l, name)[hh, :lens[l]])
        kvq.kv_session_load(h2, buf)
        q = dev(I.bf16_round(I.normal((1, 6, 64), 1070)), "bf16")
        for l in range(3):
            assert torch.equal(kvq.kv_attend_decode([h], l, q, 0.125), kvq.kv_attend_decode([h2], l, q, 0.125))
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_session_load(h3, buf)        # layer 2 stored in another layout
        assert e.value.code == kvq.KV_EINVAL
        assert kvq.kv_cache_len(h3, 0) == 0
    finally:
        torch.cuda.synchronize()
        for x in (h, h2, h3):
            kvq.kv_cache_destroy(x)

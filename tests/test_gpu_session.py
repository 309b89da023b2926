"""Session offload and restore through the C ABI: the saved bytes are the oracle's planes in
the documented order, a restored cache is byte-identical to the one saved, and attention
over it is bit-identical."""
from __future__ import annotations

import struct

import numpy as np
import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import dev, host_inputs, log, torch_mod

pytestmark = pytest.mark.gpu

PLANES = (("Kc", kvq.KV_PLANE_KC), ("Ks", kvq.KV_PLANE_KS), ("Vc", kvq.KV_PLANE_VC), ("Vs", kvq.KV_PLANE_VS))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.lib()
    yield
    torch.cuda.synchronize()


def parse_saved(buf: np.ndarray, oc: O.OracleCache):
    """Split a saved session (documented format) into header fields and per-plane rows."""
    magic, version, layout, n_layers, hkv, d, _ = struct.unpack_from("<IIiiiiq", buf, 0)
    lens = list(struct.unpack_from(f"<{n_layers}q", buf, 32))
    layouts = list(struct.unpack_from(f"<{n_layers}i", buf, 32 + 8 * n_layers))
    off = -(-(32 + 12 * n_layers) // 64) * 64
    planes = {}
    for l in range(n_layers):
        for h in range(hkv):
            for name, _ in PLANES:
                plane = oc.plane(l, name) if hasattr(oc, "plane") else getattr(oc, name)[l]
                rb = plane.shape[-1]
                n = lens[l] * rb
                planes[(l, h, name)] = buf[off:off + n].reshape(lens[l], rb)
                off += n
    return (magic, version, layout, n_layers, hkv, d), lens, layouts, planes, off


def filled_pair(layout, dtype="bf16"):
    """A 2-layer cache with different lengths per layer, and its oracle twin."""
    hkv, d, cap = 3, 64, 1000
    lid = O.LAYOUT_IDS[layout]
    h = kvq.kv_cache_create(layout, 2, hkv, d, cap)
    oc = O.OracleCache(lid, 2, hkv, d, cap)
    for layer, n in ((0, 700), (1, 333)):
        k, v, _ = I.workload_small(990 + layer, n, hkv, d, hkv, 1, bf16=(dtype == "bf16"), n_outliers=2)
        kvq.kv_append_quant(h, layer, dev(k, dtype), dev(v, dtype))
        oc.append(layer, host_inputs(k, dtype), host_inputs(v, dtype))
    return h, oc


@pytest.mark.parametrize("layout", ["K8V4", "FP16", "K4V8", "KF8V4"])
@pytest.mark.parametrize("pinned", [True, False])
def test_save_restore_round_trip(layout, pinned):
    log(f"session round trip {layout} pinned={pinned}")
    torch = torch_mod()
    h, oc = filled_pair(layout)
    h2 = kvq.kv_cache_create(layout, 2, 3, 64, 1000)
    try:
        nbytes = kvq.kv_session_bytes(h)
        buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) if pinned else np.zeros(nbytes, np.uint8)
        kvq.kv_session_save(h, buf)
        torch.cuda.synchronize()
        host = buf.numpy() if pinned else buf
        hdr, lens, layouts, planes, end = parse_saved(host, oc)
        lid = O.LAYOUT_IDS[layout]
        assert hdr == (0x5351564B, 2, lid, 2, 3, 64) and lens == [700, 333] and layouts == [lid, lid]
        assert end == nbytes
        for (l, hh, name), rows in planes.items():
            assert np.array_equal(rows, getattr(oc, name)[l, hh, :lens[l]]), (l, hh, name)
        kvq.kv_session_load(h2, buf)
        torch.cuda.synchronize()
        assert [kvq.kv_cache_len(h2, l) for l in range(2)] == [700, 333]
        for l in range(2):
            for hh in range(3):
                for _, p in PLANES:
                    assert np.array_equal(kvq.read_plane(h2, l, hh, p, 0, lens[l]), kvq.read_plane(h, l, hh, p, 0, lens[l]))
        q = dev(I.bf16_round(I.normal((1, 6, 64), 995)), "bf16")
        for l in range(2):
            a = kvq.kv_attend_decode([h], l, q, 0.125)
            b = kvq.kv_attend_decode([h2], l, q, 0.125)
            assert torch.equal(a, b)
        qc = dev(I.bf16_round(I.normal((40, 6, 64), 996)), "bf16")
        assert torch.equal(kvq.kv_attend_chunk(h, 1, qc, 40, 0.125), kvq.kv_attend_chunk(h2, 1, qc, 40, 0.125))
    finally:
        torch.cuda.synchronize()
        kvq.kv_cache_destroy(h)
        kvq.kv_cache_destroy(h2)


def test_restore_rejects_mismatches():
    log("session restore errors")
    torch = torch_mod()
    h, oc = filled_pair("K8V4")
    others = []
    try:
        buf = torch.empty(kvq.kv_session_bytes(h), dtype=torch.uint8, pin_memory=True)
        kvq.kv_session_save(h, buf)
        torch.cuda.synchronize()

        def expect(code, cache, src):
            with pytest.raises(kvq.KVError) as e:
                kvq.kv_session_load(cache, src)
            assert e.value.code == code, str(e.value)

        other = kvq.kv_cache_create("K4V4", 2, 3, 64, 1000); others.append(other)
        expect(kvq.KV_EINVAL, other, buf)                       # layout differs
        small = kvq.kv_cache_create("K8V4", 2, 3, 64, 500); others.append(small)
        expect(kvq.KV_ECAPACITY, small, buf)                    # 700 saved tokens > 500
        assert kvq.kv_cache_len(small, 0) == 0                  # unchanged on error
        good = kvq.kv_cache_create("K8V4", 2, 3, 64, 1000); others.append(good)
        expect(kvq.KV_EINVAL, good, buf[:-1])                   # truncated
        bad = buf.clone()
        bad[0] ^= 1
        expect(kvq.KV_EINVAL, good, bad)                        # magic
        with pytest.raises(ValueError):
            kvq.kv_session_load(good, buf.cuda())               # device memory (binding)
        dbuf = buf.cuda()
        assert kvq.lib().kv_session_load(good, dbuf.data_ptr(), dbuf.numel(), None) == kvq.KV_EINVAL
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_session_save(h, torch.empty(16, dtype=torch.uint8))   # too small
        assert e.value.code == kvq.KV_EINVAL
        assert [kvq.kv_cache_len(good, l) for l in range(2)] == [0, 0]
    finally:
        torch.cuda.synchronize()
        kvq.kv_cache_destroy(h)
        for o in others:
            kvq.kv_cache_destroy(o)

"""Helpers shared by the GPU parity tests (test harness, not product code)."""
from __future__ import annotations

import contextlib
import sys

import numpy as np

import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

TOL = 5e-3   # max abs error of attention outputs against the oracle


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev(x: np.ndarray, dtype: str):
    """numpy fp32 (bf16 values for 'bf16') -> contiguous device tensor of dtype."""
    torch = torch_mod()
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device="cuda").to(tdt).contiguous()


def host_inputs(x: np.ndarray, dtype: str) -> np.ndarray:
    """The values the oracle must see for a device tensor made by dev(x, dtype)."""
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":   # torch's fp32 -> bf16 conversion rounds to nearest even
        return I.bf16_round(x)
    return np.asarray(x, np.float32)


@contextlib.contextmanager
def gpu_cache(layout, n_layers, n_kv_heads, head_dim, max_tokens):
    h = kvq.kv_cache_create(layout, n_layers, n_kv_heads, head_dim, max_tokens)
    try:
        yield h
        torch_mod().cuda.synchronize()
        kvq.kv_cache_check_guard(h)   # nothing wrote past the planes
    finally:
        torch_mod().cuda.synchronize()
        kvq.kv_cache_destroy(h)


def assert_planes_equal(h, oc, layer: int, t0: int = 0, t1: int | None = None) -> None:
    """Cache bytes of rows [t0, t1) of every plane equal the oracle's, bit for bit."""
    t1 = oc.len[layer] if t1 is None else t1
    for kvh in range(oc.Hkv):
        for plane, name in ((kvq.KV_PLANE_KC, "Kc"), (kvq.KV_PLANE_KS, "Ks"),
                            (kvq.KV_PLANE_VC, "Vc"), (kvq.KV_PLANE_VS, "Vs")):
            want = getattr(oc, name)[layer, kvh, t0:t1]
            got = kvq.read_plane(h, layer, kvh, plane, t0, t1 - t0)
            assert got.shape == want.shape, (name, got.shape, want.shape)
            if not np.array_equal(got, want):
                bad = np.argwhere(got != want)
                raise AssertionError(f"plane {name} layer {layer} kv head {kvh}: {len(bad)} bytes differ, "
                                     f"first at row {t0 + bad[0][0]} byte {bad[0][1]}: "
                                     f"gpu {got[tuple(bad[0])]:#x} oracle {want[tuple(bad[0])]:#x}")


def max_err(got, want) -> float:
    g = got.detach().cpu().numpy().astype(np.float64) if hasattr(got, "detach") else np.asarray(got, np.float64)
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want)))

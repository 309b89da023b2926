"""Seeded synthetic inputs for the quantized KV cache workloads.

This module holds no arithmetic of the method: it only draws random numbers and
applies each workload's input recipe (outlier key channels, heavy-tailed channel
scales, rounding of fp32 draws to bf16).  Both the tests' oracle side and the
GPU side take their inputs from here.

Every array is drawn from numpy ``Generator(PCG64(SeedSequence(...)))``.  Large
workloads are generated per session or per chunk from their own spawned
sequence, so any slice can be regenerated on its own (random access), and the
draws are spread over a few threads.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits", "normal", "outlier_channels", "workload_small",
    "decode_128_tokens", "layers22_8192_tokens", "turn_100k_plus_500", "batch64x32k_session", "batch64x32k_queries",
    "rebuild131k_chunk", "ragged_lengths", "WORKLOADS",
]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_round(x) -> np.ndarray:
    """fp32 -> nearest-even bf16, returned as fp32 values (exactly bf16-representable)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    return (r << np.uint32(16)).astype(np.uint32).view(np.float32)


def bf16_bits(x_bf16_values) -> np.ndarray:
    """The uint16 bit patterns of fp32 arrays that already hold bf16 values."""
    b = np.ascontiguousarray(x_bf16_values, dtype=np.float32).view(np.uint32)
    return (b >> np.uint32(16)).astype(np.uint16)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def normal(shape, *key) -> np.ndarray:
    """N(0, 1) float32 of ``shape`` from the stream named by ``key``.

    The leading axis is split into slabs drawn by separate spawned streams on
    a few threads; the result depends only on ``key`` and ``shape``.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.float32)
    if out.size == 0:
        return out
    n0 = shape[0]
    slab = max(1, -(-n0 // 64))
    starts = list(range(0, n0, slab))

    def fill(i):
        s = starts[i]
        rng = _rng(*key, 0x51AB, i)
        out[s:s + slab] = rng.standard_normal(out[s:s + slab].shape, dtype=np.float32)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(starts))))
    return out


def outlier_channels(n_kv_heads: int, head_dim: int, n_out: int, *key) -> np.ndarray:
    """Boolean mask [Hkv, D]: per KV head, ``n_out`` channels chosen without replacement."""
    rng = _rng(*key, 0x0C7)
    mask = np.zeros((n_kv_heads, head_dim), bool)
    for h in range(n_kv_heads):
        mask[h, rng.choice(head_dim, size=n_out, replace=False)] = True
    return mask


def log10_uniform(shape, lo: float, hi: float, *key) -> np.ndarray:
    """float32 10^u with u uniform in [lo, hi), from the stream named by ``key``."""
    u = _rng(*key, 0x10C).uniform(lo, hi, size=tuple(int(s) for s in shape))
    return np.power(10.0, u).astype(np.float32)


def workload_small(seed: int, n_tokens: int, n_kv_heads: int, head_dim: int,
                   n_q_heads: int, n_q_rows: int, bf16: bool = False,
                   n_outliers: int = 0, outlier_factor: float = 8.0):
    """Generic small workload: K, V [n_tokens, Hkv, D], Q [n_q_rows, Hq, D]."""
    k = normal((n_tokens, n_kv_heads, head_dim), seed, 1)
    v = normal((n_tokens, n_kv_heads, head_dim), seed, 2)
    q = normal((n_q_rows, n_q_heads, head_dim), seed, 3)
    if n_outliers:
        k = np.where(outlier_channels(n_kv_heads, head_dim, n_outliers, seed, 4)[None],
                     k * np.float32(outlier_factor), k).astype(np.float32)
    if bf16:
        k, v, q = bf16_round(k), bf16_round(v), bf16_round(q)
    return k, v, q


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------
def decode_128_tokens(seed: int = 1):
    """1 layer, 128 cached tokens, Hq 32, Hkv 4, D 64, fp32 N(0,1); K8V4; one query."""
    k = normal((128, 4, 64), seed, 1)
    v = normal((128, 4, 64), seed, 2)
    q = normal((1, 32, 64), seed, 3)
    return dict(k=k, v=v, q=q, layout="K8V4", n_layers=1, n_kv_heads=4, head_dim=64,
                n_q_heads=32, dtype="f32")


def layers22_8192_tokens(seed: int = 2, n_layers: int = 22, n_tokens: int = 8192):
    """22 layers x 4 KV heads x 64, Hq 32, 8192 tokens, fp32; 4 of 64 key channels x8
    per (layer, KV head).  K, V [L, T, Hkv, D]; Q [L, 1, Hq, D]."""
    k = np.empty((n_layers, n_tokens, 4, 64), np.float32)
    v = np.empty_like(k)
    for l in range(n_layers):
        kl = normal((n_tokens, 4, 64), seed, 1, l)
        mask = outlier_channels(4, 64, 4, seed, 4, l)
        k[l] = np.where(mask[None], kl * np.float32(8.0), kl)
        v[l] = normal((n_tokens, 4, 64), seed, 2, l)
    q = normal((n_layers, 1, 32, 64), seed, 3)
    return dict(k=k, v=v, q=q, n_layers=n_layers, n_kv_heads=4, head_dim=64,
                n_q_heads=32, dtype="f32")


def turn_100k_plus_500(seed: int = 3, n_ctx: int = 100_000, n_new: int = 500):
    """1 layer, Hq 64, Hkv 8, D 128, bf16.  K, V [n_ctx + n_new, 8, 128] with 8 of 128
    key channels x8 per KV head (before the bf16 cast); Q [n_new, 64, 128]."""
    n = n_ctx + n_new
    k = normal((n, 8, 128), seed, 1)
    mask = outlier_channels(8, 128, 8, seed, 4)
    k = bf16_round(np.where(mask[None], k * np.float32(8.0), k))
    v = bf16_round(normal((n, 8, 128), seed, 2))
    q = bf16_round(normal((n_new, 64, 128), seed, 3))
    return dict(k=k, v=v, q=q, n_ctx=n_ctx, n_new=n_new, layout="K8V4", n_layers=1,
                n_kv_heads=8, head_dim=128, n_q_heads=64, dtype="bf16")


def batch64x32k_session(s: int, seed: int = 4, n_tokens: int = 32_768):
    """Session ``s`` of the batched-decode workload (bf16): K = z * c with z ~ N(0,1) and a
    per-(session, KV head, channel) scale c = exp(N(0,1)); V ~ N(0,1).  [T, 8, 128] each."""
    z = normal((n_tokens, 8, 128), seed, 1, s)
    c = np.exp(_rng(seed, 5, s).standard_normal((8, 128))).astype(np.float32)
    k = bf16_round(z * c[None])
    v = bf16_round(normal((n_tokens, 8, 128), seed, 2, s))
    return k, v


def batch64x32k_queries(seed: int = 4, n_sessions: int = 64):
    """One bf16 query per session: [S, 32, 128]."""
    return bf16_round(normal((n_sessions, 32, 128), seed, 3))


def rebuild131k_chunk(c: int, seed: int = 5, chunk: int = 4096):
    """Tokens [chunk*c, chunk*(c+1)) of the 131,072-token rebuild (bf16):
    K, V [chunk, 8, 128], Q [chunk, 40, 128], all N(0,1)."""
    k = bf16_round(normal((chunk, 8, 128), seed, 1, c))
    v = bf16_round(normal((chunk, 8, 128), seed, 2, c))
    q = bf16_round(normal((chunk, 40, 128), seed, 3, c))
    return k, v, q


def ragged_lengths(n_sessions: int = 64, lo: int = 512, hi: int = 32_768, seed: int = 7) -> np.ndarray:
    """Cached lengths of a batch of sessions at different points of their conversations:
    log-uniform integers in [lo, hi] (int64)."""
    u = _rng(seed, 0x5A6).random(n_sessions)
    return np.floor(np.exp(np.log(lo) + u * (np.log(hi + 1) - np.log(lo)))).astype(np.int64).clip(lo, hi)


WORKLOADS = {
    "decode_128_tokens": "1 layer, 128 tokens, Hq 32 / Hkv 4 / D 64, fp32, K8V4, decode",
    "layers22_8192_tokens": "22 layers x 4 KV heads x 64, Hq 32, 8192 tokens, fp32, all layouts, decode",
    "turn_100k_plus_500": "100,000 cached + 500 new tokens, Hq 64 / Hkv 8 / D 128, bf16, K8V4, chunk append",
    "batch64x32k": "64 sessions x 32,768 tokens, Hq 32 / Hkv 8 / D 128, bf16, K8V4 and K4V8, decode",
    "rebuild131k": "131,072 tokens as 32 chunks of 4096, Hq 40 / Hkv 8 / D 128, bf16, K8V4, rebuild",
}

"""ctypes binding of ``libkvq.so`` (declared in ``include/kvq.h``).

Argument marshalling only: every function here forwards to the C entry point of
the same name; torch tensors supply device pointers and the current HIP stream.
There is no fallback: if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path

LIB_PATH = Path(__file__).resolve().with_name("libkvq.so")

KV_OK, KV_EINVAL, KV_ECAPACITY, KV_ENOMEM, KV_EUNSUPPORTED, KV_EEMPTY, KV_EHIP = 0, -1, -2, -3, -4, -5, -6
KV_FP16, KV_K8V8, KV_K8V4, KV_K4V8, KV_K4V4, KV_KF8V4 = 0, 1, 2, 3, 4, 5
KV_F32, KV_BF16, KV_F16 = 0, 1, 2
KV_PLANE_KC, KV_PLANE_KS, KV_PLANE_VC, KV_PLANE_VS = 0, 1, 2, 3
LAYOUT_IDS = {"FP16": 0, "K8V8": 1, "K8V4": 2, "K4V8": 3, "K4V4": 4, "KF8V4": 5}
STATUS_NAMES = {0: "KV_OK", -1: "KV_EINVAL", -2: "KV_ECAPACITY", -3: "KV_ENOMEM",
                -4: "KV_EUNSUPPORTED", -5: "KV_EEMPTY", -6: "KV_EHIP"}

_SIGS = {
    "kv_cache_create": (C.c_void_p, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64]),
    "kv_cache_create_layered": (C.c_void_p, [C.POINTER(C.c_int), C.c_int, C.c_int, C.c_int, C.c_int64]),
    "kv_cache_layout": (C.c_int, [C.c_void_p, C.c_int]),
    "kv_cache_shape": (C.c_int, [C.c_void_p, C.POINTER(C.c_int), C.POINTER(C.c_int), C.POINTER(C.c_int),
                                 C.POINTER(C.c_int64)]),
    "kv_cache_check_guard": (C.c_int, [C.c_void_p]),
    "kv_layered_footprint_bytes": (C.c_int64, [C.POINTER(C.c_int), C.c_int, C.c_int, C.c_int, C.c_int64]),
    "kv_cache_destroy": (None, [C.c_void_p]),
    "kv_append_quant": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int64, C.c_void_p]),
    "kv_attend_decode": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_float,
                                   C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kv_attend_decode_static": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_float,
                                          C.c_void_p, C.c_void_p]),
    "kv_decode_workspace_bytes": (C.c_int64, [C.c_void_p, C.c_int, C.c_int, C.c_int]),
    "kv_decode_launch_kind": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_size_t]),
    "kv_decode_plan": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_int),
                                 C.POINTER(C.c_int64)]),
    "kv_attend_decode_partial": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_float,
                                           C.c_int, C.c_int64, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kv_merge_partials": (C.c_int, [C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "kv_chunk_plan": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int64, C.POINTER(C.c_int),
                                C.POINTER(C.c_int64)]),
    "kv_attend_chunk_partial": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_int64, C.c_float,
                                          C.c_int, C.c_int64, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kv_attend_chunk": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_int64, C.c_float,
                                  C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kv_chunk_workspace_bytes": (C.c_int64, [C.c_void_p, C.c_int, C.c_int, C.c_int64]),
    "kv_footprint_bytes": (C.c_int64, [C.c_void_p]),
    "kv_layout_footprint_bytes": (C.c_int64, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64]),
    "kv_cache_len": (C.c_int64, [C.c_void_p, C.c_int]),
    "kv_cache_reset": (C.c_int, [C.c_void_p]),
    "kv_cache_truncate": (C.c_int, [C.c_void_p, C.c_int, C.c_int64]),
    "kv_cache_plane": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_void_p),
                                 C.POINTER(C.c_int64)]),
    "kv_cache_copy_plane": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64,
                                      C.c_void_p, C.c_void_p]),
    "kv_session_bytes": (C.c_int64, [C.c_void_p]),
    "kv_session_save": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kv_session_load": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kv_last_error": (C.c_char_p, []),
    "kv_last_status": (C.c_int, []),
}

_lib = None


class KVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def lib() -> C.CDLL:
    """Load ``libkvq.so`` once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m asymmetric_quantized_kv_amd.build`")
        h = C.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _lib = h
    return _lib


def kv_last_error() -> str:
    return lib().kv_last_error().decode()


def kv_last_status() -> int:
    return lib().kv_last_status()


def _check(rc: int) -> int:
    if rc < 0:
        raise KVError(rc, kv_last_error())
    return rc


# ---------------------------------------------------------------------------
# torch plumbing
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: KV_F32, torch.bfloat16: KV_BF16, torch.float16: KV_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _dev_ptr(t, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _same_device(t, ref, name: str) -> None:
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _expect_f32(t, shape, name: str) -> None:
    """A caller-supplied output: fp32 of exactly this shape."""
    torch = _torch()
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32 (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _cache_shape(cache: int):
    """(n_layers, n_kv_heads, head_dim, max_tokens) of a cache, from the library."""
    nl, hkv, d, mt = C.c_int(), C.c_int(), C.c_int(), C.c_int64()
    _check(lib().kv_cache_shape(cache, C.byref(nl), C.byref(hkv), C.byref(d), C.byref(mt)))
    return nl.value, hkv.value, d.value, mt.value


def _sessions_shape(sessions):
    if len(sessions) == 0:
        raise ValueError("at least one session is needed")
    return _cache_shape(sessions[0])


def _check_q(q, n_rows: int, rows_name: str, head_dim: int, n_kv_heads: int) -> None:
    if q.dim() != 3:
        raise ValueError(f"q must be [{rows_name}, n_q_heads, head_dim] (got shape {tuple(q.shape)})")
    if q.shape[0] != n_rows:
        raise ValueError(f"q's first dimension must equal {rows_name} ({n_rows}, got {q.shape[0]})")
    if q.shape[2] != head_dim:
        raise ValueError(f"q's head_dim {q.shape[2]} differs from the cache's {head_dim}")
    if q.shape[1] < 1 or q.shape[1] % n_kv_heads:
        raise ValueError(f"n_q_heads {q.shape[1]} is not a positive multiple of n_kv_heads {n_kv_heads}")
    _dtype_code(q)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def kv_cache_create(layout, n_layers: int, n_kv_heads: int, head_dim: int, max_tokens: int) -> int:
    if isinstance(layout, str):
        layout = LAYOUT_IDS[layout]
    h = lib().kv_cache_create(int(layout), n_layers, n_kv_heads, head_dim, max_tokens)
    if not h:
        raise KVError(lib().kv_last_status(), kv_last_error())
    return h


def _layout_array(layouts):
    ids = [LAYOUT_IDS[x] if isinstance(x, str) else int(x) for x in layouts]
    return (C.c_int * len(ids))(*ids), len(ids)


def kv_cache_create_layered(layouts, n_kv_heads: int, head_dim: int, max_tokens: int) -> int:
    """A cache whose layer l uses layouts[l] (names or codes)."""
    arr, n = _layout_array(layouts)
    h = lib().kv_cache_create_layered(arr, n, n_kv_heads, head_dim, max_tokens)
    if not h:
        raise KVError(lib().kv_last_status(), kv_last_error())
    return h


def kv_cache_layout(cache: int, layer: int) -> int:
    return _check(lib().kv_cache_layout(cache, layer))


def kv_cache_shape(cache: int):
    """(n_layers, n_kv_heads, head_dim, max_tokens)."""
    return _cache_shape(cache)


def kv_layered_footprint_bytes(layouts, n_kv_heads: int, head_dim: int, max_tokens: int) -> int:
    arr, n = _layout_array(layouts)
    return _check(lib().kv_layered_footprint_bytes(arr, n, n_kv_heads, head_dim, max_tokens))


def kv_cache_check_guard(cache: int) -> None:
    """Raise KVError if the guard bytes after the cache's arena were overwritten."""
    _check(lib().kv_cache_check_guard(cache))


def kv_cache_destroy(cache: int) -> None:
    lib().kv_cache_destroy(cache)


def kv_append_quant(cache: int, layer: int, k, v, stream=None) -> None:
    """k, v: device tensors [n_new, n_kv_heads, head_dim] (fp32 / bf16 / fp16)."""
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 3:
        raise ValueError("k and v must be [n_new, n_kv_heads, head_dim] of one dtype")
    _, hkv, d, _ = _cache_shape(cache)
    if tuple(k.shape[1:]) != (hkv, d):
        raise ValueError(f"k and v must be [n_new, {hkv}, {d}] for this cache (got {tuple(k.shape)})")
    _dtype_code(k)
    _same_device(v, k, "v")
    _check(lib().kv_append_quant(cache, layer, _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(k),
                                 k.shape[0], _stream(stream)))


def _handles(sessions):
    arr = (C.c_void_p * len(sessions))(*sessions)
    return arr


def kv_decode_workspace_bytes(sessions, layer: int, n_q_heads: int) -> int:
    return _check(lib().kv_decode_workspace_bytes(_handles(sessions), len(sessions), layer, n_q_heads))


def kv_attend_decode(sessions, layer: int, q, sm_scale: float, out=None, workspace=None, stream=None):
    """q: device [n_sessions, n_q_heads, head_dim]; returns out (fp32, same shape)."""
    torch = _torch()
    _, hkv, d, _ = _sessions_shape(sessions)
    _check_q(q, len(sessions), "the number of sessions", d, hkv)
    n_s, hq, d = q.shape
    if out is None:
        out = torch.empty((n_s, hq, d), dtype=torch.float32, device=q.device)
    _expect_f32(out, q.shape, "out")
    _same_device(out, q, "out")
    if workspace is None:
        nb = kv_decode_workspace_bytes(sessions, layer, hq)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    _same_device(workspace, q, "workspace")
    _check(lib().kv_attend_decode(_handles(sessions), len(sessions), layer, _dev_ptr(q, "q"), _dtype_code(q),
                                  hq, float(sm_scale), _dev_ptr(out, "out"), _dev_ptr(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def kv_attend_decode_static(sessions, layer: int, q, sm_scale: float, out, stream=None):
    """kv_attend_decode with the library's static device scratch for the split partials: no
    allocation anywhere, so out (fp32, q's shape) must be supplied."""
    _, hkv, d, _ = _sessions_shape(sessions)
    _check_q(q, len(sessions), "the number of sessions", d, hkv)
    _expect_f32(out, q.shape, "out")
    _same_device(out, q, "out")
    _check(lib().kv_attend_decode_static(_handles(sessions), len(sessions), layer, _dev_ptr(q, "q"), _dtype_code(q),
                                         q.shape[1], float(sm_scale), _dev_ptr(out, "out"), _stream(stream)))
    return out


def kv_decode_launch_kind(sessions, layer: int, n_q_heads: int, q_dtype: int = KV_BF16, ws_bytes=None) -> int:
    """0: kv_attend_decode runs the split plan of kv_decode_plan; 1: the streamed launch.
    ws_bytes defaults to kv_decode_workspace_bytes (what kv_attend_decode allocates itself)."""
    if ws_bytes is None:
        ws_bytes = kv_decode_workspace_bytes(sessions, layer, n_q_heads)
    return _check(lib().kv_decode_launch_kind(_handles(sessions), len(sessions), layer, q_dtype, n_q_heads,
                                              int(ws_bytes)))


def kv_decode_plan(sessions, layer: int, n_q_heads: int):
    """(n_splits, tokens_per_split) that kv_attend_decode uses for these sessions."""
    n, t = C.c_int(), C.c_int64()
    _check(lib().kv_decode_plan(_handles(sessions), len(sessions), layer, n_q_heads, C.byref(n), C.byref(t)))
    return n.value, t.value


def kv_attend_decode_partial(sessions, layer: int, q, sm_scale: float, n_splits: int, tokens_per_split: int,
                             partials=None, stream=None):
    """First pass only; returns partials (fp32 [n_sessions, n_q_heads, n_splits, head_dim + 2])."""
    torch = _torch()
    _, hkv, d, _ = _sessions_shape(sessions)
    _check_q(q, len(sessions), "the number of sessions", d, hkv)
    n_s, hq, d = q.shape
    if partials is None:
        partials = torch.empty((n_s, hq, n_splits, d + 2), dtype=torch.float32, device=q.device)
    _expect_f32(partials, (n_s, hq, n_splits, d + 2), "partials")
    _same_device(partials, q, "partials")
    _check(lib().kv_attend_decode_partial(_handles(sessions), len(sessions), layer, _dev_ptr(q, "q"),
                                          _dtype_code(q), hq, float(sm_scale), n_splits, tokens_per_split,
                                          _dev_ptr(partials, "partials"),
                                          partials.numel() * partials.element_size(), _stream(stream)))
    return partials


def kv_merge_partials(partials, out=None, stream=None):
    """partials: fp32 [..., n_splits, head_dim + 2]; returns out (fp32 [..., head_dim])."""
    torch = _torch()
    if partials.dtype != torch.float32 or partials.dim() < 2:
        raise ValueError("partials must be fp32 [..., n_splits, head_dim + 2]")
    n_splits, d = partials.shape[-2], partials.shape[-1] - 2
    lead = tuple(partials.shape[:-2])
    rows = 1
    for x in lead:
        rows *= x
    if out is None:
        out = torch.empty(lead + (d,), dtype=torch.float32, device=partials.device)
    _expect_f32(out, lead + (d,), "out")
    _same_device(out, partials, "out")
    _check(lib().kv_merge_partials(_dev_ptr(partials, "partials"), rows, n_splits, d, _dev_ptr(out, "out"),
                                   _stream(stream)))
    return out


def kv_chunk_plan(cache: int, layer: int, n_q_heads: int, n_new: int):
    """(n_splits, keys_per_split) that kv_attend_chunk uses."""
    n, t = C.c_int(), C.c_int64()
    _check(lib().kv_chunk_plan(cache, layer, n_q_heads, n_new, C.byref(n), C.byref(t)))
    return n.value, t.value


def kv_attend_chunk_partial(cache: int, layer: int, q, n_new: int, sm_scale: float, n_splits: int,
                            keys_per_split: int, partials=None, stream=None):
    """First pass only; returns partials (fp32 [n_new, n_q_heads, n_splits, head_dim + 2])."""
    torch = _torch()
    _, hkv, d, _ = _cache_shape(cache)
    _check_q(q, n_new, "n_new", d, hkv)
    n, hq, d = q.shape
    if partials is None:
        partials = torch.empty((n, hq, n_splits, d + 2), dtype=torch.float32, device=q.device)
    _expect_f32(partials, (n, hq, n_splits, d + 2), "partials")
    _same_device(partials, q, "partials")
    _check(lib().kv_attend_chunk_partial(cache, layer, _dev_ptr(q, "q"), _dtype_code(q), hq, n_new,
                                         float(sm_scale), n_splits, keys_per_split, _dev_ptr(partials, "partials"),
                                         partials.numel() * partials.element_size(), _stream(stream)))
    return partials


def kv_chunk_workspace_bytes(cache: int, layer: int, n_q_heads: int, n_new: int) -> int:
    return _check(lib().kv_chunk_workspace_bytes(cache, layer, n_q_heads, n_new))


def kv_attend_chunk(cache: int, layer: int, q, n_new: int, sm_scale: float, out=None, workspace=None,
                    stream=None):
    """q: device [n_new, n_q_heads, head_dim]; returns out (fp32, same shape)."""
    torch = _torch()
    _, hkv, d, _ = _cache_shape(cache)
    _check_q(q, n_new, "n_new", d, hkv)
    n, hq, d = q.shape
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    _expect_f32(out, q.shape, "out")
    _same_device(out, q, "out")
    if workspace is None:
        nb = kv_chunk_workspace_bytes(cache, layer, hq, n_new)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    _same_device(workspace, q, "workspace")
    _check(lib().kv_attend_chunk(cache, layer, _dev_ptr(q, "q"), _dtype_code(q), hq, n_new, float(sm_scale),
                                 _dev_ptr(out, "out"), _dev_ptr(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def kv_footprint_bytes(cache: int) -> int:
    return _check(lib().kv_footprint_bytes(cache))


def kv_layout_footprint_bytes(layout, n_layers: int, n_kv_heads: int, head_dim: int, max_tokens: int) -> int:
    if isinstance(layout, str):
        layout = LAYOUT_IDS[layout]
    return _check(lib().kv_layout_footprint_bytes(int(layout), n_layers, n_kv_heads, head_dim, max_tokens))


def kv_cache_len(cache: int, layer: int) -> int:
    return _check(lib().kv_cache_len(cache, layer))


def kv_cache_reset(cache: int) -> None:
    _check(lib().kv_cache_reset(cache))


def kv_cache_truncate(cache: int, layer: int, new_len: int) -> None:
    _check(lib().kv_cache_truncate(cache, layer, new_len))


def kv_cache_plane(cache: int, layer: int, kv_head: int, plane: int):
    """(device address, row bytes) of one plane."""
    p, rb = C.c_void_p(), C.c_int64()
    _check(lib().kv_cache_plane(cache, layer, kv_head, plane, C.byref(p), C.byref(rb)))
    return (p.value or 0), rb.value


def kv_cache_copy_plane(cache: int, layer: int, kv_head: int, plane: int, row0: int, n_rows: int, dst,
                        stream=None):
    """Copy plane rows into the device uint8 tensor ``dst`` (n_rows * row_bytes bytes)."""
    _, rb = kv_cache_plane(cache, layer, kv_head, plane)
    if dst.numel() * dst.element_size() < n_rows * rb:
        raise ValueError(f"dst holds {dst.numel() * dst.element_size()} bytes, the rows need {n_rows * rb}")
    _check(lib().kv_cache_copy_plane(cache, layer, kv_head, plane, row0, n_rows, _dev_ptr(dst, "dst"),
                                     _stream(stream)))
    return dst


def kv_session_bytes(cache: int) -> int:
    return _check(lib().kv_session_bytes(cache))


def _host_ptr(buf, name: str) -> tuple[int, int]:
    """(address, bytes) of a host buffer: a CPU torch tensor (pinned or not) or a numpy array."""
    if hasattr(buf, "is_cuda"):
        if buf.is_cuda:
            raise ValueError(f"{name} must be host memory")
        if not buf.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return buf.data_ptr(), buf.numel() * buf.element_size()
    if not buf.flags["C_CONTIGUOUS"]:
        raise ValueError(f"{name} must be contiguous")
    return buf.ctypes.data, buf.nbytes


def kv_session_save(cache: int, dst, stream=None):
    """Write the session's saved form into the host buffer dst (uint8, >= kv_session_bytes)."""
    p, n = _host_ptr(dst, "dst")
    _check(lib().kv_session_save(cache, p, n, _stream(stream)))
    return dst


def kv_session_load(cache: int, src, stream=None) -> None:
    """Restore a saved session from the host buffer src into cache."""
    p, n = _host_ptr(src, "src")
    _check(lib().kv_session_load(cache, p, n, _stream(stream)))


def read_plane(cache: int, layer: int, kv_head: int, plane: int, row0: int, n_rows: int):
    """Host numpy copy [n_rows, row_bytes] of plane rows (synchronizes the stream)."""
    torch = _torch()
    _, rb = kv_cache_plane(cache, layer, kv_head, plane)
    buf = torch.empty((n_rows, rb), dtype=torch.uint8, device="cuda")
    if rb and n_rows:
        kv_cache_copy_plane(cache, layer, kv_head, plane, row0, n_rows, buf)
    return buf.cpu().numpy()

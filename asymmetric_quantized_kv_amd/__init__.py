"""Asymmetric quantized session KV cache for gfx950 (MI355X).

The compute path lives in ``libkvq.so`` (hand-written HIP kernels behind the C ABI
of ``include/kvq.h``); this package is its ctypes binding plus the seeded input
generators.  Importing the package does not load the library; the first call does.
"""
from ._lib import (  # noqa: F401
    KVError, LIB_PATH, LAYOUT_IDS,
    KV_OK, KV_EINVAL, KV_ECAPACITY, KV_ENOMEM, KV_EUNSUPPORTED, KV_EEMPTY, KV_EHIP,
    KV_FP16, KV_K8V8, KV_K8V4, KV_K4V8, KV_K4V4, KV_KF8V4, KV_F32, KV_BF16, KV_F16,
    KV_PLANE_KC, KV_PLANE_KS, KV_PLANE_VC, KV_PLANE_VS,
    lib, kv_cache_create, kv_cache_create_layered, kv_cache_layout, kv_cache_shape, kv_cache_check_guard, kv_layered_footprint_bytes,
    kv_cache_destroy, kv_append_quant, kv_attend_decode, kv_attend_decode_static,
    kv_decode_workspace_bytes, kv_decode_launch_kind, kv_decode_plan, kv_attend_decode_partial, kv_merge_partials,
    kv_attend_chunk, kv_chunk_workspace_bytes, kv_chunk_plan, kv_attend_chunk_partial, kv_footprint_bytes,
    kv_layout_footprint_bytes, kv_cache_len, kv_cache_reset, kv_cache_truncate, kv_cache_plane, kv_cache_copy_plane,
    kv_session_bytes, kv_session_save, kv_session_load, kv_last_error, kv_last_status, read_plane,
)

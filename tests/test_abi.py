"""The C ABI on the host: the library loads, exports every symbol include/kvq.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
from __future__ import annotations

import ctypes as C
import re
from pathlib import Path

import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import _lib

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "kvq.h"


@pytest.fixture(scope="session", autouse=True)
def built_library():
    if not _lib.LIB_PATH.exists():
        from asymmetric_quantized_kv_amd import build
        build.build(verbose=False)
    return kvq.lib()


def header_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_core_calls():
    names = header_functions()
    for n in ("kv_cache_create", "kv_append_quant", "kv_attend_decode", "kv_attend_chunk", "kv_footprint_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(built_library):
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(built_library, n), n
    assert set(names) <= set(_lib._SIGS), "binding misses a declared entry point"


@pytest.mark.parametrize("layout", range(6))
def test_layout_footprint_matches_oracle(layout):
    for L, hkv, d, t in [(22, 4, 64, 8192), (22, 4, 64, 128), (1, 8, 128, 100_500), (3, 5, 96, 1), (2, 1, 32, 257)]:
        assert kvq.kv_layout_footprint_bytes(layout, L, hkv, d, t) == O.layout_footprint_bytes(layout, L, hkv, d, t)


def test_layered_footprint_matches_oracle():
    for layouts in ([2], [0, 1, 2, 3, 4, 5], [1] * 11 + [4] * 11, [3, 0, 3]):
        for hkv, d, t in ((4, 64, 8192), (8, 128, 100_500), (3, 96, 1)):
            want = O.OracleLayeredCache(layouts, hkv, d, t).footprint_bytes()
            assert kvq.kv_layered_footprint_bytes(layouts, hkv, d, t) == want
    with pytest.raises(kvq.KVError):
        kvq.kv_layered_footprint_bytes([2, 9], 4, 64, 100)


@pytest.mark.parametrize("args,code", [
    ((7, 1, 4, 64, 100), kvq.KV_EINVAL),       # layout
    ((2, 0, 4, 64, 100), kvq.KV_EINVAL),       # n_layers
    ((2, 1, 0, 64, 100), kvq.KV_EINVAL),       # n_kv_heads
    ((2, 1, 4, 48, 100), kvq.KV_EINVAL),       # head_dim % 32
    ((2, 1, 4, 64, 0), kvq.KV_EINVAL),         # max_tokens
    ((2, 1, 4, 64, 1 << 31), kvq.KV_EINVAL),
    ((2, 1, 4, 96, 100), kvq.KV_EUNSUPPORTED), # valid but not built
])
def test_create_rejects_bad_shapes(args, code):
    with pytest.raises(kvq.KVError) as e:
        kvq.kv_cache_create(*args)
    assert e.value.code == code
    assert kvq.kv_last_status() == code and kvq.kv_last_error()


def test_forced_allocation_failure(monkeypatch):
    monkeypatch.setenv("KVQ_FAULT", "alloc")
    with pytest.raises(kvq.KVError) as e:
        kvq.kv_cache_create("K8V4", 1, 4, 64, 100)
    assert e.value.code == kvq.KV_ENOMEM and "KVQ_FAULT" in str(e.value)


def test_null_handles_are_rejected(built_library):
    L = built_library
    assert L.kv_append_quant(None, 0, None, None, 0, 1, None) == kvq.KV_EINVAL
    assert L.kv_attend_decode(None, 1, 0, None, 0, 4, 0.1, None, None, 0, None) == kvq.KV_EINVAL
    assert L.kv_attend_chunk(None, 0, None, 0, 4, 1, 0.1, None, None, 0, None) == kvq.KV_EINVAL
    assert L.kv_footprint_bytes(None) == kvq.KV_EINVAL
    n, t = C.c_int(), C.c_int64()
    assert L.kv_decode_plan(None, 1, 0, 4, C.byref(n), C.byref(t)) == kvq.KV_EINVAL
    assert L.kv_chunk_plan(None, 0, 4, 1, C.byref(n), C.byref(t)) == kvq.KV_EINVAL
    assert L.kv_attend_decode_partial(None, 1, 0, None, 0, 4, 0.1, 1, 512, None, 0, None) == kvq.KV_EINVAL
    assert L.kv_attend_chunk_partial(None, 0, None, 0, 4, 1, 0.1, 1, 64, None, 0, None) == kvq.KV_EINVAL
    assert L.kv_cache_layout(None, 0) == kvq.KV_EINVAL
    assert L.kv_cache_create_layered(None, 2, 4, 64, 100) is None and kvq.kv_last_status() == kvq.KV_EINVAL
    assert L.kv_session_bytes(None) == kvq.KV_EINVAL
    assert L.kv_session_save(None, None, 0, None) == kvq.KV_EINVAL
    assert L.kv_session_load(None, None, 0, None) == kvq.KV_EINVAL
    assert L.kv_cache_shape(None, None, None, None, None) == kvq.KV_EINVAL
    assert L.kv_cache_check_guard(None) == kvq.KV_EINVAL
    assert L.kv_attend_decode_static(None, 1, 0, None, 0, 4, 0.1, None, None) == kvq.KV_EINVAL


def test_merge_checks_arguments_on_the_host(built_library):
    L = built_library
    assert L.kv_merge_partials(None, 0, 1, 64, None, None) == kvq.KV_OK          # nothing to merge
    assert L.kv_merge_partials(None, 4, 1, 64, None, None) == kvq.KV_EINVAL      # null buffers
    assert L.kv_merge_partials(None, 4, 0, 64, None, None) == kvq.KV_EINVAL      # no split
    assert "n_splits" in kvq.kv_last_error()
    assert L.kv_merge_partials(None, -1, 1, 64, None, None) == kvq.KV_EINVAL     # negative rows
    assert L.kv_merge_partials(None, 4, 1, 0, None, None) == kvq.KV_EINVAL       # head_dim
    assert L.kv_merge_partials(C.c_void_p(8), 4, 1, 64, C.c_void_p(24), None) == kvq.KV_EINVAL  # misaligned
    assert "aligned" in kvq.kv_last_error()
    assert L.kv_cache_len(None, 0) == kvq.KV_EINVAL
    assert L.kv_cache_reset(None) == kvq.KV_EINVAL
    assert L.kv_cache_truncate(None, 0, 0) == kvq.KV_EINVAL
    assert L.kv_decode_workspace_bytes(None, 1, 0, 4) == kvq.KV_EINVAL
    assert L.kv_chunk_workspace_bytes(None, 0, 4, 1) == kvq.KV_EINVAL
    p, rb = C.c_void_p(), C.c_int64()
    assert L.kv_cache_plane(None, 0, 0, 0, C.byref(p), C.byref(rb)) == kvq.KV_EINVAL
    assert L.kv_cache_copy_plane(None, 0, 0, 0, 0, 1, None, None) == kvq.KV_EINVAL
    arr = (C.c_void_p * 2)(None, None)
    assert L.kv_attend_decode(arr, 2, 0, None, 0, 4, 0.1, None, None, 0, None) == kvq.KV_EINVAL
    assert "NULL" in kvq.kv_last_error()
    L.kv_cache_destroy(None)   # no-op


def test_status_is_cleared_by_a_good_call():
    with pytest.raises(kvq.KVError):
        kvq.kv_cache_create(9, 1, 1, 64, 1)
    assert kvq.kv_layout_footprint_bytes(2, 1, 1, 64, 1) > 0
    assert kvq.kv_last_status() == kvq.KV_OK and kvq.kv_last_error() == ""


def test_shapes_too_large_for_an_arena_are_rejected():
    """The footprint of an absurd shape is an error, never a wrapped-around int64."""
    for args in ((0, 1 << 20, 1 << 20, 128, 1 << 20), (0, 1, 1, 1 << 17, 100), (2, 1 << 30, 1 << 30, 64, 1 << 30)):
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_layout_footprint_bytes(*args)
        assert e.value.code == kvq.KV_EINVAL
    with pytest.raises(kvq.KVError):
        kvq.kv_layered_footprint_bytes([2] * 4096, 1 << 16, 128, 1 << 20)
    # the largest accepted head_dim still gives the exact formula (K8V4: D + D/16, D/2 + D/16)
    d = 65536
    assert kvq.kv_layout_footprint_bytes(2, 1, 1, d, 256) == 256 * (d + d // 16 + d // 2 + d // 16)


def test_header_compiles_as_c99_and_links(tmp_path, built_library):
    """include/kvq.h is a plain C interface: a C99 program that includes it builds with gcc,
    links against libkvq.so and runs its host-side calls."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_from_c"
    lib_dir = _lib.LIB_PATH.parent
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", str(ROOT / "include"),
                    str(ROOT / "tests" / "c" / "abi_from_c.c"), "-o", str(exe), "-L", str(lib_dir), "-lkvq",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


def test_binding_checks_tensors_against_the_cache(monkeypatch):
    """The binding rejects tensors whose shape, dtype or head_dim disagree with the cache before
    any pointer reaches the library (a mismatch would make the kernels read or write past an
    allocation).  The cache shape comes from kv_cache_shape; here it is stubbed, since creating a
    cache needs a GPU, and CPU tensors stand in (a well-formed call then stops at the device check)."""
    import torch
    monkeypatch.setattr(_lib, "_cache_shape", lambda cache: (1, 4, 128, 1000))
    f32, bf16 = torch.float32, torch.bfloat16

    def rejects(fn, *args, match, **kw):
        with pytest.raises((ValueError, TypeError)) as e:
            fn(*args, **kw)
        assert match in str(e.value), str(e.value)

    z = lambda *shape, dt=bf16: torch.zeros(shape, dtype=dt)
    # append: k, v [n_new, n_kv_heads, head_dim] of the cache
    rejects(kvq.kv_append_quant, 1, 0, z(5, 4, 64), z(5, 4, 64), match="[n_new, 4, 128]")
    rejects(kvq.kv_append_quant, 1, 0, z(5, 2, 128), z(5, 2, 128), match="[n_new, 4, 128]")
    rejects(kvq.kv_append_quant, 1, 0, z(5, 4, 128), z(5, 4, 128, dt=f32), match="one dtype")
    rejects(kvq.kv_append_quant, 1, 0, z(5, 4, 128, dt=torch.int32), z(5, 4, 128, dt=torch.int32), match="dtype")
    rejects(kvq.kv_append_quant, 1, 0, z(5, 4, 128), z(5, 4, 128), match="device tensor")   # shapes fine
    # decode: q [n_sessions, n_q_heads, head_dim], out fp32 of q's shape
    rejects(kvq.kv_attend_decode, [1], 0, z(1, 8, 64), 0.1, match="head_dim")
    rejects(kvq.kv_attend_decode, [1, 1], 0, z(1, 8, 128), 0.1, match="number of sessions")
    rejects(kvq.kv_attend_decode, [1], 0, z(1, 6, 128), 0.1, match="multiple of n_kv_heads")
    rejects(kvq.kv_attend_decode, [1], 0, z(1, 8, 128), 0.1, out=z(1, 8, 128), match="float32")
    rejects(kvq.kv_attend_decode, [1], 0, z(1, 8, 128), 0.1, out=z(1, 8, 64, dt=f32), match="shape")
    rejects(kvq.kv_attend_decode, [], 0, z(0, 8, 128), 0.1, match="session")
    rejects(kvq.kv_attend_decode_static, [1], 0, z(1, 8, 128), 0.1, z(1, 8, 128), match="float32")
    rejects(kvq.kv_attend_decode_static, [1], 0, z(1, 8, 128), 0.1, z(1, 8, 128, dt=f32), match="device tensor")
    rejects(kvq.kv_attend_decode_partial, [1], 0, z(1, 8, 128), 0.1, 2, 512, partials=z(1, 8, 3, 130, dt=f32),
            match="shape")
    # chunk: q [n_new, n_q_heads, head_dim]
    rejects(kvq.kv_attend_chunk, 1, 0, z(3, 8, 128), 4, 0.1, match="n_new")
    rejects(kvq.kv_attend_chunk, 1, 0, z(4, 8, 96), 4, 0.1, match="head_dim")
    rejects(kvq.kv_attend_chunk, 1, 0, z(4, 8, 128), 4, 0.1, out=z(4, 8, 128, dt=torch.float16), match="float32")
    rejects(kvq.kv_attend_chunk_partial, 1, 0, z(4, 8, 128), 4, 0.1, 2, 64, partials=z(4, 8, 2, 128, dt=f32),
            match="shape")
    rejects(kvq.kv_attend_chunk, 1, 0, z(4, 8, 128), 4, 0.1, workspace=z(16, dt=torch.uint8), match="device tensor")
    # merge: out [..., head_dim] fp32
    rejects(kvq.kv_merge_partials, z(4, 3, 130, dt=f32), out=z(4, 129, dt=f32), match="shape")


def test_host_library_under_address_and_undefined_behavior_sanitizers(tmp_path):
    """The host half of libkvq (argument checks, shape and footprint arithmetic, planning) built
    with g++ -fsanitize=address,undefined, the kernel launchers replaced by failing stubs, and
    driven by tests/c/host_checks.c: every size, offset and status path it reaches must run clean."""
    import shutil
    import subprocess
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None:
        pytest.skip("no g++/gcc")
    rocm = Path("/opt/rocm")
    csrc = ROOT / "asymmetric_quantized_kv_amd" / "csrc"
    so = tmp_path / "libkvq_hostsan.so"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    subprocess.run([gxx, "-std=c++17", "-O1", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__", *san,
                    "-I", str(rocm / "include"), "-I", str(ROOT / "include"), "-I", str(csrc),
                    str(csrc / "kvq_host.cpp"), str(ROOT / "tests" / "c" / "device_stubs.cpp"),
                    "-o", str(so), "-L", str(rocm / "lib"), "-lamdhip64", f"-Wl,-rpath,{rocm / 'lib'}"],
                   check=True, capture_output=True)
    exe = tmp_path / "host_checks"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", *san, "-I", str(ROOT / "include"),
                    str(ROOT / "tests" / "c" / "host_checks.c"), "-o", str(exe), str(so), f"-Wl,-rpath,{tmp_path}"],
                   check=True, capture_output=True)
    env = dict(__import__("os").environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr[-3000:])

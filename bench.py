#!/usr/bin/env python3
"""Benchmark of the quantized session KV cache on one MI355X.

Metric: K8V4 decode KV-read GB/s (% of HBM peak) + chunk-append tokens/s at a
100K-token context.  One step is one pass of the whole hot path on synthetic,
seeded inputs already resident in HBM:
  * decode:  one query per session over 64 sessions x 32,768 cached tokens,
             Hq 32 / Hkv 8 / D 128, K8V4 (split-K partial kernel + merge);
  * turn:    a 500-token turn against a 100,000-token session, Hq 64 / Hkv 8 /
             D 128, K8V4: quantize-on-append of the 500 tokens + causal chunk
             attention (+ merge of context splits).  The session is rolled back to
             100,000 tokens (a host-side length update) before every turn.
`value` is the decode's cache bytes per second; the turn's tokens/s is reported
beside it.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak, published

DEC_S, DEC_T, DEC_HQ, DEC_HKV, D = 64, 32_768, 32, 8, 128
TURN_CTX, TURN_NEW, TURN_HQ, TURN_HKV = 100_000, 500, 64, 8
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
RAG_SETTLE = 40   # further calls of the ragged batch before its steady-state timing
ASYM_SESSIONS = (0, 21, 63)    # sessions of the batched decode whose errors the asymmetry table reports


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on host cores")
    ap.add_argument("--no-k4v8", action="store_true", help="skip the K4V8 decode on the identical inputs")
    ap.add_argument("--no-kf8v4", action="store_true", help="skip the fp8-key (KF8V4) decode and chunk")
    ap.add_argument("--no-rebuild", action="store_true", help="skip the 131,072-token full rebuild")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for HBM counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the device sources with comments and blank space removed, so that a
    comment edit does not count as a kernel change."""
    h = hashlib.sha256()
    for f in ("decode.hip", "chunk.hip", "append.hip", "merge.hip", "kvq_internal.h", "wave_ops.h",
              "buffer_ops.h", "merge_row.h"):
        text = (ROOT / "asymmetric_quantized_kv_amd" / "csrc" / f).read_text()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on these sources."""
    try:
        t = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("kernel_src_sha") != kernel_source_sha():
        return None
    return e.get("hbm_bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import asymmetric_quantized_kv_amd as kvq
    from asymmetric_quantized_kv_amd import inputs as I

    torch.cuda.set_device(0)
    kvq.lib()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16).contiguous()

    # ---- decode workload ---------------------------------------------------------
    layouts = ["K8V4"] + ([] if args.no_k4v8 else ["K4V8"]) + ([] if args.no_kf8v4 else ["KF8V4"])
    t0 = time.time()
    caches = {L: [kvq.kv_cache_create(L, 1, DEC_HKV, D, DEC_T) for _ in range(DEC_S)] for L in layouts}
    keep = {}                                    # host copies of the sessions the CPU baseline uses
    n_cpu_sessions = 0 if args.no_cpu_baseline else 8
    asym_host = {}                               # host copies of the sessions the error table uses
    for s in range(DEC_S):
        k, v = I.batch64x32k_session(s)
        kd, vd = to_dev(k), to_dev(v)
        for L in layouts:
            kvq.kv_append_quant(caches[L][s], 0, kd, vd)
        if s < n_cpu_sessions:
            keep[s] = (k, v)
        if s in ASYM_SESSIONS:
            asym_host[s] = (k, v)
        del kd, vd
    q_dec = to_dev(I.batch64x32k_queries())
    torch.cuda.synchronize()
    log(f"decode caches ready ({time.time() - t0:.1f} s)")
    dec_bytes = sum(kvq.kv_footprint_bytes(h) for h in caches["K8V4"])   # every row is cached
    sm = D ** -0.5
    out_dec = torch.empty((DEC_S, DEC_HQ, D), dtype=torch.float32, device=dev)
    ws_dec = torch.empty(max([16] + [kvq.kv_decode_workspace_bytes(caches[L], 0, DEC_HQ) for L in layouts]),
                         dtype=torch.uint8, device=dev)

    # ---- turn workload -------------------------------------------------------------
    turn_in = I.turn_100k_plus_500()
    h3 = kvq.kv_cache_create("K8V4", 1, TURN_HKV, D, TURN_CTX + TURN_NEW)
    kvq.kv_append_quant(h3, 0, to_dev(turn_in["k"][:TURN_CTX]), to_dev(turn_in["v"][:TURN_CTX]))
    k_new, v_new = to_dev(turn_in["k"][TURN_CTX:]), to_dev(turn_in["v"][TURN_CTX:])
    q_new = to_dev(turn_in["q"])
    out_turn = torch.empty((TURN_NEW, TURN_HQ, D), dtype=torch.float32, device=dev)
    # the workspace is sized after the append, for the length the chunk call sees
    kvq.kv_append_quant(h3, 0, k_new, v_new)
    ws_turn = torch.empty(max(16, kvq.kv_chunk_workspace_bytes(h3, 0, TURN_HQ, TURN_NEW)), dtype=torch.uint8,
                          device=dev)
    torch.cuda.synchronize()
    log(f"turn cache ready ({time.time() - t0:.1f} s)")

    # The library's own split plans; the two passes of each attention are called one by
    # one (kv_attend_*_partial, then kv_merge_partials) so that events between them time
    # the partial kernels alone.  A one-split plan is the one-call path (no merge).
    dec_plan = kvq.kv_decode_plan(caches["K8V4"], 0, DEC_HQ)
    turn_plan = kvq.kv_chunk_plan(h3, 0, TURN_HQ, TURN_NEW)
    log(f"plans: decode {dec_plan[0]} x {dec_plan[1]} tokens, chunk {turn_plan[0]} x {turn_plan[1]} keys")
    part_dec = torch.empty((DEC_S, DEC_HQ, dec_plan[0], D + 2), dtype=torch.float32, device=dev)
    part_turn = torch.empty((TURN_NEW, TURN_HQ, turn_plan[0], D + 2), dtype=torch.float32, device=dev)

    def decode_pass1():
        if dec_plan[0] == 1:
            kvq.kv_attend_decode(caches["K8V4"], 0, q_dec, sm, out=out_dec, workspace=ws_dec)
        else:
            kvq.kv_attend_decode_partial(caches["K8V4"], 0, q_dec, sm, dec_plan[0], dec_plan[1], partials=part_dec)

    def decode_pass2():
        if dec_plan[0] > 1:
            kvq.kv_merge_partials(part_dec, out=out_dec)

    def decode(L="K8V4"):
        if L != "K8V4":          # the one-call path under its own plan
            kvq.kv_attend_decode(caches[L], 0, q_dec, sm, out=out_dec, workspace=ws_dec)
            return
        decode_pass1()
        decode_pass2()

    def turn_append():
        kvq.kv_cache_truncate(h3, 0, TURN_CTX)
        kvq.kv_append_quant(h3, 0, k_new, v_new)

    def turn_pass1():
        if turn_plan[0] == 1:
            kvq.kv_attend_chunk(h3, 0, q_new, TURN_NEW, sm, out=out_turn, workspace=ws_turn)
        else:
            kvq.kv_attend_chunk_partial(h3, 0, q_new, TURN_NEW, sm, turn_plan[0], turn_plan[1], partials=part_turn)

    def turn_pass2():
        if turn_plan[0] > 1:
            kvq.kv_merge_partials(part_turn, out=out_turn)

    for _ in range(args.warmup):
        decode()
        turn_append()
        turn_pass1()
        turn_pass2()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        decode_pass1()
        ev[i][1].record(stream)
        decode_pass2()
        ev[i][2].record(stream)
        turn_append()
        ev[i][3].record(stream)
        turn_pass1()
        ev[i][4].record(stream)
        turn_pass2()
        ev[i][5].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    mean = lambda xs: sum(xs) / len(xs)
    seg = [mean([e[j].elapsed_time(e[j + 1]) for e in ev]) for j in range(5)]
    dec1_t, dec2_t, app_t, chk1_t, chk2_t = seg
    # a one-split plan launches no merge: the events around the empty second pass time nothing
    if dec_plan[0] == 1:
        dec2_t = 0.0
    if turn_plan[0] == 1:
        chk2_t = 0.0
    dec_t, chk_t = dec1_t + dec2_t, chk1_t + chk2_t
    dec_gbps = dec_bytes / (dec_t * 1e-3) / 1e9              # whole decode (both passes)
    dec1_gbps = dec_bytes / (dec1_t * 1e-3) / 1e9            # the partial kernel alone
    turn_tok_s = TURN_NEW / ((app_t + chk_t) * 1e-3)
    # causal pairs of the turn: query j (position TURN_CTX + j) sees TURN_CTX + j + 1 keys
    pairs = TURN_HQ * sum(TURN_CTX + j + 1 for j in range(TURN_NEW))
    chunk_flop = 4.0 * D * pairs
    chunk_tflops = chunk_flop / (chk1_t * 1e-3) / 1e12       # the chunk kernel alone
    log(f"decode {dec_t:.4f} ms = partial {dec1_t:.4f} + merge {dec2_t:.4f} ({dec_gbps:.1f} GB/s; "
        f"partial kernel {dec1_gbps:.1f} GB/s), append {app_t:.4f} ms, chunk {chk_t:.4f} ms = kernel "
        f"{chk1_t:.4f} ({chunk_tflops:.1f} TFLOP/s) + merge {chk2_t:.4f}, wall {wall_ms / args.steps:.3f} ms/step")

    extra = {}
    if "K4V8" in layouts:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.warmup):
            decode("K4V8")
        e0.record(stream)
        for _ in range(args.steps):
            decode("K4V8")
        e1.record(stream)
        torch.cuda.synchronize()
        t48 = e0.elapsed_time(e1) / args.steps
        extra["decode_k4v8_GBps"] = round(dec_bytes / (t48 * 1e-3) / 1e9, 1)
        extra["decode_k4v8_ms"] = round(t48, 4)

    if "KF8V4" in layouts:
        # fp8 keys (E4M3 codes, one exponent byte per 32-element block) with 4-bit values:
        # the same decode inputs, and the same turn on its own 100,500-token session
        f8_bytes = sum(kvq.kv_footprint_bytes(h) for h in caches["KF8V4"])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.warmup):
            decode("KF8V4")
        e0.record(stream)
        for _ in range(args.steps):
            decode("KF8V4")
        e1.record(stream)
        torch.cuda.synchronize()
        tf8 = e0.elapsed_time(e1) / args.steps
        hf = kvq.kv_cache_create("KF8V4", 1, TURN_HKV, D, TURN_CTX + TURN_NEW)
        kvq.kv_append_quant(hf, 0, to_dev(turn_in["k"]), to_dev(turn_in["v"]))
        f8_plan = kvq.kv_chunk_plan(hf, 0, TURN_HQ, TURN_NEW)
        part_f8 = torch.empty((TURN_NEW, TURN_HQ, f8_plan[0], D + 2), dtype=torch.float32, device=dev)

        def f8_pass1():
            if f8_plan[0] == 1:
                kvq.kv_attend_chunk(hf, 0, q_new, TURN_NEW, sm, out=out_turn, workspace=ws_turn)
            else:
                kvq.kv_attend_chunk_partial(hf, 0, q_new, TURN_NEW, sm, f8_plan[0], f8_plan[1], partials=part_f8)

        for _ in range(args.warmup):
            f8_pass1()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            f8_pass1()
        e1.record(stream)
        torch.cuda.synchronize()
        tcf8 = e0.elapsed_time(e1) / args.steps
        kvq.kv_cache_destroy(hf)
        del part_f8
        f8_tflops = chunk_flop / (tcf8 * 1e-3) / 1e12
        extra["kf8v4"] = {
            "workload": "the decode and turn workloads above with fp8 (E4M3, MX block exponent) keys and "
                        "4-bit values",
            "decode_cache_bytes": f8_bytes, "decode_ms": round(tf8, 4),
            "decode_GBps": round(f8_bytes / (tf8 * 1e-3) / 1e9, 1),
            "decode_hbm_frac": round(f8_bytes / (tf8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "chunk_kernel_ms": round(tcf8, 4), "chunk_plan": {"n_splits": f8_plan[0], "keys_per_split": f8_plan[1]},
            "chunk_TFLOPs": round(f8_tflops, 1), "chunk_mfma_frac": round(f8_tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic_decode": load_traffic("decode_kf8v4"), "traffic_chunk": load_traffic("chunk_kf8v4"),
        }
        log(f"KF8V4 decode {tf8:.4f} ms ({extra['kf8v4']['decode_GBps']} GB/s), chunk kernel {tcf8:.4f} ms "
            f"({f8_tflops:.1f} TFLOP/s, plan {f8_plan})")

    # error asymmetry (KVSplit page, "Assimetria entre key e value"): each layout's decode of the
    # batched-decode inputs (heavy-tailed key channels) against attention over the unquantized
    # inputs, on sampled sessions
    extra["asymmetry"] = asymmetry(kvq, torch, I, caches, q_dec, sm, out_dec, ws_dec, asym_host, layouts)
    log(f"asymmetry: {extra['asymmetry']}")

    # session offload / restore of the 100,500-token turn cache through pinned host memory
    # (host-link rate, PCIe included: context for a cache hit, not the metric)
    sess_bytes = kvq.kv_session_bytes(h3)
    host_buf = torch.empty(sess_bytes, dtype=torch.uint8, pin_memory=True)
    h3b = kvq.kv_cache_create("K8V4", 1, TURN_HKV, D, TURN_CTX + TURN_NEW)
    kvq.kv_session_save(h3, host_buf)
    kvq.kv_session_load(h3b, host_buf)
    torch.cuda.synchronize()
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    n_rep = 5
    ev_s[0].record(stream)
    for _ in range(n_rep):
        kvq.kv_session_save(h3, host_buf)
    ev_s[1].record(stream)
    for _ in range(n_rep):
        kvq.kv_session_load(h3b, host_buf)
    ev_s[2].record(stream)
    torch.cuda.synchronize()
    t_save, t_load = ev_s[0].elapsed_time(ev_s[1]) / n_rep, ev_s[1].elapsed_time(ev_s[2]) / n_rep
    extra["session_offload"] = {
        "workload": "K8V4 session of 100,500 tokens x 8 KV heads x D 128, pinned host buffer",
        "bytes": sess_bytes, "save_ms": round(t_save, 3), "load_ms": round(t_load, 3),
        "save_GBps": round(sess_bytes / (t_save * 1e-3) / 1e9, 1), "load_GBps": round(sess_bytes / (t_load * 1e-3) / 1e9, 1),
    }
    kvq.kv_cache_destroy(h3b)
    del host_buf
    log(f"session offload {sess_bytes / 1e6:.1f} MB: save {t_save:.3f} ms, load {t_load:.3f} ms")

    # The KVSplit page's table shape: 22 layers x 4 KV heads x 64 at 8192 tokens.  One decode
    # step is a call per layer (cache-resident: the whole cache fits the 256 MB MALL), timed
    # for each of the five layouts of the page's table and for a cache with a layout per layer
    # (K8V8 in the first 4 layers, K8V4 in the middle 14, K4V4 in the last 4).
    lay22_in = I.layers22_8192_tokens()
    k22 = [torch.from_numpy(lay22_in["k"][l]).to(dev) for l in range(22)]
    v22 = [torch.from_numpy(lay22_in["v"][l]).to(dev) for l in range(22)]
    q22 = torch.from_numpy(lay22_in["q"]).to(dev)
    per_layout = {}
    for name, lays in [(L, [L] * 22) for L in ("FP16", "K8V8", "K8V4", "K4V8", "K4V4")] + \
                      [("mixed", ["K8V8"] * 4 + ["K8V4"] * 14 + ["K4V4"] * 4)]:
        per_layout[name] = decode22(kvq, torch, dev, stream, lays, k22, v22, q22, args)
        log(f"22-layer decode step, {name}: {per_layout[name]['us_per_step']:.1f} us "
            f"({per_layout[name]['GBps_cache_resident']} GB/s)")
    extra["layered_decode"] = dict(per_layout["mixed"], workload="22 layers x 4 KV heads x D 64, 8192 tokens, "
                                   "Hq 32; K8V8 layers 0-3, K8V4 4-17, K4V4 18-21")
    extra["decode22_layouts"] = {
        "workload": "22 layers x 4 KV heads x D 64, Hq 32, 8192 cached tokens, one decode step (22 calls, HIP "
                    "graph replay); the KVSplit page's table shape, all five layouts",
        **{L: {k: per_layout[L][k] for k in ("footprint_MiB", "us_per_step", "GBps_cache_resident")}
           for L in ("FP16", "K8V8", "K8V4", "K4V8", "K4V4")},
    }
    del k22, v22, q22

    # ragged batch: the same 64 K8V4 sessions cut back to log-uniform lengths (512..32,768),
    # decoded with the library's plan (the caches are not used at full length afterwards)
    rag_lens = I.ragged_lengths(DEC_S, 512, DEC_T)
    for h, n in zip(caches["K8V4"], rag_lens):
        kvq.kv_cache_truncate(h, 0, int(n))
    rag_bytes = int(rag_lens.sum()) * DEC_HKV * 208
    rag_plan = kvq.kv_decode_plan(caches["K8V4"], 0, DEC_HQ)
    ws_rag = torch.empty(max(16, kvq.kv_decode_workspace_bytes(caches["K8V4"], 0, DEC_HQ)), dtype=torch.uint8,
                         device=dev)
    for _ in range(args.warmup):
        kvq.kv_attend_decode(caches["K8V4"], 0, q_dec, sm, out=out_dec, workspace=ws_rag)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rag_time():
        e0.record(stream)
        for _ in range(args.steps):
            kvq.kv_attend_decode(caches["K8V4"], 0, q_dec, sm, out=out_dec, workspace=ws_rag)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # the batch's first few dozen calls run slower than the steady state a serving loop sees:
    # both are reported, the steady state after RAG_SETTLE more calls
    t_rag_first = rag_time()
    for _ in range(RAG_SETTLE):
        kvq.kv_attend_decode(caches["K8V4"], 0, q_dec, sm, out=out_dec, workspace=ws_rag)
    t_rag = rag_time()
    extra["ragged_decode"] = {
        "workload": "64 K8V4 sessions, log-uniform lengths 512..32,768 (seeded), Hq 32 / Hkv 8 / D 128",
        "cache_bytes": rag_bytes, "ms": round(t_rag, 4), "GBps": round(rag_bytes / (t_rag * 1e-3) / 1e9, 1),
        "timing": f"{args.steps} calls after {args.warmup + args.steps + RAG_SETTLE} others (steady state)",
        "ms_first_calls": round(t_rag_first, 4), "GBps_first_calls": round(rag_bytes / (t_rag_first * 1e-3) / 1e9, 1),
        "hbm_frac": round(rag_bytes / (t_rag * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "plan": {"n_splits": rag_plan[0], "tokens_per_split": rag_plan[1]},
        "launch": ("streamed: the sessions' 512-token blocks cut into one range per resident workgroup of each KV "
                   "head (the split plan above is what it replaces; include/kvq.h, kv_attend_decode)"
                   if kvq.kv_decode_launch_kind(caches["K8V4"], 0, DEC_HQ, kvq.KV_BF16, ws_rag.numel()) == 1
                   else "the split plan above"),
    }
    log(f"ragged decode {t_rag:.4f} ms ({extra['ragged_decode']['GBps']} GB/s; first calls {t_rag_first:.4f} ms), "
        f"plan {rag_plan}")

    # the same session recomputed from scratch as one chunk (append 100,500 + causal attention
    # of all 100,500 positions) against the turn: what keeping the cache saves at this shape
    extra["reuse"] = reuse_recompute(kvq, torch, dev, stream, turn_in, q_new, app_t + chk_t, to_dev, args)
    log(f"reuse: turn {extra['reuse']['turn_ms']} ms, recompute {extra['reuse']['recompute_ms']} ms, "
        f"ratio {extra['reuse']['recompute_over_turn']}")
    extra["hbm_probe"] = hbm_probe(torch, dev, stream, dec_bytes)
    log(f"HBM probe: {extra['hbm_probe']}")

    if not args.no_rebuild:
        extra["full_rebuild"] = full_rebuild(args, kvq, I, torch, dev, stream, log_fn=log)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device-to-device copy done")

    cpu = None
    if n_cpu_sessions:
        cpu, extra["cpu_baseline_quantize"] = cpu_baseline(keep, sm)
        extra["cpu_baseline_chunk"] = cpu_baseline_chunk(turn_in, sm)

    record = {
        "metric": "K8V4 decode KV-read GB/s (% HBM peak) + chunk-append tokens/s at 100K ctx",
        "value": round(dec_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec_t + app_t + chk_t, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 dot (QK), f16 dot2 (PV), f16 MFMA (chunk); f32 accumulate",
        "data": "synthetic (seeded numpy; bf16 K/V/Q)",
        "config": {
            "workload": "decode: 64 sessions x 32,768 cached tokens, Hq 32 / Hkv 8 / D 128, K8V4, one bf16 query "
                        "per session; turn: 500 new tokens appended to a 100,000-token session then causal chunk "
                        "attention, Hq 64 / Hkv 8 / D 128, K8V4",
            "decode_cache_bytes": dec_bytes,
            "turn_causal_pairs": pairs,
        },
        "hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "chunk_append_tokens_per_s": round(turn_tok_s, 1),
        "decode_ms": round(dec_t, 4),
        "decode_partial_ms": round(dec1_t, 4),
        "decode_merge_ms": round(dec2_t, 4),
        "append_ms": round(app_t, 4),
        "chunk_ms": round(chk_t, 4),
        "chunk_kernel_ms": round(chk1_t, 4),
        "chunk_merge_ms": round(chk2_t, 4),
        "decode_plan": {"n_splits": dec_plan[0], "tokens_per_split": dec_plan[1]},
        "chunk_plan": {"n_splits": turn_plan[0], "keys_per_split": turn_plan[1]},
        "roofline": {
            "bound": "hbm", "kernel": "decode_kernel<8,4,128,4,16> ("
                                      + ("one split: normalized output" if dec_plan[0] == 1 else "split-K partial pass") + ")",
            "achieved": round(dec1_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dec1_gbps / HBM_PEAK_GBPS, 4), "traffic": load_traffic("decode_k8v4"),
        },
        "roofline_chunk": {
            "bound": "mfma", "kernel": "chunk_kernel<8,4,128> (bf16 queries)",
            "achieved": round(chunk_tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(chunk_tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": load_traffic("chunk_k8v4"),
        },
        "cpu_baseline": cpu,
        "kernel_src_sha": kernel_source_sha(),
    }
    record.update(extra)
    print(json.dumps(record), flush=True)


def asymmetry(kvq, torch, I, caches, q_dec, sm, out, ws, host, layouts):
    """Max and RMS error of each layout's decode, on the sessions in `host`, against attention
    over their unquantized (bf16) keys and values in fp64, and the K4V8 / K8V4 ratios."""
    import numpy as np
    q = I.batch64x32k_queries().astype(np.float64)
    g = DEC_HQ // DEC_HKV
    ref = {}
    for s, (k, v) in host.items():
        o = np.empty((DEC_HQ, D))
        for h in range(DEC_HKV):
            kh, vh = k[:, h, :].astype(np.float64), v[:, h, :].astype(np.float64)
            x = sm * (q[s, h * g:(h + 1) * g] @ kh.T)
            w = np.exp(x - x.max(axis=1, keepdims=True))
            o[h * g:(h + 1) * g] = (w @ vh) / w.sum(axis=1, keepdims=True)
        ref[s] = o
    res = {"workload": f"decode of sessions {', '.join(map(str, sorted(host)))} of the 64 x 32,768-token batch "
                       "(keys with log-normal per-channel scales), all 32 heads; error against softmax attention over "
                       "the unquantized bf16 K and V in fp64"}
    for L in layouts:
        kvq.kv_attend_decode(caches[L], 0, q_dec, sm, out=out, workspace=ws)
        got = out.cpu().numpy().astype(np.float64)
        e = np.concatenate([(got[s] - ref[s]).ravel() for s in sorted(host)])
        res[L] = {"max_abs": float(np.abs(e).max()), "rms": float(np.sqrt(np.mean(e ** 2)))}
    if "K8V4" in res and "K4V8" in res:
        res["K4V8_over_K8V4"] = {m: round(res["K4V8"][m] / res["K8V4"][m], 2) for m in ("max_abs", "rms")}
    return res


def reuse_recompute(kvq, torch, dev, stream, turn_in, q_new, turn_ms, to_dev, args):
    """The 100,500-token session rebuilt from nothing as one chunk: append all tokens, then causal
    attention of every position (queries synthetic, seeded; the turn's own 500 are the last rows)."""
    n = TURN_CTX + TURN_NEW
    h = kvq.kv_cache_create("K8V4", 1, TURN_HKV, D, n)
    kd, vd = to_dev(turn_in["k"]), to_dev(turn_in["v"])
    gen = torch.Generator(device=dev)
    gen.manual_seed(3_100_500)
    q = torch.randn((n, TURN_HQ, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q[TURN_CTX:] = q_new
    out = torch.empty((n, TURN_HQ, D), dtype=torch.float32, device=dev)
    kvq.kv_append_quant(h, 0, kd, vd)
    ws = torch.empty(max(16, kvq.kv_chunk_workspace_bytes(h, 0, TURN_HQ, n)), dtype=torch.uint8, device=dev)
    plan = kvq.kv_chunk_plan(h, 0, TURN_HQ, n)

    def recompute():
        kvq.kv_cache_reset(h)
        kvq.kv_append_quant(h, 0, kd, vd)
        kvq.kv_attend_chunk(h, 0, q, n, D ** -0.5, out=out, workspace=ws)

    recompute()
    torch.cuda.synchronize()
    reps = 2
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        recompute()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps
    flop = 4.0 * D * TURN_HQ * n * (n + 1) / 2
    kvq.kv_cache_destroy(h)
    del q, out, ws, kd, vd
    return {"workload": "the 100,000 + 500 session recomputed as one 100,500-token chunk (append + causal "
                        "attention of every position) vs the 500-token turn on the kept cache; Hq 64 / Hkv 8 / D 128, K8V4",
            "turn_ms": round(turn_ms, 4), "recompute_ms": round(t, 3), "recompute_over_turn": round(t / turn_ms, 1),
            "recompute_TFLOPs": round(flop / (t * 1e-3) / 1e12, 1), "recompute_chunk_plan":
                {"n_splits": plan[0], "keys_per_split": plan[1]}}


def hbm_probe(torch, dev, stream, nbytes):
    """Plain-PyTorch reads of a buffer the size of the batched decode's cache: a sum (read once)
    and a copy of half of it (read + write), for the practical HBM ceiling beside the decode."""
    x = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)
    half = x.numel() // 2
    y = torch.empty(half, dtype=torch.float32, device=dev)
    for _ in range(2):
        x.sum()
        y.copy_(x[:half])
    torch.cuda.synchronize()
    reps = 10
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(reps):
        x.sum()
    e[1].record(stream)
    for _ in range(reps):
        y.copy_(x[:half])
    e[2].record(stream)
    torch.cuda.synchronize()
    t_sum, t_copy = e[0].elapsed_time(e[1]) / reps, e[1].elapsed_time(e[2]) / reps
    del x, y
    return {"bytes": nbytes, "sum_ms": round(t_sum, 4), "sum_read_GBps": round(nbytes / (t_sum * 1e-3) / 1e9, 1),
            "copy_ms": round(t_copy, 4), "copy_read_plus_write_GBps": round(2 * half * 4 / (t_copy * 1e-3) / 1e9, 1)}


def decode22(kvq, torch, dev, stream, lays, k22, v22, q22, args):
    """One decode step over a 22-layer x 4 x 64 cache of 8192 tokens with layer l in layout
    lays[l]: 22 calls replayed from a HIP graph (the small launches are host-bound one by one),
    and the same 22 calls launched eagerly."""
    h = kvq.kv_cache_create_layered(lays, 4, 64, 8192)
    for l in range(22):
        kvq.kv_append_quant(h, l, k22[l], v22[l])
    out = torch.empty((1, 32, 64), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, max(kvq.kv_decode_workspace_bytes([h], l, 32) for l in range(22))),
                     dtype=torch.uint8, device=dev)

    def step():
        for l in range(22):
            kvq.kv_attend_decode([h], l, q22[l], 64 ** -0.5, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(graph, stream=cap_stream):
            step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / args.steps
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) / args.steps
    del graph
    nbytes = sum(8192 * 4 * (kvq.kv_layout_footprint_bytes(x, 1, 1, 64, 8192) // 8192) for x in lays)
    res = {"footprint_MiB": kvq.kv_footprint_bytes(h) / 2 ** 20, "cache_bytes_per_step": nbytes,
           "us_per_step": round(t * 1e3, 1), "GBps_cache_resident": round(nbytes / (t * 1e-3) / 1e9, 1),
           "timing": "HIP graph replay of the 22 per-layer calls", "us_per_step_eager_launches": round(t_eager * 1e3, 1)}
    kvq.kv_cache_destroy(h)
    return res


def full_rebuild(args, kvq, I, torch, dev, stream, log_fn):
    """A full cache miss: reset, then 131,072 tokens as 32 chunks of 4,096, each appended and
    attended causally (Hq 40 / Hkv 8 / D 128, bf16), K8V4 and the fp8-key layout on the same
    inputs.  Inputs are resident on the device before the timed region; the chunk workspace
    is sized for the largest split plan of the 32 calls."""
    n_chunks, chunk, hq, hkv = 32, 4096, 40, 8
    ks, vs, qs = [], [], []
    for c in range(n_chunks):
        k, v, q = I.rebuild131k_chunk(c)
        ks.append(torch.from_numpy(k).to(dev).to(torch.bfloat16))
        vs.append(torch.from_numpy(v).to(dev).to(torch.bfloat16))
        qs.append(torch.from_numpy(q).to(dev).to(torch.bfloat16))
        del k, v, q
    out = torch.empty((chunk, hq, D), dtype=torch.float32, device=dev)
    pairs = hq * sum(c * chunk * chunk + chunk * (chunk + 1) // 2 for c in range(n_chunks))
    flop = 4.0 * D * pairs
    res = {"workload": "reset + 32 x (append 4,096 tokens + causal chunk attention), 131,072 tokens, "
                       "Hq 40 / Hkv 8 / D 128, bf16 inputs", "visible_pairs": pairs}
    for L in ("K8V4",) + (() if args.no_kf8v4 else ("KF8V4",)):
        h = kvq.kv_cache_create(L, 1, hkv, D, n_chunks * chunk)
        ws_bytes = 16
        kvq.kv_cache_reset(h)
        for c in range(n_chunks):      # sizing pass (also the warm-up)
            kvq.kv_append_quant(h, 0, ks[c], vs[c])
            ws_bytes = max(ws_bytes, kvq.kv_chunk_workspace_bytes(h, 0, hq, chunk))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def rebuild():
            kvq.kv_cache_reset(h)
            for c in range(n_chunks):
                kvq.kv_append_quant(h, 0, ks[c], vs[c])
                kvq.kv_attend_chunk(h, 0, qs[c], chunk, D ** -0.5, out=out, workspace=ws)

        rebuild()
        torch.cuda.synchronize()
        if L == "K8V4":   # the 32 appends alone: quantize-on-append at 4,096 tokens per call
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            kvq.kv_cache_reset(h)
            ea.record(stream)
            for c in range(n_chunks):
                kvq.kv_append_quant(h, 0, ks[c], vs[c])
            eb.record(stream)
            torch.cuda.synchronize()
            t_eager = ea.elapsed_time(eb) / n_chunks
            # the same 32 calls replayed from a HIP graph: the kernel time without the
            # binding's per-call host work (eager calls issue slower than the kernels run)
            kvq.kv_cache_reset(h)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                with torch.cuda.graph(graph, stream=cap):
                    for c in range(n_chunks):
                        kvq.kv_append_quant(h, 0, ks[c], vs[c])
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            ea.record(stream)
            for _ in range(5):
                graph.replay()
            eb.record(stream)
            torch.cuda.synchronize()
            t_app = ea.elapsed_time(eb) / (5 * n_chunks)
            del graph
            io = chunk * hkv * (2 * D * 2 + kvq.kv_layout_footprint_bytes(L, 1, 1, D, 256) // 256)
            res["append_4096"] = {"layout": L, "us_per_call": round(t_app * 1e3, 2), "bytes_per_call": io,
                                  "GBps": round(io / (t_app * 1e-3) / 1e9, 1),
                                  "hbm_frac": round(io / (t_app * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                  "timing": "HIP graph replay of the 32 calls",
                                  "us_per_call_eager": round(t_eager * 1e3, 2)}
            log_fn(f"append of 4,096 tokens: {t_app * 1e3:.2f} us ({res['append_4096']['GBps']} GB/s in + out; "
                   f"{t_eager * 1e3:.2f} us per eager call)")
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            rebuild()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps
        kvq.kv_cache_destroy(h)
        del ws
        tf = flop / (t * 1e-3) / 1e12
        res[L] = {"ms": round(t, 2), "tokens_per_s": round(n_chunks * chunk / (t * 1e-3), 1),
                  "TFLOPs": round(tf, 1), "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
        log_fn(f"full rebuild {L}: {t:.2f} ms ({tf:.1f} TFLOP/s, {res[L]['tokens_per_s']:.0f} tokens/s)")
    del ks, vs, qs, out
    return res


def cpu_baseline(keep, sm):
    """The oracle's decode on 8 of the 64 sessions (full length, all heads), on host cores."""
    import numpy as np

    import oracle as O
    from asymmetric_quantized_kv_amd import inputs as I

    q = I.batch64x32k_queries()
    ocs = []
    q_spent, q_cpu0 = 0.0, time.process_time()
    for s in sorted(keep):
        k, v = keep[s]
        c = O.OracleCache(2, 1, DEC_HKV, D, DEC_T)
        t = time.perf_counter()
        c.append(0, k, v)                       # the oracle's quantize-on-append of the session
        q_spent += time.perf_counter() - t
        ocs.append(c)
    q_cpu = time.process_time() - q_cpu0
    n_tok = len(keep) * DEC_T
    quant = {"value": round(n_tok / q_spent, 1), "unit": "tokens/s", "cores": max(1, round(q_cpu / q_spent)),
             "kind": "oracle", "GBps_in": round(n_tok * DEC_HKV * 2 * D * 2 / q_spent / 1e9, 4),
             "sample": f"quantize-on-append (K8V4) of sessions 0-{len(keep) - 1} of the batched decode, {n_tok} tokens "
                       f"x 8 KV heads x D 128 of bf16 K and V, {q_spent:.1f} s"}
    sample_bytes = sum(c.footprint_bytes() for c in ocs)
    qs = q[:len(ocs)]
    reps, spent, cpu0 = 0, 0.0, time.process_time()
    while spent < 10.0 and reps < 20:
        t = time.perf_counter()
        O.attend_decode(ocs, 0, qs, sm)
        spent += time.perf_counter() - t
        reps += 1
    cpu_used = time.process_time() - cpu0
    gbps = sample_bytes * reps / spent / 1e9
    return ({"value": round(gbps, 4), "unit": "GB/s", "cores": max(1, round(cpu_used / spent)), "kind": "oracle",
             "sample": f"decode of sessions 0-{len(ocs) - 1} of 64 (all 8 KV heads, 32,768 tokens each), "
                       f"{reps} repetitions, {spent:.1f} s; quantization timed apart (cpu_baseline_quantize)",
             "affinity_cpus": len(os.sched_getaffinity(0))}, quant)


def cpu_baseline_chunk(turn_in, sm):
    """The oracle's chunk attention for 16 of the 500 new tokens (all 64 heads), on host cores."""
    import numpy as np

    import oracle as O

    c = O.OracleCache(2, 1, TURN_HKV, D, TURN_CTX + TURN_NEW)
    c.append(0, turn_in["k"], turn_in["v"])
    rows = np.linspace(0, TURN_NEW - 1, 16).astype(int)
    t, cpu0 = time.perf_counter(), time.process_time()
    O.attend_chunk(c, 0, turn_in["q"], TURN_NEW, sm, rows=rows)
    spent = time.perf_counter() - t
    cpu_used = time.process_time() - cpu0
    return {"value": round(len(rows) / spent, 2), "unit": "tokens/s", "cores": max(1, round(cpu_used / spent)),
            "kind": "oracle", "sample": f"{len(rows)} of the 500 new tokens x 64 heads at 100,000 cached tokens, "
                                        f"{spent:.1f} s; attention only"}


if __name__ == "__main__":
    main()

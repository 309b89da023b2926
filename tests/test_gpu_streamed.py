"""GPU parity of the streamed decode launch: uneven sessions in one fused call, their token
blocks laid end to end and cut into one range per resident workgroup of each KV head,
balanced by blocks plus a fixed cost per session part (a range may hold the tail of one
session and the head of the next; a long session spans many ranges and leaves a partial per
range, merged in the launch).

kv_attend_decode takes the streamed launch when its split plan would launch only the busy
splits of uneven sessions (more than one split, some session shorter than the split range),
one launch holds every session (at most 64), no cache is passed twice, the device's resident
workgroups per KV head number 2 to 128 (4 or 8 KV heads on 256 compute units) and the
workspace holds one partial per range a session spans (kv_decode_workspace_bytes always
does).  Each case below asserts, through kv_decode_launch_kind, that it takes that launch;
the oracle is the plain fp64 attention over its quantized cache.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import TOL, dev, log, max_err, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.lib()
    yield
    torch.cuda.synchronize()


def _streamed(sessions, hq, qdt="bf16"):
    """Whether kv_attend_decode takes the streamed launch here (with the workspace it
    allocates itself)."""
    return kvq.kv_decode_launch_kind(sessions, 0, hq, kvq.KV_BF16 if qdt == "bf16" else kvq.KV_F32) == 1


def _build(layout, lens, hkv, d, hq, seed, bf16):
    sessions, ocs = [], []
    for i, n in enumerate(lens):
        k, v, _ = I.workload_small(seed + i, n, hkv, d, hq, 1, bf16=bf16, n_outliers=4 if d >= 64 else 0)
        h = kvq.kv_cache_create(layout, 1, hkv, d, n)
        sessions.append(h)
        dt = "bf16" if bf16 else "f32"
        kvq.kv_append_quant(h, 0, dev(k, dt), dev(v, dt))
        oc = O.OracleCache(O.LAYOUT_IDS[layout], 1, hkv, d, n)
        oc.append(0, k, v)
        ocs.append(oc)
    return sessions, ocs


STREAM_CASES = [
    # layout, head_dim, n_kv_heads, group, query dtype, lengths
    ("K8V4", 128, 8, 4, "bf16", [9000, 5000, 2500, 1300, 700, 513, 512, 300, 100, 30, 2, 1]),
    ("K4V8", 128, 8, 4, "bf16", [7000, 4100, 1025, 64, 33]),
    ("K8V8", 64, 4, 8, "f32", [12000, 3000, 600, 1]),
    ("K4V4", 64, 4, 8, "bf16", [6000, 6000, 511, 129, 5]),
    ("FP16", 128, 4, 4, "f32", [8192, 1000, 17]),
    ("KF8V4", 128, 8, 4, "f32", [9000, 2100, 513, 3]),
    ("K8V4", 128, 4, 16, "bf16", [5000, 260]),
    ("K8V4", 64, 4, 2, "f32", [20000, 1500, 40, 1]),
]


@pytest.mark.parametrize("layout,d,hkv,g,qdt,lens", STREAM_CASES)
def test_streamed_decode_matches_oracle(layout, d, hkv, g, qdt, lens):
    """Every layout, head_dim 64 and 128, groups 2 to 16 and fp32 or bf16 queries, over
    lengths from 1 token to 20,000 (ranges that cut a session and ranges that hold several).
    The same call twice gives the same bits: the launch leaves its merge counters at zero for
    the next, and each merge sums its partials in range order."""
    torch = torch_mod()
    hq = hkv * g
    log(f"streamed {layout} D {d} Hkv {hkv} G {g} q {qdt} lens {lens}")
    sessions, ocs = _build(layout, lens, hkv, d, hq, 1200 + sum(lens) % 97, qdt == "bf16")
    try:
        assert _streamed(sessions, hq, qdt)
        q = I.normal((len(lens), hq, d), 1300 + d + g, 9)
        if qdt == "bf16":
            q = I.bf16_round(q)
        qd = dev(q, qdt)
        scale = d ** -0.5
        want = O.attend_decode(ocs, 0, q, scale)
        first = kvq.kv_attend_decode(sessions, 0, qd, scale)
        err = max_err(first, want)
        log(f"  err {err:.3e}")
        assert err <= TOL
        assert torch.equal(kvq.kv_attend_decode(sessions, 0, qd, scale), first)   # run to run
    finally:
        torch.cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)


def test_streamed_decode_64_sessions_log_uniform():
    """64 sessions of log-uniform lengths (the ragged-batch shape at a sixth of its lengths),
    Hq 32 / Hkv 8 / D 128, K8V4: against the oracle, over a NaN-filled workspace (no partial is
    read that the launch did not write), and through kv_attend_decode_static (its scratch
    holds this call's partials)."""
    torch = torch_mod()
    lens = [int(x) for x in I.ragged_lengths(64, 16, 5461, seed=11)]
    hkv, g, d = 8, 4, 128
    hq = hkv * g
    log(f"streamed 64 sessions, {sum(lens)} tokens")
    sessions, ocs = _build("K8V4", lens, hkv, d, hq, 1400, True)
    try:
        assert _streamed(sessions, hq)
        q = I.bf16_round(I.normal((64, hq, d), 1401, 9))
        qd = dev(q, "bf16")
        scale = d ** -0.5
        want = O.attend_decode(ocs, 0, q, scale)
        err = max_err(kvq.kv_attend_decode(sessions, 0, qd, scale), want)
        log(f"  one call err {err:.3e}")
        assert err <= TOL
        nb = kvq.kv_decode_workspace_bytes(sessions, 0, hq)
        ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=qd.device)   # every float NaN
        err = max_err(kvq.kv_attend_decode(sessions, 0, qd, scale, workspace=ws), want)
        log(f"  NaN-filled workspace err {err:.3e}")
        assert err <= TOL
        out = torch.empty((64, hq, d), dtype=torch.float32, device=qd.device)
        kvq.kv_attend_decode_static(sessions, 0, qd, scale, out=out)
        err = max_err(out, want)
        log(f"  static scratch err {err:.3e}")
        assert err <= TOL
    finally:
        torch.cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)


def test_streamed_decode_tracks_growing_sessions():
    """Decode steps of a batch whose sessions grow by one token per step (appends between the
    calls): every step's output matches the oracle, so the ranges follow the lengths."""
    torch = torch_mod()
    lens0 = [3000, 1200, 511, 40, 1]
    hkv, g, d = 4, 4, 128
    hq = hkv * g
    steps = 3
    sessions, ocs = [], []
    try:
        ks, vs = [], []
        for i, n in enumerate(lens0):
            k, v, _ = I.workload_small(1500 + i, n + steps, hkv, d, hq, 1, bf16=True)
            ks.append(k)
            vs.append(v)
            h = kvq.kv_cache_create("K8V4", 1, hkv, d, n + steps)
            sessions.append(h)
            kvq.kv_append_quant(h, 0, dev(k[:n], "bf16"), dev(v[:n], "bf16"))
            oc = O.OracleCache(O.LAYOUT_IDS["K8V4"], 1, hkv, d, n + steps)
            oc.append(0, k[:n], v[:n])
            ocs.append(oc)
        scale = d ** -0.5
        for step in range(steps):
            for i, n in enumerate(lens0):
                t = n + step
                kvq.kv_append_quant(sessions[i], 0, dev(ks[i][t:t + 1], "bf16"), dev(vs[i][t:t + 1], "bf16"))
                ocs[i].append(0, ks[i][t:t + 1], vs[i][t:t + 1])
            assert _streamed(sessions, hq)
            q = I.bf16_round(I.normal((len(lens0), hq, d), 1600 + step, 9))
            want = O.attend_decode(ocs, 0, q, scale)
            err = max_err(kvq.kv_attend_decode(sessions, 0, dev(q, "bf16"), scale), want)
            log(f"  step {step}: err {err:.3e}")
            assert err <= TOL
    finally:
        torch.cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)


def test_streamed_decode_random_batches():
    """Seeded random batches (2 to 64 sessions, log-uniform lengths from 1 to 6,000 tokens,
    4 or 8 KV heads, groups 2 to 8, a random layout), each against the oracle: the cut's
    corner cases (ranges inside one session, ranges over many, sessions of one block) come
    up in many combinations."""
    torch = torch_mod()
    rng = np.random.default_rng(4242)
    layouts = ["K8V4", "K4V8", "K8V8", "K4V4", "FP16", "KF8V4"]
    ran = 0
    for case in range(16):
        n = int(rng.integers(2, 65))
        lens = [int(x) for x in np.exp(rng.uniform(0, np.log(6000), n)).astype(np.int64).clip(1, 6000)]
        hkv = int(rng.choice([4, 8]))
        g = int(rng.choice([2, 4, 8]))
        layout = str(rng.choice(layouts))
        d = 64
        hq = hkv * g
        sessions, ocs = _build(layout, lens, hkv, d, hq, 1700 + 37 * case, True)
        try:
            if not _streamed(sessions, hq):
                log(f"  case {case}: split plan, skipped")
                continue
            q = I.bf16_round(I.normal((n, hq, d), 1800 + case, 9))
            want = O.attend_decode(ocs, 0, q, d ** -0.5)
            err = max_err(kvq.kv_attend_decode(sessions, 0, dev(q, "bf16"), d ** -0.5), want)
            log(f"  case {case}: {layout} Hkv {hkv} G {g}, {n} sessions, {sum(lens)} tokens: err {err:.3e}")
            assert err <= TOL
            ran += 1
        finally:
            torch.cuda.synchronize()
            for h in sessions:
                kvq.kv_cache_destroy(h)
    assert ran >= 10

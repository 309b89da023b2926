"""Seeded random sweep of the GPU path against the oracle (48 cases): layouts, head_dims, group sizes,
input dtypes, session lengths and turn sizes drawn at random (fixed seed), each case small
enough for the oracle to finish in well under a second.  Planes bit-exact; decode and chunk
outputs within 5e-3, through the one-call entry points and through the two passes with a
random split."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import TOL, assert_planes_equal, dev, host_inputs, log, max_err, torch_mod

pytestmark = pytest.mark.gpu

LAYOUTS = ["FP16", "K8V8", "K8V4", "K4V8", "K4V4", "KF8V4"]


def draw_cases(n: int, seed: int = 20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = LAYOUTS[i % len(LAYOUTS)]
        d = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        hkv = int(rng.integers(1, 4))
        dtype = str(rng.choice(["f32", "bf16", "f16"]))
        n_sess = int(rng.integers(1, 4))
        lens = [int(x) for x in np.exp(rng.uniform(0, np.log(3000), n_sess)).astype(int) + 1]
        n_new = int(rng.integers(1, min(lens[0], 300) + 1))
        cases.append((i, layout, d, g, hkv, dtype, lens, n_new))
    return cases


CASES = draw_cases(48)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-D{c[2]}-G{c[3]}-H{c[4]}-{c[5]}")
def test_random_case_matches_oracle(case):
    i, layout, d, g, hkv, dtype, lens, n_new = case
    log(f"random case {case}")
    torch = torch_mod()
    hq = hkv * g
    lid = O.LAYOUT_IDS[layout]
    sessions, ocs = [], []
    try:
        for si, n in enumerate(lens):
            k, v, _ = I.workload_small(3000 + 17 * i + si, n, hkv, d, hq, 1, bf16=(dtype == "bf16"), n_outliers=3)
            h = kvq.kv_cache_create(layout, 1, hkv, d, n + 7)
            sessions.append(h)
            oc = O.OracleCache(lid, 1, hkv, d, n + 7)
            cut = n // 3
            for a, b in ((0, cut), (cut, n)):      # two appends per session
                if b > a:
                    kvq.kv_append_quant(h, 0, dev(k[a:b], dtype), dev(v[a:b], dtype))
                    oc.append(0, host_inputs(k[a:b], dtype), host_inputs(v[a:b], dtype))
            ocs.append(oc)
        assert_planes_equal(sessions[0], ocs[0], 0)
        scale = d ** -0.5
        q = I.normal((len(lens), hq, d), 3100 + i)
        if dtype == "bf16":
            q = I.bf16_round(q)
        out = kvq.kv_attend_decode(sessions, 0, dev(q, dtype), scale)
        err_d = max_err(out, O.attend_decode(ocs, 0, host_inputs(q, dtype), scale))
        qc = I.normal((n_new, hq, d), 3200 + i)
        if dtype == "bf16":
            qc = I.bf16_round(qc)
        outc = kvq.kv_attend_chunk(sessions[0], 0, dev(qc, dtype), n_new, scale)
        err_c = max_err(outc, O.attend_chunk(ocs[0], 0, host_inputs(qc, dtype), n_new, scale))
        # the two passes with a split of the test's choosing
        rng = np.random.default_rng(4000 + i)
        longest = max(lens)
        per = 512 * int(rng.integers(1, max(1, -(-longest // 512)) + 1))
        parts = kvq.kv_attend_decode_partial(sessions, 0, dev(q, dtype), scale, -(-longest // per), per)
        err_p = max_err(kvq.kv_merge_partials(parts), O.attend_decode(ocs, 0, host_inputs(q, dtype), scale))
        kper = 64 * int(rng.integers(1, max(1, -(-lens[0] // 64)) + 1))
        cparts = kvq.kv_attend_chunk_partial(sessions[0], 0, dev(qc, dtype), n_new, scale, -(-lens[0] // kper), kper)
        err_cp = max_err(kvq.kv_merge_partials(cparts), O.attend_chunk(ocs[0], 0, host_inputs(qc, dtype), n_new, scale))
        log(f"  decode err {err_d:.3e}, chunk err {err_c:.3e}; two-pass {per}: {err_p:.3e}, {kper}: {err_cp:.3e}")
        assert err_d <= TOL and err_c <= TOL and err_p <= TOL and err_cp <= TOL
    finally:
        torch.cuda.synchronize()
        for h in sessions:
            kvq.kv_cache_destroy(h)

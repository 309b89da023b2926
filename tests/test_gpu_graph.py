"""The library's launches can be captured in a HIP graph: a captured append + chunk +
decode sequence, replayed several times with eager work and synchronizations between
the replays, reproduces the eager results every time."""
from __future__ import annotations

import pytest

import asymmetric_quantized_kv_amd as kvq
from asymmetric_quantized_kv_amd import inputs as I

from gpu_util import dev, log, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.lib()
    yield
    torch.cuda.synchronize()


def test_graph_replays_match_eager():
    log("graph capture and replay")
    torch = torch_mod()
    hkv, d, n_ctx, n_new = 4, 128, 3000, 70
    k, v, _ = I.workload_small(1100, n_ctx + n_new, hkv, d, 16, 1, bf16=True, n_outliers=4)
    q_new = dev(I.bf16_round(I.normal((n_new, 16, d), 1101)), "bf16")
    q_dec = dev(I.bf16_round(I.normal((2, 16, d), 1102)), "bf16")
    kd, vd = dev(k, "bf16"), dev(v, "bf16")
    h = kvq.kv_cache_create("K8V4", 1, hkv, d, n_ctx + n_new)
    h2 = kvq.kv_cache_create("K8V4", 1, hkv, d, n_ctx + n_new)
    try:
        kvq.kv_append_quant(h, 0, kd[:n_ctx], vd[:n_ctx])
        kvq.kv_append_quant(h2, 0, kd, vd)
        out_c = torch.empty((n_new, 16, d), dtype=torch.float32, device="cuda")
        out_d = torch.empty((2, 16, d), dtype=torch.float32, device="cuda")
        ws_c = torch.empty(max(16, kvq.kv_chunk_workspace_bytes(h, 0, 16, n_new)), dtype=torch.uint8, device="cuda")
        ws_d = torch.empty(max(16, kvq.kv_decode_workspace_bytes([h, h2], 0, 16)), dtype=torch.uint8, device="cuda")

        def turn():
            kvq.kv_cache_truncate(h, 0, n_ctx)        # host-side length: captured as of now
            kvq.kv_append_quant(h, 0, kd[n_ctx:], vd[n_ctx:])
            kvq.kv_attend_chunk(h, 0, q_new, n_new, d ** -0.5, out=out_c, workspace=ws_c)
            kvq.kv_attend_decode([h, h2], 0, q_dec, d ** -0.5, out=out_d, workspace=ws_d)

        turn()
        torch.cuda.synchronize()
        want_c, want_d = out_c.clone(), out_d.clone()
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            kvq.kv_cache_truncate(h, 0, n_ctx)
            with torch.cuda.graph(graph, stream=s):
                kvq.kv_append_quant(h, 0, kd[n_ctx:], vd[n_ctx:])
                kvq.kv_attend_chunk(h, 0, q_new, n_new, d ** -0.5, out=out_c, workspace=ws_c)
                kvq.kv_attend_decode([h, h2], 0, q_dec, d ** -0.5, out=out_d, workspace=ws_d)
        torch.cuda.synchronize()
        for rep in range(3):
            out_c.fill_(float("nan"))
            out_d.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_c, want_c) and torch.equal(out_d, want_d), rep
            turn()                                      # eager work between the replays
            torch.cuda.synchronize()
            assert torch.equal(out_c, want_c) and torch.equal(out_d, want_d), rep
        del graph
    finally:
        torch.cuda.synchronize()
        kvq.kv_cache_destroy(h)
        kvq.kv_cache_destroy(h2)

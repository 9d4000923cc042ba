"""The whole layer captured in a HIP graph (as the benchmark runs it) gives the
same results as eager launches, on every replay.

Between replays the inputs are rewritten by ordinary eager work and the
program synchronises; each replay is compared bit for bit with an eager run of
the same inputs (the kernels are deterministic).
"""
import pytest
import torch

import workloads
from helpers import announce, require_gpu

import top_expert_routing_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("name", ["olmoe_decode", "dsv2_decode_t64", "tiny", "qwen3_prefill", "gptoss_mixed"])
def test_graph_replays_match_eager(name):
    announce(f"graph {name}")
    wl = workloads.make(name, DEV)
    s = wl.spec
    stats_ids = torch.empty((1, s.T, s.k), dtype=torch.int32, device=DEV)
    layer = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, wl.w_gate, wl.w_up, wl.w_down,
                         n_shared=s.S, n_priority=s.n_priority, stats_layers=1, req_offsets=wl.req_offsets,
                         device=DEV, topk_ids=stats_ids[0])
    logits = wl.logits.clone()
    x = wl.x.clone()
    stream = torch.cuda.Stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()      # the default stream's set-up is done before `stream` uses its buffers
    with torch.cuda.stream(stream):
        layer.forward(logits, x, stats_ids, stats_stream=side)     # warm-up, allocates stats outputs
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        layer.forward(logits, x, stats_ids, stats_stream=side)
    torch.cuda.synchronize()

    def snapshot():
        out = {"y": layer.y.clone(), "ids": layer.topk_ids.clone(), "w": layer.topk_w.clone(),
               "h": layer.h_sorted.clone()}
        for k, v in layer.perm.items():
            out["perm_" + k] = v.clone()
        for k, v in layer.stats_out.items():
            out["stats_" + k] = v.clone()
        return out

    gen = torch.Generator(device=DEV)
    for rep in range(3):
        gen.manual_seed(100 + rep)
        # eager work between replays: new inputs written in place
        logits.copy_(wl.logits + 0.5 * torch.randn(logits.shape, device=DEV, generator=gen))
        x.copy_((wl.x.float() + 0.1 * torch.randn(x.shape, device=DEV, generator=gen)).to(x.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        with torch.cuda.stream(stream):
            layer.forward(logits, x, stats_ids, stats_stream=side)
        torch.cuda.synchronize()
        ref = snapshot()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs from eager"

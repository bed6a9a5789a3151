"""moe_forward captured in a HIP graph and replayed: every schedule carries
state from call to call in the workspace (the single-launch layer's hand-off
buffers and call counts, the decode top-k's arrival count, the streaming
queues and per-tile completion counts), and the library resets it with
kernels, never with memsets. Each replay, with eager calls on another input
on the same workspace between replays, must give the eager result bit for
bit. Layer: hidden 2048, intermediate 1024, 64 experts, top-6, so T = 1, 2
take the single launch, T = 17, 64 the fused streaming launch and T = 200
the grouped GEMMs."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
GR = synth.Workload("graph", T=2, H=2048, E=64, k=6, I=1024, V=5000, bias_sigma=0.05, seed=11)


@pytest.fixture(scope="module")
def gr():
    L = synth.make_layer(GR)
    return GR, mx.DeviceLayer.from_host(L, DEV), mx.config_of(GR)


@pytest.mark.parametrize("T", [1, 2, 17, 64, 200])
def test_graph_replays_match_eager(gr, T):
    wl, D, cfg = gr
    print(f"[graph T={T} schedule={mx.forward_schedule(cfg, T)}]", flush=True)
    ws = mx.Workspace(DEV)
    x = mx.bf16_from_numpy(synth.make_tokens(wl, rep=300 + T, T=T), DEV)
    x2 = mx.bf16_from_numpy(synth.make_tokens(wl, rep=600 + T, T=T), DEV)
    # eager results first (this also sizes the workspace before capture)
    ref = mx.forward(cfg, x, D, out_fp32=True, ws=ws).clone()
    ref2 = mx.forward(cfg, x2, D, out_fp32=True, ws=ws).clone()
    torch.cuda.synchronize()

    out_g = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            mx.forward(cfg, x, D, out_fp32=True, ws=ws, out=out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for i in range(3):
        out_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {i} differs from the eager call"
        o2 = mx.forward(cfg, x2, D, out_fp32=True, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref2), f"eager call after replay {i} differs"

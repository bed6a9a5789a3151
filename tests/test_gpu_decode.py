"""GPU parity of the decode schedules (T <= 64) against the CPU oracle on a
layer whose shapes take the branch-free kernels: hidden 1024 (the routed w13
block streams 2 super-steps per wave, the slim shared w13 block 1),
intermediate 512, 32 experts, top-6. T = 1 and 2 run the three-launch tiny
schedule (top-k inside the w13 blocks, w2 + shared w2 + combine in one
output-stationary launch); T = 3 .. 64 the five-launch schedule."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
DEC = synth.Workload("dec", T=2, H=1024, E=32, k=6, I=512, V=5000, bias_sigma=0.05)


@pytest.fixture(scope="module")
def dec():
    L = synth.make_layer(DEC)
    return DEC, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(DEC)


@pytest.mark.parametrize("T", [1, 2, 3, 17, 64])
def test_forward_decode_matches_oracle(dec, T):
    wl, L, D, cfg = dec
    print(f"[forward dec T={T}]", flush=True)
    xh = synth.make_tokens(wl, rep=T, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, D, out_fp32=False)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward dec T={T}")
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


def test_forward_decode_repeatable(dec):
    wl, L, D, cfg = dec
    xh = synth.make_tokens(wl, rep=99, T=1)
    x = mx.bf16_from_numpy(xh, DEV)
    a = mx.forward(cfg, x, D, out_fp32=True)
    b = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# hidden 2048 and intermediate 1024 (multiples of 1024): T = 3 .. 64 run both
# expert stages in one launch (k_stream_fused), the w2 units waiting on the
# per-tile counts of the w13 units
DEC2 = synth.Workload("dec2", T=2, H=2048, E=64, k=6, I=1024, V=5000, bias_sigma=0.05)


@pytest.fixture(scope="module")
def dec2():
    L = synth.make_layer(DEC2)
    return DEC2, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(DEC2)


@pytest.mark.parametrize("T", [3, 17, 64, 5])
def test_forward_fused_stages_match_oracle(dec2, T):
    """One workspace across the cases, so each call also checks that the
    previous one left the queue and tile counters ready."""
    wl, L, D, cfg = dec2
    print(f"[forward dec2 T={T}]", flush=True)
    assert mx.forward_schedule(cfg, T) == "decode"
    xh = synth.make_tokens(wl, rep=100 + T, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    again = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward dec2 T={T}")
    assert torch.equal(out, again)

"""GPU parity of the single-launch layer (T <= 2: router, shared expert,
top-k, routed w13, w2 and combine in one launch of one block per CU) against
the CPU oracle, on a layer of hidden 2048, intermediate 1024, 64 experts,
top-6 (grid of 128 blocks; blocks past the 64 experts only stream weights),
and on repeated and interleaved calls that share one workspace: the launch's
hand-off counters must be back at zero after every call."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
LAY = synth.Workload("lay", T=2, H=2048, E=64, k=6, I=1024, V=5000, bias_sigma=0.05, seed=7)


@pytest.fixture(scope="module")
def lay():
    L = synth.make_layer(LAY)
    return LAY, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(LAY)


def _check(wl, L, D, cfg, T, rep, ws=None):
    print(f"[single-launch {wl.name} T={T} rep={rep}]", flush=True)
    xh = synth.make_tokens(wl, rep=rep, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True, ws=ws)
    out_bf = mx.forward(cfg, x, D, out_fp32=False, ws=ws)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    e = assert_outputs_close(out.cpu().numpy(), ref, f"single-launch T={T} rep={rep}")
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))
    return out, e


@pytest.mark.parametrize("T", [1, 2])
def test_single_launch_schedule_taken(lay, T):
    wl, L, D, cfg = lay
    assert mx.forward_schedule(cfg, T) == "single"
    assert mx.forward_schedule(cfg, 3) == "decode"
    assert mx.forward_schedule(cfg, T, hash_layer=True) == "single"
    assert mx.forward_schedule(cfg, 3, hash_layer=True) == "decode"
    assert mx.forward_schedule(cfg, 65, hash_layer=True) == "large"


@pytest.mark.parametrize("T,rep", [(1, 0), (1, 1), (2, 0), (2, 1)])
def test_single_launch_matches_oracle(lay, T, rep):
    wl, L, D, cfg = lay
    _check(wl, L, D, cfg, T, rep)


def test_single_launch_logit_offset(lay):
    """Per-expert logit offsets (added before the softplus) shift the routing."""
    wl, L, D, cfg = lay
    off = synth.normal_f32(wl.seed, synth.S_OFFSET, 0, wl.E, 0.5)
    Lv = dataclasses.replace(L, logit_offset=off)
    Dv = dataclasses.replace(D, logit_offset=torch.from_numpy(off).to(DEV))
    _check(wl, Lv, Dv, cfg, 2, 3)


def test_single_launch_interleaved_calls(lay):
    """One workspace through T = 1, 2, 3 (the five-launch schedule), 1, 2
    again: every single-launch call must find its counters at zero, and
    repeating an input gives the same bits."""
    wl, L, D, cfg = lay
    ws = mx.Workspace(DEV)
    first = {}
    for i, T in enumerate([1, 2, 3, 1, 2, 2, 1]):
        xh = synth.make_tokens(wl, rep=40 + T, T=T)
        x = mx.bf16_from_numpy(xh, DEV)
        out = mx.forward(cfg, x, D, out_fp32=True, ws=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), f"call {i} (T={T}) returned non-finite values"
        if T in first:
            assert torch.equal(out, first[T]), f"call {i} (T={T}) differs from the first call with this input"
        else:
            first[T] = out.clone()
    for T in (1, 2):
        xh = synth.make_tokens(wl, rep=40 + T, T=T)
        _, ref = reference_rows(L, xh, np.arange(T, dtype=np.int32))
        assert_outputs_close(first[T].cpu().numpy(), ref, f"interleaved T={T}")


@pytest.fixture(scope="module")
def lay_stack():
    """Three layers of the same shape (hidden 2048, 64 experts: a grid of
    128 blocks, blocks past the experts only stream weights), the second
    routed by a token-id table."""
    wls = [dataclasses.replace(LAY, seed=31), dataclasses.replace(LAY, seed=32, hash_layer=True),
           dataclasses.replace(LAY, seed=33)]
    hosts = [synth.make_layer(wl) for wl in wls]
    return wls, hosts, [mx.DeviceLayer.from_host(L, DEV) for L in hosts]


@pytest.mark.parametrize("T", [1, 2])
def test_stack_of_single_launch_layers(lay_stack, T):
    """moe_forward_stack at T <= 2 runs up to eight single-launch layers in
    one launch, each handing its output rows to the next inside it: eleven
    layers (two launches) equal the layers called one by one bit for bit,
    the intermediate outputs left in act, twice in a row."""
    wls, hosts, devs = lay_stack
    cfg = mx.config_of(LAY)
    order = [l % 3 for l in range(11)]
    layers = [devs[l] for l in order]
    x = mx.bf16_from_numpy(synth.make_tokens(LAY, rep=70 + T, T=T), DEV)
    tids = torch.from_numpy(synth.make_token_ids(wls[1], rep=70 + T, T=T)).to(DEV)
    act = torch.empty(2, T, LAY.H, dtype=torch.bfloat16, device=DEV)
    print(f"[stack of single-launch layers T={T}]", flush=True)
    out = mx.forward_stack(cfg, x, layers, token_ids=tids, out_fp32=True, act=act)
    again = mx.forward_stack(cfg, x, layers, token_ids=tids, out_fp32=True)
    y, outs = x, []
    for i, l in enumerate(order):
        y = mx.forward(cfg, y, devs[l], token_ids=tids if wls[l].hash_layer else None,
                       out_fp32=i == len(order) - 1)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, outs[-1])
    assert torch.equal(again, out)
    assert torch.equal(act[(len(order) - 2) % 2], outs[-2])
    assert mx.device_flags() == set()

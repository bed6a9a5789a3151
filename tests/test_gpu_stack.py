"""GPU parity of a stack of MoE layers run back to back (moe_forward_stack):
the model's first layers route by the token-id table and the rest by the
learned router (page "DeepSeek-V4-Flash export design", section "Source
configuration"; page "deepseek-v4-mxfp4-int8 config.json", num_hidden_layers
43, num_hash_layers 3). Four full-shape layers (three hash-routed, one
learned), each with its own router, shared expert, table and expert order,
layer l + 1 reading layer l's bf16 output.

  * every layer on its own seeded tokens against the oracle (each layer's own
    router, table, shared expert and expert order);
  * the first two layers chained, against the oracle's own chain (its layer 1
    reads the bf16 rounding of its own layer 0). Without the normalisation and
    residual the model has between MoE layers, a chain amplifies the
    one-ulp bf16 differences of each layer's output (relative error ~1e-6
    after layer 0, ~4e-4 after layer 1, ~2e-3 after layer 2), so deeper
    chains are compared GPU to GPU:
  * the stack equals the same layers called one by one with moe_forward, bit
    for bit;
at T = 1 (single-launch layers) and T = 5 (streaming layers)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close, f32_to_bf16_bits

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"
N_LAYERS = 4


def _device_layer(base_dev, Lh):
    order = torch.from_numpy(Lh.extra["expert_order"]).to(DEV)
    pick = (lambda t: t.index_select(0, order)) if Lh.extra["layer"] else (lambda t: t)

    def d(a):
        return None if a is None else torch.from_numpy(a).to(DEV)
    return mx.DeviceLayer(d(Lh.gate_w), d(Lh.bias), None, pick(base_dev.w13_codes), pick(base_dev.w13_scales),
                          pick(base_dev.w2_codes), pick(base_dev.w2_scales), d(Lh.sh_w13), d(Lh.sh_w13_scale),
                          d(Lh.sh_w2), d(Lh.sh_w2_scale), d(Lh.tid2eid))


@pytest.fixture(scope="module")
def stack(full_layer):
    base, base_dev = full_layer
    print("[stack] building 4 layers", flush=True)
    host = [synth.make_stack_layer(base, l) for l in range(N_LAYERS)]
    dev = [_device_layer(base_dev, Lh) for Lh in host]
    torch.cuda.synchronize()
    return host, dev


def _inputs(wl, T, rep):
    xh = synth.make_tokens(wl, rep=rep, T=T)
    tids_h = synth.make_token_ids(synth.WORKLOADS["hash_t4096"], rep=rep, T=T)
    return xh, tids_h, mx.bf16_from_numpy(xh, DEV), torch.from_numpy(tids_h).to(DEV)


@pytest.mark.parametrize("T", [1, 5])
def test_each_stack_layer_matches_oracle(stack, T):
    host, dev = stack
    cfg = mx.config_of(host[0].wl)
    for l, (L, D) in enumerate(zip(host, dev)):
        xh, tids_h, x, tids = _inputs(L.wl, T, 520 + 10 * l + T)
        hsh = L.wl.hash_layer
        out = mx.forward(cfg, x, D, token_ids=tids if hsh else None, out_fp32=True)
        torch.cuda.synchronize()
        r = oracle.forward(L, xh, token_ids=tids_h if hsh else None)
        if not hsh:
            assert (r["gap"] >= 1e-5).all(), "near-tie: pick another seed"
        e = assert_outputs_close(out.cpu().numpy(), r["out"], f"stack layer {l} T={T}")
        print(f"[stack layer {l} T={T}] rel L2 {e['rel_l2']:.2e}", flush=True)


@pytest.mark.parametrize("T", [1, 5])
def test_stack_chain_matches_oracle_chain(stack, T):
    host, dev = stack
    cfg = mx.config_of(host[0].wl)
    xh, tids_h, x, tids = _inputs(host[0].wl, T, 500 + T)
    xo = xh
    for m in (1, 2):
        L = host[m - 1]
        r = oracle.forward(L, xo, token_ids=tids_h if L.wl.hash_layer else None)
        xo = f32_to_bf16_bits(r["out"].astype(np.float32))
        out = mx.forward_stack(cfg, x, dev[:m], token_ids=tids, out_fp32=True)
        out_bf = mx.forward_stack(cfg, x, dev[:m], token_ids=tids)
        torch.cuda.synchronize()
        e = assert_outputs_close(out.cpu().numpy(), r["out"], f"stack chain T={T} layer {m - 1}")
        print(f"[stack chain T={T}] layer {m - 1}: rel L2 {e['rel_l2']:.2e}", flush=True)
        assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("T", [1, 5])
def test_stack_equals_layer_by_layer(stack, T):
    host, dev = stack
    cfg = mx.config_of(host[0].wl)
    _, _, x, tids = _inputs(host[0].wl, T, 540 + T)
    out = mx.forward_stack(cfg, x, dev, token_ids=tids, out_fp32=True)
    y = x
    for l, D in enumerate(dev):
        last = l == len(dev) - 1
        y = mx.forward(cfg, y, D, token_ids=tids if host[l].wl.hash_layer else None, out_fp32=last)
    again = mx.forward_stack(cfg, x, dev, token_ids=tids, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, y)
    assert torch.equal(out, again)
    assert mx.device_flags() == set()


def test_stack_argument_checks(stack):
    host, dev = stack
    cfg = mx.config_of(host[0].wl)
    x = torch.zeros(1, host[0].wl.H, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mx.MoEError):  # hash layers need token ids
        mx.forward_stack(cfg, x, dev[:1])


@pytest.mark.parametrize("T", [1, 2])
def test_stack_ten_layers_equals_layer_by_layer(stack, T):
    """Ten layers (the four built ones in turn, hash and learned mixed) at
    T = 1, 2: one launch runs up to eight layers, handing each layer's output
    rows to the next inside the launch, so this crosses a launch boundary.
    Bit for bit against the layers called one by one, with every
    intermediate output left in act as documented."""
    host, dev = stack
    cfg = mx.config_of(host[0].wl)
    order = [l % N_LAYERS for l in range(10)]
    layers = [dev[l] for l in order]
    _, _, x, tids = _inputs(host[0].wl, T, 560 + T)
    act = torch.empty(2, T, host[0].wl.H, dtype=torch.bfloat16, device=DEV)
    out = mx.forward_stack(cfg, x, layers, token_ids=tids, out_fp32=True, act=act)
    y, outs = x, []
    for l, D in zip(order, layers):
        last = len(outs) == len(layers) - 1
        y = mx.forward(cfg, y, D, token_ids=tids if host[l].wl.hash_layer else None, out_fp32=last)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, outs[-1])
    assert torch.equal(act[(len(layers) - 2) % 2], outs[-2])
    assert torch.equal(act[(len(layers) - 3) % 2], outs[-3])
    assert mx.device_flags() == set()


def test_stack_interleaved_with_single_layers(stack):
    """Stack calls and single-layer calls on one workspace: the hand-off
    buffers' parity and counters stay in step whichever runs (the stack
    advances them by its layer count)."""
    host, dev = stack
    cfg = mx.config_of(host[0].wl)
    ws = mx.Workspace(torch.device(DEV))
    _, _, x, tids = _inputs(host[0].wl, 1, 580)
    first = mx.forward_stack(cfg, x, dev[:3], token_ids=tids, out_fp32=True, ws=ws)
    single = mx.forward(cfg, x, dev[3], out_fp32=True, ws=ws)
    second = mx.forward_stack(cfg, x, dev[:3], token_ids=tids, out_fp32=True, ws=ws)
    single2 = mx.forward(cfg, x, dev[3], out_fp32=True, ws=ws)
    third = mx.forward_stack(cfg, x, dev[:2], token_ids=tids, out_fp32=True, ws=ws)
    two = mx.forward_stack(cfg, x, dev[:2], token_ids=tids, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(first, second)
    assert torch.equal(single, single2)
    assert torch.equal(third, two)
    assert mx.device_flags() == set()

"""The largest accepted batch, T = 65536 tokens (393,216 slots), on the tiny
layer (hidden 256, 16 experts, top-6, intermediate 128): the router GEMM
over 512 token tiles, the multi-block permutation (bit-exact against the
oracle's stable sort), the grouped GEMMs over about 3,100 tiles. Routing
of every token against the oracle, outputs of 640 rows (the first and last
tokens, tokens whose slots sit in each expert's last, partial tile, and
uniform ones), and a second call repeats the bits."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
T = 65536


def test_forward_max_tokens():
    wl = synth.Workload("tiny_maxt", T=T, H=256, E=16, k=6, I=128, V=1000, bias_sigma=0.05, seed=3)
    L = synth.make_layer(wl)
    D = mx.DeviceLayer.from_host(L, DEV)
    cfg = mx.config_of(wl)
    assert mx.forward_schedule(cfg, T) == "large"
    print(f"[forward T={T}] gpu", flush=True)
    xh = synth.make_tokens(wl, rep=1, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    again = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    ids_h, w_h = ids.cpu().numpy(), w.cpu().numpy()

    print(f"[forward T={T}] routing of every token", flush=True)
    oi, ow, og, on = oracle.route(xh, L.gate_w, L.bias, L.logit_offset, k=wl.k)
    rt = compare_routing(ids_h, w_h, oi, ow, og, on)
    print(f"[forward T={T}] near-ties {rt['near_ties']} swapped {rt['swapped']}", flush=True)

    print(f"[forward T={T}] permutation", flush=True)
    offsets, sorted_slots, slot_pos = mx.permute(cfg, ids)
    oo, os_, op = oracle.permute(ids_h, wl.E)
    assert np.array_equal(offsets.cpu().numpy(), oo)
    assert np.array_equal(sorted_slots.cpu().numpy(), os_)
    assert np.array_equal(slot_pos.cpu().numpy(), op)

    rng = np.random.default_rng(7)
    picks = [np.arange(64), np.arange(T - 64, T)]
    flat = ids_h.ravel()
    for e in range(wl.E):  # tokens in expert e's last (partial) 128-position tile
        slots = np.nonzero(flat == e)[0]
        tail = slots[(len(slots) - 1) // 128 * 128:] // wl.k
        picks.append(rng.choice(tail, size=min(16, len(tail)), replace=False))
    rows = np.unique(np.concatenate(picks))
    rest = np.setdiff1d(np.arange(T), rows)
    rows = np.sort(np.concatenate([rows, rng.choice(rest, size=max(0, 640 - len(rows)), replace=False)]))
    rows = rows.astype(np.int32)
    print(f"[forward T={T}] oracle outputs for {len(rows)} rows", flush=True)
    _, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy()[rows], ref, f"forward T={T}")


def test_forward_two_router_slices():
    """20,000 tokens (157 token tiles): the learned router's GEMM splits K in
    two slices, the only batch sizes (16,257-32,640 tokens) where it does, and
    the top-k adds the two partial logits. Routing of every token against the
    oracle, outputs of 256 evenly spread rows, a second call repeats the bits."""
    T2 = 20000
    wl = synth.Workload("tiny_t20000", T=T2, H=256, E=16, k=6, I=128, V=1000, bias_sigma=0.05, seed=5)
    L = synth.make_layer(wl)
    D = mx.DeviceLayer.from_host(L, DEV)
    cfg = mx.config_of(wl)
    assert mx.forward_schedule(cfg, T2) == "large"
    print(f"[forward T={T2}] gpu", flush=True)
    xh = synth.make_tokens(wl, rep=2, T=T2)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    again = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    print(f"[forward T={T2}] routing of every token", flush=True)
    oi, ow, og, on = oracle.route(xh, L.gate_w, L.bias, L.logit_offset, k=wl.k)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), oi, ow, og, on)
    rows = np.unique(np.linspace(0, T2 - 1, 256).astype(np.int32))
    _, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy()[rows], ref, f"forward T={T2}")

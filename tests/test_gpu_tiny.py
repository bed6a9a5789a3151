"""GPU parity on the tiny layer (T=16, hidden 256, 16 experts, top-6,
intermediate 128) and ragged variants of it, through the C ABI, against the
CPU oracle. Also the edge cases: T=1, T crossing the one-launch router limit
(64) and the permutation block (1024 slots), all tokens on one expert,
empty experts, and bitwise determinism."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assert_outputs_close, compare_routing, reference_rows)

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"


@pytest.fixture(scope="module")
def tiny():
    wl = synth.WORKLOADS["tiny"]
    L = synth.make_layer(wl)
    return wl, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(wl)


def _x(wl, T, rep=0):
    xh = synth.make_tokens(wl, rep=rep, T=T)
    return xh, mx.bf16_from_numpy(xh, DEV)


@pytest.mark.parametrize("T", [1, 3, 16, 64, 65, 200, 1100])
def test_route_matches_oracle(tiny, T):
    wl, L, D, cfg = tiny
    print(f"[route tiny T={T}]", flush=True)
    xh, x = _x(wl, T, rep=T)
    ids, w = mx.route(cfg, x, D.gate_w, D.bias)
    torch.cuda.synchronize()
    oi, ow, og, on = oracle.route(xh, L.gate_w, L.bias, k=wl.k)
    r = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), oi, ow, og, on)
    assert r["swapped"] <= max(1, T // 100)


def test_route_with_offset(tiny):
    wl, L, D, cfg = tiny
    T = 100
    xh, x = _x(wl, T, rep=7)
    off_h = synth.normal_f32(0, synth.S_OFFSET, 0, wl.E, 0.5)
    ids, w = mx.route(cfg, x, D.gate_w, D.bias, torch.from_numpy(off_h).to(DEV))
    oi, ow, og, on = oracle.route(xh, L.gate_w, L.bias, off_h, k=wl.k)
    compare_routing(ids.cpu().numpy(), w.cpu().numpy(), oi, ow, og, on)


@pytest.mark.parametrize("T", [1, 16, 300])
def test_hash_route_matches_oracle(tiny, T):
    wl, L, D, cfg = tiny
    xh, x = _x(wl, T, rep=3)
    t2e_h = synth.tid2eid(0, synth.S_TID2EID, 0, wl.V, wl.E, wl.k)
    tid_h = synth.zipf_ids(0, synth.S_TIDS, 0, T, wl.V)
    ids, w = mx.hash_route(cfg, x, torch.from_numpy(tid_h).to(DEV), torch.from_numpy(t2e_h).to(DEV), D.gate_w)
    oi, ow = oracle.hash_route(xh, tid_h, t2e_h, L.gate_w)
    assert np.array_equal(ids.cpu().numpy(), oi)
    assert np.abs(w.cpu().numpy() - ow).max() <= 1e-5


def _ids_cases(E, k):
    rng = np.random.default_rng(0)
    cases = {}
    for T in (1, 5, 64, 65, 171, 1500):
        p = np.exp(rng.standard_normal(E) * 1.5)
        cases[f"skew{T}"] = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum())
                                      for _ in range(T)]).astype(np.int32)
    # every token on the same experts (the rest empty)
    cases["same"] = np.tile(np.arange(k, dtype=np.int32), (300, 1))
    return cases


@pytest.mark.parametrize("case", list(_ids_cases(16, 6)))
def test_permute_bit_exact(tiny, case):
    wl, L, D, cfg = tiny
    ids_h = _ids_cases(wl.E, wl.k)[case]
    offsets, sorted_slots, slot_pos = mx.permute(cfg, torch.from_numpy(ids_h).to(DEV))
    oo, os_, op = oracle.permute(ids_h, wl.E)
    assert np.array_equal(offsets.cpu().numpy(), oo)
    assert np.array_equal(sorted_slots.cpu().numpy(), os_)
    assert np.array_equal(slot_pos.cpu().numpy(), op)


@pytest.mark.parametrize("case", ["skew5", "skew65", "same"])
def test_expert_ffn_matches_oracle(tiny, case):
    wl, L, D, cfg = tiny
    ids_h = _ids_cases(wl.E, wl.k)[case]
    T = ids_h.shape[0]
    xh, x = _x(wl, T, rep=11)
    rng = np.random.default_rng(1)
    w_h = rng.uniform(0.05, 0.5, size=ids_h.shape).astype(np.float32)
    ids = torch.from_numpy(ids_h).to(DEV)
    offsets, sorted_slots, _ = mx.permute(cfg, ids)
    out = mx.expert_ffn(cfg, x, offsets, sorted_slots, torch.from_numpy(w_h).to(DEV), D.w13_codes, D.w13_scales,
                        D.w2_codes, D.w2_scales)
    ref = oracle.expert_ffn(xh, ids_h, w_h.astype(np.float64), L.w13_codes, L.w13_scales, L.w2_codes,
                            L.w2_scales)
    assert_outputs_close(out.cpu().numpy(), ref, f"expert_ffn {case}")


@pytest.mark.parametrize("T", [1, 16, 64, 65, 300])
def test_forward_matches_oracle(tiny, T):
    wl, L, D, cfg = tiny
    print(f"[forward tiny T={T}]", flush=True)
    xh, x = _x(wl, T, rep=100 + T)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, D, out_fp32=False)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward tiny T={T}")
    # the bf16 output is the round-to-nearest-even of the fp32 output
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


def test_forward_hash_matches_oracle(tiny):
    wl, L, D, cfg = tiny
    wlh = synth.Workload("tiny_hash", T=40, H=wl.H, E=wl.E, k=wl.k, I=wl.I, V=wl.V, hash_layer=True)
    Lh = synth.make_layer(wlh)
    Dh = mx.DeviceLayer.from_host(Lh, DEV)
    xh, x = _x(wlh, 40, rep=5)
    tid_h = synth.make_token_ids(wlh, rep=0)
    out, (ids, w) = mx.forward(cfg, x, Dh, token_ids=torch.from_numpy(tid_h).to(DEV), out_fp32=True,
                               return_routing=True)
    r = oracle.forward(Lh, xh, token_ids=tid_h)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.abs(w.cpu().numpy() - r["w"]).max() <= 1e-5
    assert_outputs_close(out.cpu().numpy(), r["out"], "forward tiny hash")


def test_forward_deterministic(tiny):
    wl, L, D, cfg = tiny
    xh, x = _x(wl, 64, rep=9)
    a = mx.forward(cfg, x, D, out_fp32=True)
    b = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_forward_empty_batch(tiny):
    wl, L, D, cfg = tiny
    x = torch.empty(0, wl.H, dtype=torch.bfloat16, device=DEV)
    out = mx.forward(cfg, x, D)
    assert out.shape == (0, wl.H)

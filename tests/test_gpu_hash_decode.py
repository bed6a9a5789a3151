"""GPU parity of hash-routed layers (the first three layers of the model take
their experts from a token-id table: page "DeepSeek-V4-Flash export design",
section "Source configuration"; page "Tidalluna/DeepSeek-V4-Flash-0731-Tina-
CQ4KM", section "Compatibility", item 2) at decode sizes, where they take the
single-launch and streaming schedules with the table row in place of the
top-k: ids bit-exact against the oracle, weights within 1e-5, outputs at the
usual bar; Zipf(1.1) token ids, so repeated tokens share their experts."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"

LAYH = synth.Workload("layh", T=2, H=2048, E=64, k=6, I=1024, V=5000, hash_layer=True, seed=21)
DEC2H = synth.Workload("dec2h", T=2, H=2048, E=64, k=6, I=1024, V=5000, hash_layer=True, seed=22)
DECH = synth.Workload("dech", T=2, H=1024, E=32, k=6, I=512, V=5000, hash_layer=True, seed=23)
_LAYERS = {}


def _layer(wl):
    if wl.name not in _LAYERS:
        L = synth.make_layer(wl)
        _LAYERS[wl.name] = (L, mx.DeviceLayer.from_host(L, DEV))
    return _LAYERS[wl.name]


def _check(wl, L, D, T, rep, schedule, ws=None):
    cfg = mx.config_of(wl)
    assert mx.forward_schedule(cfg, T, hash_layer=True) == schedule
    print(f"[hash {wl.name} T={T} {schedule}]", flush=True)
    xh = synth.make_tokens(wl, rep=rep, T=T)
    tid_h = synth.make_token_ids(wl, rep=rep, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    tids = torch.from_numpy(tid_h).to(DEV)
    out, (ids, w) = mx.forward(cfg, x, D, token_ids=tids, out_fp32=True, return_routing=True, ws=ws)
    out_bf = mx.forward(cfg, x, D, token_ids=tids, ws=ws)
    torch.cuda.synchronize()
    r = oracle.forward(L, xh, token_ids=tid_h)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.array_equal(r["ids"], L.tid2eid[tid_h])
    assert np.abs(w.cpu().numpy() - r["w"]).max() <= 1e-5
    e = assert_outputs_close(out.cpu().numpy(), r["out"], f"hash {wl.name} T={T}")
    print(f"[hash {wl.name} T={T}] rel L2 {e['rel_l2']:.2e} max abs/rms {e['max_abs'] / e['rms']:.2e}", flush=True)
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))
    return out


@pytest.mark.parametrize("T", [1, 2])
def test_hash_single_launch(T):
    L, D = _layer(LAYH)
    _check(LAYH, L, D, T, 300 + T, "single")


@pytest.mark.parametrize("T", [3, 17, 64])
def test_hash_decode_fused(T):
    L, D = _layer(DEC2H)
    _check(DEC2H, L, D, T, 310 + T, "decode")


@pytest.mark.parametrize("T", [1, 2, 17])
def test_hash_decode_two_launches(T):
    """hidden 1024 has no single-launch kernel: the hash layer takes the
    decode schedule even at one or two tokens."""
    L, D = _layer(DECH)
    _check(DECH, L, D, T, 320 + T, "decode")


def test_hash_full_shape(full_layer):
    """The full-shape layer with a hash table: T=1 in one launch, T=64 in the
    streaming schedule."""
    L, D = full_layer
    wl = dataclasses.replace(synth.WORKLOADS["hash_t4096"], name="hash_full_decode")
    t2e = synth.tid2eid(wl.seed, synth.S_TID2EID, 0, wl.V, wl.E, wl.k)
    Lh = dataclasses.replace(L, wl=wl, tid2eid=t2e)
    Dh = dataclasses.replace(D, tid2eid=torch.from_numpy(t2e).to(DEV))
    _check(wl, Lh, Dh, 1, 330, "single")
    _check(wl, Lh, Dh, 64, 331, "decode")


def test_hash_and_learned_interleaved():
    """One workspace through learned and hash calls of the single-launch
    kernel and the streaming schedule: each call leaves the hand-off state
    and the queue counters ready for the next."""
    L, D = _layer(LAYH)
    wl_l = dataclasses.replace(LAYH, name="layl", hash_layer=False, bias_sigma=0.05)
    ws = mx.Workspace(DEV)
    cfg = mx.config_of(LAYH)
    first = {}
    for i, (T, hsh) in enumerate([(1, True), (1, False), (2, True), (5, True), (2, False), (1, True), (5, True)]):
        xh = synth.make_tokens(LAYH, rep=340 + T, T=T)
        x = mx.bf16_from_numpy(xh, DEV)
        tids = torch.from_numpy(synth.make_token_ids(LAYH, rep=340 + T, T=T)).to(DEV) if hsh else None
        out = mx.forward(cfg, x, D, token_ids=tids, out_fp32=True, ws=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), (i, T, hsh)
        key = (T, hsh)
        if key in first:
            assert torch.equal(out, first[key]), f"call {i} {key} differs from the first"
        else:
            first[key] = out.clone()
    assert mx.device_flags() == set()

"""Indices that come from the caller are checked on the device: an
out-of-range hash-layer token id or table entry, an out-of-range expert id
given to moe_permute, and an inconsistent permutation given to
moe_expert_ffn are never used to index memory. The kernels substitute an
in-range value, write NaN weights for such a hash-layer token, and set a bit
of the device error flags, which moe_device_flags reads and clears. Valid
inputs leave the flags clear. (Every access stays in bounds by
construction: these are error paths, not faults.)"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"
TINY = synth.WORKLOADS["tiny"]
MIDH = synth.Workload("mid_hash", T=250, H=512, E=32, k=6, I=384, V=5000, hash_layer=True)


@pytest.fixture(scope="module")
def hashed():
    L = synth.make_layer(MIDH)
    return MIDH, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(MIDH)


def _x(wl, T, rep):
    return mx.bf16_from_numpy(synth.make_tokens(wl, rep=rep, T=T), DEV)


def test_valid_calls_leave_flags_clear(hashed):
    wl, L, D, cfg = hashed
    mx.device_flags(clear=True)
    tids = torch.from_numpy(synth.make_token_ids(wl, rep=0)).to(DEV)
    out = mx.forward(cfg, _x(wl, wl.T, 1), D, token_ids=tids, out_fp32=True)
    assert torch.isfinite(out).all()
    assert mx.device_flags() == set()


def test_hash_token_id_out_of_range(hashed):
    wl, L, D, cfg = hashed
    mx.device_flags(clear=True)
    T = 40
    tid_h = synth.make_token_ids(wl, rep=2, T=T)
    bad = [3, 17, 39]
    tid_h[3], tid_h[17], tid_h[39] = wl.V, -1, 2**31 - 1
    tids = torch.from_numpy(tid_h).to(DEV)
    ids, w = mx.hash_route(cfg, _x(wl, T, 2), tids, D.tid2eid, D.gate_w)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert ((ids >= 0) & (ids < wl.E)).all()
    good = np.setdiff1d(np.arange(T), bad)
    assert np.isnan(w[bad]).all() and np.isfinite(w[good]).all()
    assert np.array_equal(ids[good], L.tid2eid[tid_h[good]])
    assert mx.device_flags(clear=True) == {"token_id"}
    assert mx.device_flags() == set()
    # the whole layer: the bad tokens' outputs are NaN, the others finite
    out = mx.forward(cfg, _x(wl, 300, 3), D, token_ids=torch.from_numpy(
        np.concatenate([tid_h, synth.make_token_ids(wl, rep=4, T=260)])).to(DEV), out_fp32=True)
    o = out.cpu().numpy()
    assert np.isnan(o[bad]).all(axis=1).all()
    assert np.isfinite(o[np.setdiff1d(np.arange(300), bad)]).all()
    assert mx.device_flags(clear=True) == {"token_id"}


def test_hash_table_entry_out_of_range(hashed):
    wl, L, D, cfg = hashed
    mx.device_flags(clear=True)
    t2e = L.tid2eid.copy()
    t2e[7, 2] = wl.E
    t2e[9, 0] = -5
    T = 8
    tid_h = np.array([7, 1, 9, 2, 3, 7, 4, 5], np.int32)
    ids, w = mx.hash_route(cfg, _x(wl, T, 5), torch.from_numpy(tid_h).to(DEV), torch.from_numpy(t2e).to(DEV),
                           D.gate_w)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert ((ids >= 0) & (ids < wl.E)).all()
    assert np.isnan(w[[0, 2, 5]]).all() and np.isfinite(w[[1, 3, 4, 6, 7]]).all()
    assert mx.device_flags(clear=True) == {"table_entry"}


def test_permute_expert_id_out_of_range():
    cfg = mx.config_of(TINY)
    mx.device_flags(clear=True)
    rng = np.random.default_rng(3)
    for T in (5, 300):  # the decode-size and the multi-block permutation
        ids_h = np.stack([rng.choice(TINY.E, size=TINY.k, replace=False) for _ in range(T)]).astype(np.int32)
        ids_h[T // 2, 1] = TINY.E + 3
        ids_h[0, 0] = -2
        offsets, sorted_slots, slot_pos = mx.permute(cfg, torch.from_numpy(ids_h).to(DEV))
        torch.cuda.synchronize()
        o, s, sp = offsets.cpu().numpy(), sorted_slots.cpu().numpy(), slot_pos.cpu().numpy()
        # a valid permutation of the slots in which the bad ids count as expert 0
        fixed = np.where((ids_h >= 0) & (ids_h < TINY.E), ids_h, 0).ravel()
        assert o[-1] == T * TINY.k
        assert np.array_equal(s, np.argsort(fixed, kind="stable"))
        assert np.array_equal(sp[s], np.arange(T * TINY.k))
        assert mx.device_flags(clear=True) == {"expert_id"}


def test_expert_ffn_inconsistent_permutation():
    wl = TINY
    cfg = mx.config_of(wl)
    L = synth.make_layer(wl)
    D = mx.DeviceLayer.from_host(L, DEV)
    mx.device_flags(clear=True)
    for T in (5, 200):  # streaming and GEMM schedules
        n = T * wl.k
        x = _x(wl, T, 6)
        w = torch.full((T, wl.k), 0.25, dtype=torch.float32, device=DEV)
        offsets = torch.zeros(wl.E + 1, dtype=torch.int32, device=DEV)
        offsets[1:] = torch.arange(1, wl.E + 1, dtype=torch.int32) * 10**6  # past T*k
        sorted_slots = torch.arange(n, dtype=torch.int32, device=DEV)
        mx.expert_ffn(cfg, x, offsets, sorted_slots, w, D.w13_codes, D.w13_scales, D.w2_codes, D.w2_scales)
        torch.cuda.synchronize()
        assert mx.device_flags(clear=True) == {"permutation"}
        good = torch.zeros(wl.E + 1, dtype=torch.int32, device=DEV)
        good[-1] = n  # every slot on expert E-1
        bad_slots = sorted_slots.clone()
        bad_slots[n // 2] = n + 7
        bad_slots[1] = -1
        mx.expert_ffn(cfg, x, good, bad_slots, w, D.w13_codes, D.w13_scales, D.w2_codes, D.w2_scales)
        torch.cuda.synchronize()
        assert mx.device_flags(clear=True) == {"permutation"}

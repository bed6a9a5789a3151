"""GPU parity at the layer's real shapes (hidden 4096, 256 experts, top-6,
intermediate 2048, MXFP4 routed experts, int8 shared expert), through the C
ABI, in the same configuration the benchmark times:

  decode T=1   several fresh token batches, every row (and T=2)
  decode T=3, 17, 40, 64  router bias N(0, 0.05) (mild expert skew), every row
  prefill T=8192, per-expert logit offsets N(0, 0.5): routing of every token,
               outputs of sampled rows (tokens are independent)
  hash layer T=4096, Zipf(1.1) token ids: routing exact, sampled rows
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"


def _variant(L, D, wl):
    """Same expert weights, the workload's own router bias / offset / table."""
    bias = synth.normal_f32(wl.seed, synth.S_BIAS, 0, wl.E, wl.bias_sigma)
    off = synth.normal_f32(wl.seed, synth.S_OFFSET, 0, wl.E, wl.offset_sigma) if wl.offset_sigma > 0 else None
    t2e = synth.tid2eid(wl.seed, synth.S_TID2EID, 0, wl.V, wl.E, wl.k) if wl.hash_layer else None
    Lv = dataclasses.replace(L, wl=wl, bias=bias, logit_offset=off, tid2eid=t2e)
    Dv = dataclasses.replace(D, bias=torch.from_numpy(bias).to(DEV),
                             logit_offset=None if off is None else torch.from_numpy(off).to(DEV),
                             tid2eid=None if t2e is None else torch.from_numpy(t2e).to(DEV))
    return Lv, Dv


def _run(wl, Lv, Dv, rep, rows=None, check_all_routing=True):
    cfg = mx.config_of(wl)
    xh = synth.make_tokens(wl, rep=rep)
    x = mx.bf16_from_numpy(xh, DEV)
    tids_h = synth.make_token_ids(wl, rep=rep) if wl.hash_layer else None
    tids = None if tids_h is None else torch.from_numpy(tids_h).to(DEV)
    print(f"[{wl.name} rep={rep}] gpu forward", flush=True)
    out, (ids, w) = mx.forward(cfg, x, Dv, token_ids=tids, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, Dv, token_ids=tids)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    routing = None
    print(f"[{wl.name} rep={rep}] oracle routing", flush=True)
    if wl.hash_layer:
        oi, ow = oracle.hash_route(xh, tids_h, Lv.tid2eid, Lv.gate_w)
        assert np.array_equal(ids, oi)
        assert np.abs(w - ow).max() <= 1e-5
    else:
        oi, ow, og, on = oracle.route(xh, Lv.gate_w, Lv.bias, Lv.logit_offset, k=wl.k)
        routing = compare_routing(ids, w, oi, ow, og, on)
        print(f"[{wl.name}] near-ties {routing['near_ties']} swapped {routing['swapped']}", flush=True)
    rows = np.arange(wl.T, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    print(f"[{wl.name} rep={rep}] oracle outputs for {len(rows)} rows", flush=True)
    _, ref = reference_rows(Lv, xh, rows, token_ids=tids_h, routing=routing)
    got = out.cpu().numpy()[rows]
    e = assert_outputs_close(got, ref, f"{wl.name} rep={rep}")
    print(f"[{wl.name} rep={rep}] rel L2 {e['rel_l2']:.2e} max abs {e['max_abs']:.2e} rms {e['rms']:.2e}",
          flush=True)
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))
    return ids


@pytest.mark.parametrize("rep", [0, 1, 2])
def test_decode_t1_full(full_layer, rep):
    L, D = full_layer
    wl = synth.WORKLOADS["decode_t1"]
    assert mx.forward_schedule(mx.config_of(wl), 1) == "single"
    Lv, Dv = _variant(L, D, wl)
    _run(wl, Lv, Dv, rep)


def test_decode_t2_full(full_layer):
    """Two tokens: twelve slots and two shared columns in the one launch."""
    L, D = full_layer
    wl = dataclasses.replace(synth.WORKLOADS["decode_t1"], name="decode_t2", T=2)
    assert mx.forward_schedule(mx.config_of(wl), 2) == "single"
    Lv, Dv = _variant(L, D, wl)
    _run(wl, Lv, Dv, 5)


@pytest.mark.parametrize("T", [3, 17, 40])
def test_decode_mid_t_full(full_layer, T):
    """Decode batches between the single launch and 64 tokens at the full
    shape: the fused streaming launch with routed tiles of 1-6 positions and
    shared tiles of up to 16 tokens (T=3: one of 3; T=17: 16 and 1; T=40:
    16, 16 and 8), every token against the oracle."""
    L, D = full_layer
    wl = dataclasses.replace(synth.WORKLOADS["decode_t64"], name=f"decode_t{T}", T=T)
    assert mx.forward_schedule(mx.config_of(wl), T) == "decode"
    Lv, Dv = _variant(L, D, wl)
    _run(wl, Lv, Dv, T)


def test_decode_t64_full(full_layer):
    L, D = full_layer
    wl = synth.WORKLOADS["decode_t64"]
    Lv, Dv = _variant(L, D, wl)
    ids = _run(wl, Lv, Dv, 0)
    assert len(set(ids.ravel().tolist())) > 100


def _stratified_rows(ids, k, n, seed, tile=128, top=4, per=8):
    """Rows to compare at a large T: the first and last tokens, tokens whose
    slots sit in the last (partial) 128-position tile of the `top` most-loaded
    experts and in their first tile, then uniform random tokens up to n."""
    T = ids.shape[0]
    flat = ids.ravel()
    counts = np.bincount(flat, minlength=int(flat.max()) + 1)
    picks = [0, 1, T - 2, T - 1]
    rng = np.random.default_rng(seed)
    for e in np.argsort(-counts, kind="stable")[:top]:
        slots = np.nonzero(flat == e)[0]  # ascending slot order = sorted positions of expert e
        last0 = ((len(slots) - 1) // tile) * tile
        tail = slots[last0:] // k
        head = slots[:tile] // k
        picks += rng.choice(tail, size=min(per, len(tail)), replace=False).tolist()
        picks += rng.choice(head, size=min(per // 2, len(head)), replace=False).tolist()
    picks = np.unique(np.array(picks, np.int64))
    rest = np.setdiff1d(np.arange(T), picks)
    fill = rng.choice(rest, size=max(0, n - len(picks)), replace=False)
    return np.sort(np.concatenate([picks, fill])).astype(np.int32)


def _gpu_ids(wl, Dv, rep):
    cfg = mx.config_of(wl)
    x = mx.bf16_from_numpy(synth.make_tokens(wl, rep=rep), DEV)
    tids = torch.from_numpy(synth.make_token_ids(wl, rep=rep)).to(DEV) if wl.hash_layer else None
    _, (ids, _) = mx.forward(cfg, x, Dv, token_ids=tids, return_routing=True)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


def test_prefill_t8192_full_sampled(full_layer):
    """256 stratified rows, including the ragged last tiles of the most-loaded
    experts (the persistent GEMM's tile queue runs at this size)."""
    L, D = full_layer
    wl = synth.WORKLOADS["prefill_t8192"]
    Lv, Dv = _variant(L, D, wl)
    rows = _stratified_rows(_gpu_ids(wl, Dv, 0), wl.k, 256, seed=0)
    assert len(rows) >= 256
    ids = _run(wl, Lv, Dv, 0, rows=rows)
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts.max() > 2 * counts.mean()  # the offsets skew the loads


def test_hash_t4096_full_sampled(full_layer):
    L, D = full_layer
    wl = synth.WORKLOADS["hash_t4096"]
    Lv, Dv = _variant(L, D, wl)
    rows = _stratified_rows(_gpu_ids(wl, Dv, 0), wl.k, 128, seed=1)
    assert len(rows) >= 128
    _run(wl, Lv, Dv, 0, rows=rows)

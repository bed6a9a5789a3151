"""Other top-k and expert counts than the model's (k = 6 of 256): the
library accepts 1 <= top_k <= 8 and top_k <= E <= 256, and every schedule
(tiny fallback, decode streaming, grouped GEMMs) must route and combine
them like the oracle. Hidden 512 and intermediate 256, so that T = 1 and 3
take the three-launch fallback or the decode schedule, 17 and 64 the fused
streaming launch, and 65 and 300 the grouped GEMMs; learned and hash
routing, every token against the oracle, bf16 output equal to the rounded
fp32 one."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
CASES = [(1, 8), (2, 16), (3, 32), (4, 64), (5, 64), (7, 128), (8, 64), (8, 256)]  # (top_k, experts)
TS = [1, 3, 17, 64, 65, 300]
_layers = {}


def _layer(k, E, hash_layer=False):
    key = (k, E, hash_layer)
    if key not in _layers:
        wl = synth.Workload(f"k{k}e{E}{'h' if hash_layer else ''}", T=300, H=512, E=E, k=k, I=256, V=700,
                            bias_sigma=0.05, hash_layer=hash_layer, seed=k * 1000 + E)
        L = synth.make_layer(wl)
        _layers[key] = (wl, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(wl))
    return _layers[key]


@pytest.mark.parametrize("T", TS)
@pytest.mark.parametrize("k,E", CASES)
def test_forward_general_topk(k, E, T):
    wl, L, D, cfg = _layer(k, E)
    print(f"[forward k={k} E={E} T={T} schedule {mx.forward_schedule(cfg, T)}]", flush=True)
    xh = synth.make_tokens(wl, rep=T + 3, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, D, out_fp32=False)
    torch.cuda.synchronize()
    assert ids.shape == (T, k)
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward k={k} E={E} T={T}")
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("T", [1, 17, 300])
@pytest.mark.parametrize("k,E", [(1, 8), (8, 64)])
def test_forward_hash_general_topk(k, E, T):
    wl, L, D, cfg = _layer(k, E, hash_layer=True)
    print(f"[forward hash k={k} E={E} T={T}]", flush=True)
    xh = synth.make_tokens(wl, rep=T + 5, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    tid_h = synth.make_token_ids(wl, rep=T)[:T]
    out, (ids, w) = mx.forward(cfg, x, D, token_ids=torch.from_numpy(tid_h).to(DEV), out_fp32=True,
                               return_routing=True)
    torch.cuda.synchronize()
    r = oracle.forward(L, xh, token_ids=tid_h)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.abs(w.cpu().numpy() - r["w"]).max() <= 1e-5
    assert_outputs_close(out.cpu().numpy(), r["out"], f"forward hash k={k} E={E} T={T}")

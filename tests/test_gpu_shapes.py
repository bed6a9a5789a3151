"""Hidden and intermediate sizes away from the model's: multiples of 128 that
are not multiples of 256 or 1024 (the library accepts any multiple of 128 up
to 8192), and the largest accepted sizes.
They take the paths the model's shapes never take: the router fallback,
two-launch streaming passes with 3, 5 or 10 stages of 128 K-values, the
per-slot GEMV schedule above 64 tokens where the hidden size is not a
multiple of 256, and grouped GEMMs with odd stage counts and 3 or 5 N tiles.
Every token against the oracle, bf16 output equal to the rounded fp32 one."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
SHAPES = [(384, 640), (768, 640), (1280, 384)]  # (hidden, intermediate)
TS = [1, 2, 5, 17, 64, 65, 200]
_layers = {}


def _layer(H, I):
    if (H, I) not in _layers:
        wl = synth.Workload(f"h{H}i{I}", T=200, H=H, E=32, k=6, I=I, V=900, bias_sigma=0.05, seed=H + I)
        L = synth.make_layer(wl)
        _layers[(H, I)] = (wl, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(wl))
    return _layers[(H, I)]


@pytest.mark.parametrize("T", TS)
@pytest.mark.parametrize("H,I", SHAPES)
def test_forward_odd_shapes(H, I, T):
    wl, L, D, cfg = _layer(H, I)
    print(f"[forward H={H} I={I} T={T} schedule {mx.forward_schedule(cfg, T)}]", flush=True)
    xh = synth.make_tokens(wl, rep=T + 11, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, D, out_fp32=False)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward H={H} I={I} T={T}")
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


# The largest accepted sizes (8192) and one just below them that is not a
# multiple of 256: streaming units whose tile width is cut so that the
# tile's rows and 256 rows of scales fit a block's LDS, the tiny schedule
# only where its w2 launch fits (else the decode schedule), GEMMs with
# K = 8192. Top-2 of 8 experts keeps the oracle quick.
BIG = [((8192, 256), [1, 2, 5, 17, 64, 65, 130]), ((256, 8192), [1, 2, 5, 17, 64, 65, 130]),
       ((8064, 384), [1, 17, 65, 130]), ((8192, 8192), [1, 5, 17])]
_big = {}


def _big_layer(H, I):
    if (H, I) not in _big:
        wl = synth.Workload(f"big{H}x{I}", T=130, H=H, E=8, k=2, I=I, V=900, bias_sigma=0.05, seed=H + 3 * I)
        L = synth.make_layer(wl)
        _big.clear()  # one large layer on the device at a time
        _big[(H, I)] = (wl, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(wl))
    return _big[(H, I)]


@pytest.mark.parametrize("H,I,T", [(h, i, t) for (h, i), ts in BIG for t in ts])
def test_forward_largest_shapes(H, I, T):
    wl, L, D, cfg = _big_layer(H, I)
    print(f"[forward H={H} I={I} T={T} schedule {mx.forward_schedule(cfg, T)}]", flush=True)
    xh = synth.make_tokens(wl, rep=T + 13, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward H={H} I={I} T={T}")


# Hash layers above 64 tokens at hidden sizes that are not multiples of 512:
# the hash router's last row piece is partly past the hidden size on some
# lanes (those lanes read in-range addresses and add zero products); and at
# the largest hidden sizes (8064, 8192), where it requests one expert's row
# at a time. Ids bit-exact with the table, weights within 1e-5, every
# token's output against the oracle.
def _check_hash(wl, T):
    import dataclasses

    import oracle

    wlh = dataclasses.replace(wl, name=f"{wl.name}hash", hash_layer=True)
    Lh = synth.make_layer(wlh)
    Dh = mx.DeviceLayer.from_host(Lh, DEV)
    cfgh = mx.config_of(wlh)
    print(f"[hash H={wl.H} I={wl.I} T={T} schedule {mx.forward_schedule(cfgh, T, hash_layer=True)}]", flush=True)
    xh = synth.make_tokens(wlh, rep=T + 5, T=T)
    tid_h = synth.make_token_ids(wlh, rep=T + 5, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    tids = torch.from_numpy(tid_h).to(DEV)
    out, (ids, w) = mx.forward(cfgh, x, Dh, token_ids=tids, out_fp32=True, return_routing=True)
    torch.cuda.synchronize()
    r = oracle.forward(Lh, xh, token_ids=tid_h)
    assert np.array_equal(ids.cpu().numpy(), Lh.tid2eid[tid_h])
    assert np.array_equal(r["ids"], Lh.tid2eid[tid_h])
    assert np.abs(w.cpu().numpy() - r["w"]).max() <= 1e-5
    assert_outputs_close(out.cpu().numpy(), r["out"], f"hash H={wl.H} I={wl.I} T={T}")


@pytest.mark.parametrize("T", [65, 200])
@pytest.mark.parametrize("H,I", SHAPES)
def test_hash_odd_hidden(H, I, T):
    _check_hash(_layer(H, I)[0], T)


@pytest.mark.parametrize("T", [65, 130])
@pytest.mark.parametrize("H,I", [(8192, 256), (8064, 384)])
def test_hash_largest_hidden(H, I, T):
    wl = synth.Workload(f"bigh{H}x{I}", T=130, H=H, E=8, k=2, I=I, V=900, seed=H + 5 * I)
    _check_hash(wl, T)

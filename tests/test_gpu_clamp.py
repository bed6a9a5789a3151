"""GPU parity where the clamped SwiGLU actually clamps, in every schedule.

The layer's expert MLP is down(silu(min(gate, L)) * clamp(up, -L, L)) with
L = swiglu_limit = 10, on the routed experts and on the shared expert alike
(page "DeepSeek-V4-Flash-0731", section "Checked in its code", row "SwiGLU
feed-forward"; page "deepseek-v4-mxfp4-int8 config.json", key swiglu_limit).

With N(0,1) tokens and N(0, 0.02) weights the gate and up pre-activations
have a standard deviation of 0.02 * sqrt(H) (0.45 at hidden 512, 1.3 at
4096), so |g| > 10 never happens in the ordinary parity tests. Here every
token is multiplied by a power of two (exact in bf16) chosen per hidden size
so that the pre-activations spread to about +-10 to +-15. Each case first
proves, from g and u computed in numpy with the weights decoded through the
E2M1 table of the OCP MX specification, that at least 5 % of the routed and
of the shared pre-activations lie in each clamped region (g > L, g < -L,
|u| > L), then compares the layer with the oracle at the usual bar.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle_pins
import synth
from parity import (assert_outputs_close, bf16_bits_to_f64, compare_routing, f32_to_bf16_bits,
                    reference_rows)

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"
LIMIT = 10.0
MIN_FRAC = 0.05

LAY = synth.Workload("lay", T=2, H=2048, E=64, k=6, I=1024, V=5000, bias_sigma=0.05, seed=7)
DEC = synth.Workload("dec", T=2, H=1024, E=32, k=6, I=512, V=5000, bias_sigma=0.05)
DEC2 = synth.Workload("dec2", T=2, H=2048, E=64, k=6, I=1024, V=5000, bias_sigma=0.05)
MID = synth.Workload("mid", T=300, H=512, E=32, k=6, I=384, V=5000, bias_sigma=0.05)
MID_HASH = synth.Workload("mid_hash", T=250, H=512, E=32, k=6, I=384, V=5000, hash_layer=True)

# token scale per hidden size: the pre-activation sigma becomes about 10-15
SCALE = {512: 32.0, 1024: 16.0, 2048: 16.0, 4096: 8.0}

_LAYERS = {}


def _layer(wl):
    if wl.name not in _LAYERS:
        L = synth.make_layer(wl)
        _LAYERS[wl.name] = (L, mx.DeviceLayer.from_host(L, DEV))
    return _LAYERS[wl.name]


def _scaled_tokens(wl, T, rep):
    xh = synth.make_tokens(wl, rep=rep, T=T)
    xs = bf16_bits_to_f64(xh) * SCALE[wl.H]
    xb = f32_to_bf16_bits(xs.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(xb), xs), "scaling by a power of two must be exact in bf16"
    return xb


def _clamp_regions(L, xb, ids):
    """Fractions of routed and shared gate/up values beyond the clamps."""
    xd = bf16_bits_to_f64(xb)
    I = L.wl.I
    g_r, u_r = [], []
    for t in range(xd.shape[0]):
        for e in ids[t]:
            W = oracle_pins.decode_mxfp4_table(L.w13_codes[e], L.w13_scales[e])
            g_r.append(W[:I] @ xd[t])
            u_r.append(W[I:] @ xd[t])
    S13 = L.sh_w13.astype(np.float64) * L.sh_w13_scale.astype(np.float64)[:, None]
    g_s, u_s = xd @ S13[:I].T, xd @ S13[I:].T
    frac = {}
    for name, g, u in (("routed", np.concatenate(g_r), np.concatenate(u_r)), ("shared", g_s.ravel(), u_s.ravel())):
        frac[name] = dict(gate_hi=float(np.mean(g > LIMIT)), gate_lo=float(np.mean(g < -LIMIT)),
                          up=float(np.mean(np.abs(u) > LIMIT)))
    return frac


def _check(wl, T, rep, schedule, hash_layer=False):
    L, D = _layer(wl)
    cfg = mx.config_of(wl)
    assert mx.forward_schedule(cfg, T, hash_layer=hash_layer) == schedule
    print(f"[clamp {wl.name} T={T} {schedule}]", flush=True)
    xb = _scaled_tokens(wl, T, rep)
    x = mx.bf16_from_numpy(xb, DEV)
    tids_h = synth.make_token_ids(wl, rep=rep, T=T) if hash_layer else None
    tids = None if tids_h is None else torch.from_numpy(tids_h).to(DEV)
    out, (ids, w) = mx.forward(cfg, x, D, token_ids=tids, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, D, token_ids=tids)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xb, rows, token_ids=tids_h)
    if hash_layer:
        assert np.array_equal(ids.cpu().numpy(), r["ids"])
        assert np.abs(w.cpu().numpy() - r["w"]).max() <= 1e-5
    else:
        rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
        if rt["alt_rows"]:
            r, ref = reference_rows(L, xb, rows, routing=rt)
    frac = _clamp_regions(L, xb, r["ids"])
    print(f"[clamp {wl.name} T={T}] regions {frac}", flush=True)
    for side, f in frac.items():
        for region, v in f.items():
            assert v >= MIN_FRAC, f"{side} {region}: only {v:.3f} of the values are beyond the clamp"
    e = assert_outputs_close(out.cpu().numpy(), ref, f"clamp {wl.name} T={T}")
    print(f"[clamp {wl.name} T={T}] rel L2 {e['rel_l2']:.2e} max abs/rms {e['max_abs'] / e['rms']:.2e}",
          flush=True)
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("T", [1, 2])
def test_clamp_single_launch(T):
    _check(LAY, T, 200 + T, "single")


def test_clamp_single_launch_full_shape(full_layer):
    L, D = full_layer
    wl = synth.WORKLOADS["decode_t1"]
    _LAYERS[wl.name] = (L, D)
    _check(wl, 1, 201, "single")


def test_clamp_tiny_schedule():
    _check(DEC, 1, 202, "tiny")


def test_clamp_decode_fused():
    _check(DEC2, 17, 203, "decode")


def test_clamp_decode_two_launches():
    _check(DEC, 17, 204, "decode")


def test_clamp_large():
    _check(MID, 300, 205, "large")


def test_clamp_hash_large():
    _check(MID_HASH, 250, 206, "large", hash_layer=True)


DEC2_HASH = synth.Workload("dec2_hash", T=17, H=2048, E=64, k=6, I=1024, V=5000, hash_layer=True, seed=3)
LAY_HASH = synth.Workload("lay_hash", T=1, H=2048, E=64, k=6, I=1024, V=5000, hash_layer=True, seed=4)


def test_clamp_hash_decode():
    _check(DEC2_HASH, 17, 207, "decode", hash_layer=True)


def test_clamp_hash_single_launch():
    _check(LAY_HASH, 1, 208, "single", hash_layer=True)

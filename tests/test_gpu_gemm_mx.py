"""GPU parity of the block-scaled routed GEMMs (MXFP4 weights x activations
split exactly into hi/lo fp8 halves with E8M0 block exponents, on gfx950's
scaled MFMA; the option MOE_OPTION_PREFILL_BLOCK_SCALED) against the CPU
oracle: the large-batch schedule on a layer whose
shapes take that path (hidden 512: one 512-row w2 tile; intermediate 512: two
256-column w13 tiles; 32 experts, top-6). Ragged 64-position tiles, a skewed
and an all-on-six-experts expert FFN, the hash-routed layer, a batch whose
live tiles are several times the persistent grid (every row compared), and
inputs scaled so the SwiGLU clamps are hit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assert_outputs_close, bf16_bits_to_f64, compare_routing, f32_to_bf16_bits,
                    reference_rows)

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
MXL = synth.Workload("mxl", T=300, H=512, E=32, k=6, I=512, V=5000, bias_sigma=0.05, seed=11)


@pytest.fixture(scope="module")
def mxl():
    prev = mx.set_option("prefill_block_scaled", 1)
    L = synth.make_layer(MXL)
    yield MXL, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(MXL)
    mx.set_option("prefill_block_scaled", prev)


def _x(wl, T, rep, scale=1.0):
    xh = synth.make_tokens(wl, rep=rep, T=T)
    if scale != 1.0:
        xh = f32_to_bf16_bits((bf16_bits_to_f64(xh) * scale).astype(np.float32))
    return xh, mx.bf16_from_numpy(xh, DEV)


def _forward_check(wl, L, D, cfg, T, rep, scale=1.0):
    assert mx.forward_schedule(cfg, T) == "large"
    xh, x = _x(wl, T, rep, scale)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, D, out_fp32=False)
    again = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "not deterministic"
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    e = assert_outputs_close(out.cpu().numpy(), ref, f"forward mxl T={T} scale {scale}")
    print(f"[mxl T={T} scale {scale}] rel L2 {e['rel_l2']:.2e} max abs/rms {e['max_abs'] / e['rms']:.2e}",
          flush=True)
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))
    return ids.cpu().numpy()


@pytest.mark.parametrize("T", [65, 129, 300, 1000])
def test_forward_mx_matches_oracle(mxl, T):
    wl, L, D, cfg = mxl
    print(f"[forward mxl T={T}]", flush=True)
    _forward_check(wl, L, D, cfg, T, rep=T)


def test_forward_mx_clamped(mxl):
    """Tokens x32 (exact in bf16): gate and up pre-activations spread to about
    +-14, so both clamps are hit in the routed and the shared experts."""
    wl, L, D, cfg = mxl
    _forward_check(wl, L, D, cfg, 300, rep=77, scale=32.0)


def test_forward_mx_tile_queue_every_row(mxl):
    """4096 tokens: about 6 * 4096 / 64 live tiles x 2 w13 N tiles, several
    times the persistent grid."""
    wl, L, D, cfg = mxl
    ids = _forward_check(wl, L, D, cfg, 4096, rep=41)
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    live = int(np.sum((counts + 63) // 64))
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    assert live * (wl.I // 256) > 2 * grid, (live, grid)


@pytest.mark.parametrize("case", ["skew", "same"])
def test_expert_ffn_mx_matches_oracle(mxl, case):
    wl, L, D, cfg = mxl
    rng = np.random.default_rng(5)
    T = 777
    if case == "same":
        ids_h = np.tile(np.arange(wl.k, dtype=np.int32) * 5, (T, 1))
    else:
        p = np.exp(rng.standard_normal(wl.E) * 2.0)
        ids_h = np.stack([rng.choice(wl.E, size=wl.k, replace=False, p=p / p.sum())
                          for _ in range(T)]).astype(np.int32)
    w_h = rng.uniform(0.05, 0.5, size=ids_h.shape).astype(np.float32)
    xh, x = _x(wl, T, rep=3)
    offsets, sorted_slots, _ = mx.permute(cfg, torch.from_numpy(ids_h).to(DEV))
    out = mx.expert_ffn(cfg, x, offsets, sorted_slots, torch.from_numpy(w_h).to(DEV), D.w13_codes, D.w13_scales,
                        D.w2_codes, D.w2_scales)
    ref = oracle.expert_ffn(xh, ids_h, w_h.astype(np.float64), L.w13_codes, L.w13_scales, L.w2_codes,
                            L.w2_scales)
    assert_outputs_close(out.cpu().numpy(), ref, f"expert_ffn mxl {case}")


def test_forward_mx_hash_matches_oracle(mxl):
    wl, _, _, cfg = mxl
    wlh = synth.Workload("mxl_hash", T=250, H=wl.H, E=wl.E, k=wl.k, I=wl.I, V=wl.V, hash_layer=True, seed=12)
    Lh = synth.make_layer(wlh)
    Dh = mx.DeviceLayer.from_host(Lh, DEV)
    xh, x = _x(wlh, 250, rep=1)
    tid_h = synth.make_token_ids(wlh, rep=0)
    out, (ids, w) = mx.forward(cfg, x, Dh, token_ids=torch.from_numpy(tid_h).to(DEV), out_fp32=True,
                               return_routing=True)
    r = oracle.forward(Lh, xh, token_ids=tid_h)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.abs(w.cpu().numpy() - r["w"]).max() <= 1e-5
    assert_outputs_close(out.cpu().numpy(), r["out"], "forward mxl hash")

"""GPU parity of the large-batch schedule (grouped GEMMs, T > 64) against the
CPU oracle, on a mid-size layer: hidden 512 (two 256-row output tiles of w2),
intermediate 384 (three 128-column SwiGLU tiles of w13), 32 experts, top-6.
Token counts give ragged 128-position tiles per expert; one case sends every
token to the same six experts (tiles full up to one ragged tail), and the
hash-routed layer runs the same GEMMs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")

DEV = "cuda"
MID = synth.Workload("mid", T=300, H=512, E=32, k=6, I=384, V=5000, bias_sigma=0.05)


@pytest.fixture(scope="module")
def mid():
    L = synth.make_layer(MID)
    return MID, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(MID)


def _x(wl, T, rep):
    xh = synth.make_tokens(wl, rep=rep, T=T)
    return xh, mx.bf16_from_numpy(xh, DEV)


@pytest.mark.parametrize("T", [65, 129, 300, 1000])
def test_forward_gemm_matches_oracle(mid, T):
    wl, L, D, cfg = mid
    print(f"[forward mid T={T}]", flush=True)
    xh, x = _x(wl, T, rep=T)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    out_bf = mx.forward(cfg, x, D, out_fp32=False)
    torch.cuda.synchronize()
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward mid T={T}")
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("case", ["skew", "same"])
def test_expert_ffn_gemm_matches_oracle(mid, case):
    wl, L, D, cfg = mid
    print(f"[expert_ffn mid {case}]", flush=True)
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
    assert_outputs_close(out.cpu().numpy(), ref, f"expert_ffn mid {case}")


def test_forward_hash_gemm_matches_oracle(mid):
    wl, _, _, cfg = mid
    print("[forward mid hash T=250]", flush=True)
    wlh = synth.Workload("mid_hash", T=250, H=wl.H, E=wl.E, k=wl.k, I=wl.I, V=wl.V, hash_layer=True)
    Lh = synth.make_layer(wlh)
    Dh = mx.DeviceLayer.from_host(Lh, DEV)
    xh, x = _x(wlh, 250, rep=1)
    tid_h = synth.make_token_ids(wlh, rep=0)
    out, (ids, w) = mx.forward(cfg, x, Dh, token_ids=torch.from_numpy(tid_h).to(DEV), out_fp32=True,
                               return_routing=True)
    r = oracle.forward(Lh, xh, token_ids=tid_h)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.abs(w.cpu().numpy() - r["w"]).max() <= 1e-5
    assert_outputs_close(out.cpu().numpy(), r["out"], "forward mid hash")


def test_forward_gemm_tile_queue_every_row(mid):
    """4096 tokens: the live 128-position tiles (about 6 * 4096 / 128 + 32 per
    N tile, times 3 or 2 N tiles) are several times the persistent grid, so
    blocks take tiles from the per-XCD queues past their first fixed ones;
    every output row is compared, and a second call on the same workspace
    (queue counters reset by the last block out) must repeat the bits."""
    wl, L, D, cfg = mid
    T = 4096
    print(f"[forward mid T={T} tile queue]", flush=True)
    xh, x = _x(wl, T, rep=41)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    again = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    ids_h = ids.cpu().numpy()
    counts = np.bincount(ids_h.ravel(), minlength=wl.E)
    live = int(np.sum((counts + 127) // 128))
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    assert live * (wl.I // 128) > 2 * grid, (live, grid)
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids_h, w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward mid T={T}")


def test_forward_gemm_deterministic(mid):
    wl, L, D, cfg = mid
    xh, x = _x(wl, 500, rep=2)
    a = mx.forward(cfg, x, D, out_fp32=True)
    b = mx.forward(cfg, x, D, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_expert_ffn_gemm_unequal_runs(mid):
    """Every token on experts 0-5 but 26 (one slot each moved to experts
    6-31): the tile list is 192 full tiles, then 26 one-position tiles, so
    the persistent GEMM's eight per-XCD runs of equal tile counts are
    unequal work (the last XCD's run is nearly all one-position tiles) and
    its blocks take tiles from the other XCDs' runs. Every row against the
    oracle, and a second call gives the same bits."""
    wl, L, D, cfg = mid
    T = 4096
    print(f"[expert_ffn mid T={T} unequal runs]", flush=True)
    rng = np.random.default_rng(11)
    ids_h = np.tile(np.arange(wl.k, dtype=np.int32), (T, 1))
    movers = rng.choice(T, size=wl.E - wl.k, replace=False)
    for e, t in zip(range(wl.k, wl.E), movers):
        ids_h[t, rng.integers(wl.k)] = e
    w_h = rng.uniform(0.05, 0.5, size=ids_h.shape).astype(np.float32)
    xh, x = _x(wl, T, rep=13)
    offsets, sorted_slots, _ = mx.permute(cfg, torch.from_numpy(ids_h).to(DEV))
    args = (cfg, x, offsets, sorted_slots, torch.from_numpy(w_h).to(DEV), D.w13_codes, D.w13_scales, D.w2_codes,
            D.w2_scales)
    out = mx.expert_ffn(*args)
    again = mx.expert_ffn(*args)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    counts = np.bincount(ids_h.ravel(), minlength=wl.E)
    live = int(np.sum((counts + 127) // 128))
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    assert live * (wl.I // 128) > 2 * grid, (live, grid)
    ref = oracle.expert_ffn(xh, ids_h, w_h.astype(np.float64), L.w13_codes, L.w13_scales, L.w2_codes,
                            L.w2_scales)
    assert_outputs_close(out.cpu().numpy(), ref, f"expert_ffn mid T={T} unequal runs")


LONGK = synth.Workload("longk", T=300, H=256, E=8, k=6, I=2176, V=5000, bias_sigma=0.05)


@pytest.mark.parametrize("T", [256, 300])
def test_forward_gemm_long_shared_k(T):
    """Intermediate 2176 = 17 x 128: routed w2 runs an odd number of MXFP4
    stages (17, the K loop's last stage after its stage pairs) and the
    shared expert's int8 w2 + combine 34 stages; 17 SwiGLU column tiles of
    w13. T=256 is two full token tiles, T=300 adds a ragged one. Every row
    against the oracle, bf16 output equal to the rounded fp32 one, and a
    second call repeats the bits."""
    wl = LONGK
    print(f"[forward longk T={T}]", flush=True)
    L = synth.make_layer(wl)
    D = mx.DeviceLayer.from_host(L, DEV)
    cfg = mx.config_of(wl)
    xh, x = _x(wl, T, rep=T + 7)
    out, (ids, w) = mx.forward(cfg, x, D, out_fp32=True, return_routing=True)
    again = mx.forward(cfg, x, D, out_fp32=True)
    out_bf = mx.forward(cfg, x, D, out_fp32=False)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))
    rows = np.arange(T, dtype=np.int32)
    r, ref = reference_rows(L, xh, rows)
    rt = compare_routing(ids.cpu().numpy(), w.cpu().numpy(), r["ids"], r["w"], r["gap"], r["next"])
    if rt["alt_rows"]:
        r, ref = reference_rows(L, xh, rows, routing=rt)
    assert_outputs_close(out.cpu().numpy(), ref, f"forward longk T={T}")

"""GPU parity of the layer with the routed experts' down projection (w2) in
3-bit blocks (moe_forward_w2q3): 14 bytes per 32 weights, one code book for
every block (uniform) or a table per expert (adaptive), page
"Geometric-AI/DeepSeek-V4-Flash-0731-ROCmFP3-MIX", introduction and section
"What 'adaptive' means here"; the field layout is the library's own (12
code bytes, a binary16 scale). Against the oracle's or_forward_w2q3 at the
usual bar (the kernels round each decoded weight, scale x level, to bf16:
at most 2^-9 relative per weight, far inside rel L2 5e-3):
  * decode sizes, T = 1, 2 (the single-launch layer), 5, 17, 64 (one
    streaming launch), learned and hash routing, uniform and tables, every
    row;
  * the grouped GEMM, T = 65, 300 and 1000 (several tiles per expert and
    ragged last tiles), every row;
  * the full-shape layer at T = 1, 64 (sampled rows) and 8192 (32
    stratified rows);
  * binary16 subnormal scales (tiny weights);
  * the MXFP4-equal case: uniform book and power-of-two scales hold exactly
    the numbers of an MXFP4 w2, so moe_forward_w2q3 and moe_forward agree
    to the bit when h and the routing agree (same kernels' sums except the
    w2 decode)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close, compare_routing, reference_rows

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"

MID = synth.Workload("q3mid", T=1, H=2048, E=64, k=6, I=1024, V=5000, seed=31)
MIDH = synth.Workload("q3midh", T=1, H=2048, E=64, k=6, I=1024, V=5000, hash_layer=True, seed=32)
_CACHE = {}


def _layer(wl, tables):
    key = (wl.name, tables)
    if key not in _CACHE:
        if wl.name not in _CACHE:
            L = synth.make_layer(wl)
            _CACHE[wl.name] = (L, mx.DeviceLayer.from_host(L, DEV))
        L, D = _CACHE[wl.name]
        c, s, lv = synth.make_w2q3(wl, tables)
        dev = (torch.from_numpy(c).to(DEV), torch.from_numpy(s.view(np.int16)).to(DEV),
               None if lv is None else torch.from_numpy(lv).to(DEV))
        _CACHE[key] = (L, D, (c, s, lv), dev)
    return _CACHE[key]


def _oracle_fwd(host_w2):
    c, s, lv = host_w2
    return lambda layer, x, **kw: oracle.forward_w2q3(layer, c, s, lv, x, **kw)


def _run(wl, tables, T, rep, rows=None, hash_layer=False):
    L, D, hw, dw = _layer(wl, tables)
    cfg = mx.config_of(wl)
    tag = f"[w2q3 {wl.name} {'tables' if tables else 'uniform'} T={T}]"
    print(tag, flush=True)
    xh = synth.make_tokens(wl, rep=rep, T=T)
    x = mx.bf16_from_numpy(xh, DEV)
    tid_h = synth.make_token_ids(wl, rep=rep, T=T) if hash_layer else None
    tids = None if tid_h is None else torch.from_numpy(tid_h).to(DEV)
    out, (ids, w) = mx.forward_w2q3(cfg, x, D, *dw, token_ids=tids, out_fp32=True, return_routing=True)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    rows = np.arange(T, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    fwd = _oracle_fwd(hw)
    r = fwd(L, xh, token_ids=tid_h, rows=rows)
    routing = None
    if hash_layer:
        assert np.array_equal(ids[rows], r["ids"])
    else:
        routing = compare_routing(ids[rows], w[rows], r["ids"], r["w"], r["gap"], r["next"])
        if routing["alt_rows"]:
            routing["alt_rows"] = {int(rows[i]): a for i, a in routing["alt_rows"].items()}
            _, ref = reference_rows(L, xh, rows, routing=routing, fwd=fwd)
            r["out"] = ref
    e = assert_outputs_close(out.cpu().numpy()[rows], r["out"], tag)
    print(f"{tag} rel L2 {e['rel_l2']:.2e} max abs/rms {e['max_abs'] / e['rms']:.2e}", flush=True)
    return out, ids


@pytest.mark.parametrize("tables", [False, True])
@pytest.mark.parametrize("T", [1, 2, 5, 17, 64])
def test_w2q3_decode(T, tables):
    _run(MID, tables, T, 400 + T)


@pytest.mark.parametrize("tables", [False, True])
@pytest.mark.parametrize("T", [65, 300, 1000])
def test_w2q3_gemm(T, tables):
    _run(MID, tables, T, 420 + T)


@pytest.mark.parametrize("T", [1, 2, 17, 300])
def test_w2q3_hash(T):
    _run(MIDH, True, T, 440 + T, hash_layer=True)


def test_w2q3_subnormal_scales():
    """Weights of about 1e-6: every block scale is a binary16 subnormal."""
    wl = synth.Workload("q3tiny", T=1, H=2048, E=64, k=6, I=1024, V=5000, seed=33, weight_sigma=2e-7)
    L, D, hw, dw = _layer(wl, True)
    s = hw[1]
    assert ((s & 0x7C00) == 0).mean() > 0.99 and (s & 0x03FF).max() > 0
    for T in (3, 100):
        _run(wl, True, T, 460 + T)


def test_w2q3_equals_mxfp4_when_exact():
    """Uniform book, power-of-two scales: the 3-bit w2 holds the MXFP4 w2's
    numbers exactly, so both entry points give the same bits at every
    schedule the 3-bit path takes (the streaming launch and the GEMM)."""
    wl = synth.Workload("q3eq", T=1, H=2048, E=64, k=6, I=1024, V=5000, seed=34)
    rng = np.random.default_rng(34)
    E, H, I = wl.E, wl.H, wl.I
    c = rng.integers(0, 8, size=(E * H, I))
    c[:, ::32] = 0
    xexp = rng.integers(-10, -6, size=(E * H, I // 32))
    wts = (np.repeat(np.ldexp(1.0, xexp), 32, axis=1) * (c - 4.0)).astype(np.float32)
    qc, qs = synth.quant_q3(wts)
    mc, ms = synth.quant_mxfp4(wts)
    L = synth.make_layer(wl)
    L.w2_codes, L.w2_scales = mc.reshape(E, H, I // 2), ms.reshape(E, H, I // 32)
    D = mx.DeviceLayer.from_host(L, DEV)
    dq = (torch.from_numpy(qc.reshape(E, H, -1)).to(DEV), torch.from_numpy(qs.view(np.int16).reshape(E, H, -1)).to(DEV))
    cfg = mx.config_of(wl)
    for T in (1, 2, 3, 64, 200):
        print(f"[w2q3 == mxfp4 T={T}]", flush=True)
        x = mx.bf16_from_numpy(synth.make_tokens(wl, rep=470 + T, T=T), DEV)
        a = mx.forward_w2q3(cfg, x, D, *dq, None, out_fp32=True)
        # the MXFP4 layer in the same schedule (single launch, streaming launch or GEMM)
        b = mx.forward(cfg, x, D, out_fp32=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b), T


def _full(full_layer):
    L, D = full_layer
    wl = synth.WORKLOADS["decode_t1"]
    key = ("decode_t1", True)
    if key not in _CACHE:
        print("[generating the full-shape 3-bit w2]", flush=True)
        c, s, lv = synth.make_w2q3(wl, True)
        _CACHE[key] = (L, D, (c, s, lv), (torch.from_numpy(c).to(DEV), torch.from_numpy(s.view(np.int16)).to(DEV),
                                          torch.from_numpy(lv).to(DEV)))
    return wl, _CACHE[key]


def test_w2q3_full_shape_decode(full_layer):
    """The full-shape layer (hidden 4096, 256 experts, intermediate 2048)
    with a 3-bit w2 (tables): T = 1, and T = 64 on sampled rows."""
    wl, _ = _full(full_layer)
    _run(wl, True, 1, 480)
    _run(wl, True, 64, 481, rows=[0, 5, 17, 33, 50, 63])


def test_w2q3_full_shape_prefill(full_layer):
    """T = 8192 on 32 stratified rows (the ragged last tiles of the
    most-loaded experts among them)."""
    from test_gpu_full import _stratified_rows
    wl, (L, D, hw, dw) = _full(full_layer)
    x = mx.bf16_from_numpy(synth.make_tokens(wl, rep=482, T=8192), DEV)
    _, (ids, _) = mx.forward_w2q3(mx.config_of(wl), x, D, *dw, return_routing=True)
    torch.cuda.synchronize()
    rows = _stratified_rows(ids.cpu().numpy(), wl.k, 32, seed=3, per=4)
    _run(wl, True, 8192, 482, rows=rows)

"""Pins of the CPU oracle: each check ties one step of the oracle to something
other than the oracle itself.

What the checks compare against:
  * the E2M1 code table of the OCP MX v1.0 specification (tests/golden),
  * the E8M0 definition 2^(b-127) through ``math.ldexp``,
  * byte counts the pages state (17 B and 14 B per 32 weights; about 3.4 GB
    per full layer),
  * closed forms (sqrt(ln 2), silu(10), the clamps), library routines
    (``numpy.logaddexp``, ``scipy.special.expit``, ``numpy.matmul``,
    ``numpy.lexsort``/``argsort``, torch's bf16 conversion),
  * brute force over every k-subset on tiny expert counts,
  * invariants (weights sum to the routed scale, a shared bias shift does not
    change the selection, a +1 on every w2 scale byte doubles the output),
  * the E=1, k=1 special case, which is a dense SwiGLU MLP.

Every check raises AssertionError on a mismatch. ``test_oracle_pins`` runs them
against the oracle; ``test_oracle_mutations`` runs them against copies of the
oracle with one mistake planted and requires that some check fails.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
from scipy.special import expit

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ fixtures

def golden_e2m1() -> np.ndarray:
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert sorted(vals) == list(range(16))
    return np.array([vals[c] for c in range(16)], np.float64)


def golden_constants() -> dict:
    with open(os.path.join(GOLDEN, "layer_constants.json")) as f:
        return json.load(f)


def golden_block_bytes() -> list[tuple[str, int, int, int, int]]:
    rows = []
    with open(os.path.join(GOLDEN, "block_bytes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, bits, group, sbits, nbytes = line.split()
            rows.append((name, int(bits), int(group), int(sbits), int(nbytes)))
    return rows


def decode_mxfp4_table(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 [.., K/2] codes + [.., K/32] scales -> fp64 [.., K] via the golden
    table and ldexp; element 2i is the low nibble of byte i, scale g covers
    elements [32g, 32g+32)."""
    tab = golden_e2m1()
    vals = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.float64)
    vals[..., 0::2] = tab[codes & 15]
    vals[..., 1::2] = tab[codes >> 4]
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_round_bf16(v: np.ndarray) -> np.ndarray:
    import torch

    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def np_score(logits: np.ndarray) -> np.ndarray:
    return np.sqrt(np.logaddexp(0.0, logits))


def np_swiglu(g, u, limit=10.0):
    gc = np.minimum(g, limit)
    return gc * expit(gc) * np.clip(u, -limit, limit)


def np_topk(b32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest values, descending, ties to the lower index."""
    order = np.lexsort((np.arange(b32.shape[-1]), -b32.astype(np.float64)))
    return order[:k]


def _rng(seed):
    return np.random.default_rng(seed)


def _mxfp4_random(rng, shape_nk):
    """Random codes/scales for an [N, K] MXFP4 matrix (scales near 2^-3..2^1)."""
    N, K = shape_nk
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(124, 129, size=(N, K // 32), dtype=np.uint8)
    return codes, scales


# ------------------------------------------------------------------ format pins

def check_e2m1_codes():
    tab = golden_e2m1()
    for c in range(16):
        v = oracle.e2m1(c)
        assert v == tab[c] and math.copysign(1, v) == math.copysign(1, tab[c]), (c, v, tab[c])


def check_e8m0_bytes():
    for b in range(255):
        assert oracle.e8m0(b) == math.ldexp(1.0, b - 127), b
    assert math.isnan(oracle.e8m0(255))


def check_mxfp4_layout():
    rng = _rng(1)
    codes, scales = _mxfp4_random(rng, (3, 96))
    got = oracle.mxfp4_decode(codes, scales)
    want = decode_mxfp4_table(codes, scales)
    assert np.array_equal(got, want)


def check_block_bytes():
    for name, bits, group, sbits, nbytes in golden_block_bytes():
        assert oracle.block_bytes(bits, group, sbits) == nbytes, name
    c = golden_constants()
    H, I, E = c["hidden_size"], c["moe_intermediate_size"], c["n_routed_experts"]
    q = c["experts_w4a16"]
    per32 = oracle.block_bytes(q["num_bits"], q["group_size"], 8)
    per_expert = (2 * I * H + H * I) // q["group_size"] * per32
    assert per_expert == 13_369_344
    layer = E * per_expert
    assert layer == 3_422_552_064 and abs(layer / 1e9 - 3.4) < 0.05  # "about 3.4 GB"


def check_bf16_values():
    rng = _rng(2)
    bits = rng.integers(0, 1 << 16, size=2000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite values
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    import torch

    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)
    vals = np.concatenate([rng.standard_normal(500) * 10.0 ** rng.integers(-6, 6, 500),
                           [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, 3.0]])
    vals = vals.astype(np.float32).astype(np.float64)  # exactly fp32, so torch rounds once
    got = np.array([oracle.round_bf16(float(v)) for v in vals])
    assert np.array_equal(got, torch_round_bf16(vals))


# ------------------------------------------------------------------ elementwise pins

def check_softplus_score():
    assert abs(oracle.score(0.0) - math.sqrt(math.log(2.0))) < 1e-15
    assert abs(oracle.score(0.0) - 0.8325546111576977) < 1e-15
    zs = np.linspace(-60.0, 60.0, 241)
    sp = np.array([oracle.softplus(float(z)) for z in zs])
    ref = np.logaddexp(0.0, zs)
    assert np.all(np.abs(sp - ref) <= 1e-14 * np.maximum(ref, 1e-300) + 1e-300)
    sc = np.array([oracle.score(float(z)) for z in zs])
    assert np.allclose(sc, np.sqrt(ref), rtol=1e-14, atol=0)
    assert np.all(np.diff(sc) > 0) and np.all(sc > 0)


def check_swiglu():
    L = 10.0
    silu10 = 10.0 * expit(10.0)
    assert abs(silu10 - 9.999546021312976) < 1e-12
    cases = [(20.0, 50.0, silu10 * 10.0),            # gate clamped above, up clamped above
             (20.0, -50.0, silu10 * -10.0),          # up clamped below
             (-20.0, 1.0, -20.0 * expit(-20.0)),     # no lower clamp on the gate
             (-50.0, 2.0, -50.0 * expit(-50.0) * 2.0),
             (2.0, 3.0, 2.0 * expit(2.0) * 3.0),
             (10.0, 10.0, silu10 * 10.0),
             (0.0, 7.0, 0.0)]
    for g, u, want in cases:
        got = oracle.swiglu(g, u, L)
        assert abs(got - want) <= 1e-15 * max(1.0, abs(want)) or got == want, (g, u, got, want)
    assert abs(oracle.swiglu(-20.0, 1.0, L) - (-4.1223072363804074e-08)) < 1e-20


# ------------------------------------------------------------------ routing pins

def _route_with_bias(bias: np.ndarray, k: int, H: int = 32):
    """Router with a zero gate: every logit is 0, every score sqrt(ln 2), so
    the selection is decided by the biases alone."""
    E = bias.shape[0]
    x = np.zeros((1, H), np.uint16)
    gate = np.zeros((E, H), np.float32)
    return oracle.route(x, gate, bias.astype(np.float32), k=k)


def check_topk_exhaustive():
    rng = _rng(3)
    for E in (6, 7, 8, 9):
        for k in range(1, min(6, E - 1) + 1):
            for _ in range(12):
                bias = rng.integers(-2, 3, size=E).astype(np.float32)  # many exact ties
                ids, w, gap, nxt = _route_with_bias(bias, k)
                b = (np.float64(math.sqrt(math.log(2.0))) + bias).astype(np.float32)
                valid = []
                for S in itertools.combinations(range(E), k):
                    inS = set(S)
                    ok = all((b[i] > b[j]) or (b[i] == b[j] and i < j)
                             for i in inS for j in range(E) if j not in inS)
                    if ok:
                        valid.append(S)
                assert len(valid) == 1, (bias, valid)
                want = sorted(valid[0], key=lambda e: (-b[e], e))
                assert list(ids[0]) == want, (E, k, bias, ids[0], want)
                assert np.allclose(w[0], 1.5 / k, rtol=1e-15, atol=0)
                rest = [e for e in range(E) if e not in valid[0]]
                best_rest = sorted(rest, key=lambda e: (-b[e], e))[0]
                assert nxt[0] == best_rest
                assert gap[0] == float(b[want[-1]]) - float(b[best_rest])


def check_topk_random():
    rng = _rng(4)
    T, H, E, k = 40, 64, 16, 6
    x = synth.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    gate = (rng.standard_normal((E, H)) * 0.2).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    off = (rng.standard_normal(E) * 0.5).astype(np.float32)
    for use_off in (False, True):
        ids, w, gap, nxt = oracle.route(x, gate, bias, off if use_off else None, k=k)
        logits = bf16_to_f64(x) @ gate.astype(np.float64).T
        if use_off:
            logits = logits + off.astype(np.float64)
        s = np_score(logits)
        b32 = (s + bias.astype(np.float64)).astype(np.float32)
        for t in range(T):
            srt = np.sort(b32[t])[::-1]
            if srt[k - 1] - srt[k] < 1e-6:
                continue  # fp64 sum order could flip a near-tie here
            want = np_topk(b32[t], k)
            assert list(ids[t]) == list(want), (t, ids[t], want)
            ww = 1.5 * s[t, want] / s[t, want].sum()
            assert np.allclose(w[t], ww, rtol=1e-13, atol=0)


def check_fp32_decision():
    # Two biases one fp32 ulp apart: in fp64 the biased scores differ, after
    # rounding to fp32 (the precision the selection is decided in) they tie,
    # and the tie goes to the lower expert id.
    E = 3
    x = np.zeros((1, 32), np.uint16)
    gate = np.zeros((E, 32), np.float32)
    s0 = math.sqrt(math.log(2.0))  # every score with a zero gate
    b0 = np.float32(0.25)  # its fp32 ulp is a quarter of the ulp of s0 + b0
    while True:
        b1 = np.nextafter(b0, np.float32(1.0))
        if np.float32(s0 + float(b1)) == np.float32(s0 + float(b0)):
            break
        b0 = b1
    assert s0 + float(b1) > s0 + float(b0)                      # fp64 would pick expert 1
    assert np.float32(s0 + float(b1)) == np.float32(s0 + float(b0))  # fp32 ties
    ids, *_ = oracle.route(x, gate, np.array([b0, b1, 0.25], np.float32), k=1)
    assert ids[0, 0] == 0
    b2 = np.float32(0.5 + 2.0 ** -20)                           # distinct in fp32 too
    ids, *_ = oracle.route(x, gate, np.array([b0, b2, 0.25], np.float32), k=1)
    assert ids[0, 0] == 1


def check_noaux_bias():
    rng = _rng(5)
    T, H, E, k = 30, 64, 16, 6
    x = synth.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    gate = (rng.standard_normal((E, H)) * 0.2).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ids0, w0, gap0, _ = oracle.route(x, gate, bias, k=k)
    ids1, w1, gap1, _ = oracle.route(x, gate, (bias + np.float32(0.25)).astype(np.float32), k=k)
    stable = (gap0 > 1e-5) & (gap1 > 1e-5)
    assert stable.sum() >= T // 2
    assert np.array_equal(ids0[stable], ids1[stable])
    assert np.array_equal(w0[stable], w1[stable])
    # A large bias forces an expert in; its weight still comes from the
    # unbiased score (the bias only selects).
    e_star = 3
    bb = bias.copy()
    bb[e_star] += 100.0
    ids2, w2, _, _ = oracle.route(x, gate, bb, k=k)
    s = np_score(bf16_to_f64(x) @ gate.astype(np.float64).T)
    for t in range(T):
        assert ids2[t, 0] == e_star
        want = 1.5 * s[t, ids2[t]] / s[t, ids2[t]].sum()
        assert np.allclose(w2[t], want, rtol=1e-13, atol=0)


def check_weights_sum():
    L = synth.make_layer(synth.WORKLOADS["tiny"])
    x = synth.make_tokens(L.wl)
    ids, w, gap, _ = oracle.route(x, L.gate_w, L.bias, k=L.wl.k)
    assert np.all(np.abs(w.sum(1) - 1.5) <= 1e-12) and np.all(w > 0)
    assert all(len(set(r)) == L.wl.k for r in ids)


def check_hash_route():
    rng = _rng(6)
    T, H, E, k, V = 25, 64, 16, 6, 50
    x = synth.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    gate = (rng.standard_normal((E, H)) * 0.2).astype(np.float32)
    t2e = synth.tid2eid(0, 10, 0, V, E, k)
    tids = rng.integers(0, V, size=T).astype(np.int32)
    ids, w = oracle.hash_route(x, tids, t2e, gate)
    assert np.array_equal(ids, t2e[tids])
    s = np_score(bf16_to_f64(x) @ gate.astype(np.float64).T)
    for t in range(T):
        want = 1.5 * s[t, ids[t]] / s[t, ids[t]].sum()
        assert np.allclose(w[t], want, rtol=1e-13, atol=0)


# ------------------------------------------------------------------ permutation pins

def check_permute():
    rng = _rng(7)
    for T, k, E in ((0, 6, 16), (1, 6, 256), (37, 6, 16), (200, 6, 256), (64, 1, 4)):
        p = np.exp(rng.standard_normal(E) * 1.5)
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]
                       ).astype(np.int32).reshape(T, k) if T else np.zeros((0, k), np.int32)
        offsets, sorted_slots, slot_pos = oracle.permute(ids, E)
        flat = ids.ravel()
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert np.array_equal(sorted_slots, np.argsort(flat, kind="stable"))
        assert np.array_equal(slot_pos[sorted_slots], np.arange(T * k))


# ------------------------------------------------------------------ expert pins

def _tiny_weights(rng, E, H, I, sigma_scale=(124, 131)):
    c13 = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
    s13 = rng.integers(*sigma_scale, size=(E, 2 * I, H // 32), dtype=np.uint8)
    c2 = rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    s2 = rng.integers(*sigma_scale, size=(E, H, I // 32), dtype=np.uint8)
    return c13, s13, c2, s2


def np_expert(xd, c13, s13, c2, s2, round_h, limit=10.0):
    W13 = decode_mxfp4_table(c13, s13)
    W2 = decode_mxfp4_table(c2, s2)
    I = W13.shape[0] // 2
    g = W13[:I] @ xd
    u = W13[I:] @ xd
    h = np_swiglu(g, u, limit)
    if round_h:
        h = torch_round_bf16(h.astype(np.float32).astype(np.float64))
    return W2 @ h, g, u


def check_expert_ffn():
    rng = _rng(8)
    E, H, I, T, k = 4, 64, 32, 5, 2
    c13, s13, c2, s2 = _tiny_weights(rng, E, H, I)
    x = synth.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    xd = bf16_to_f64(x)
    saw_clamp_hi = saw_low = False
    for round_h in (False, True):
        got = oracle.expert_ffn(x, ids, w, c13, s13, c2, s2, round_h=round_h)
        for t in range(T):
            want = np.zeros(H)
            for j in range(k):
                y, g, u = np_expert(xd[t], c13[ids[t, j]], s13[ids[t, j]], c2[ids[t, j]], s2[ids[t, j]],
                                    round_h)
                saw_clamp_hi |= bool((g > 10).any() and (np.abs(u) > 10).any())
                saw_low |= bool((g < -10).any())
                want += w[t, j] * y
            assert np.allclose(got[t], want, rtol=1e-12, atol=1e-12 * np.abs(want).max()), (round_h, t)
    assert saw_clamp_hi and saw_low  # the data exercised both clamps and the unclamped low gate


def check_shared_ffn():
    rng = _rng(9)
    H, I, T = 64, 32, 4
    q13 = rng.integers(-127, 128, size=(2 * I, H), dtype=np.int8)
    s13 = rng.uniform(0.01, 0.1, size=2 * I).astype(np.float32)
    q2 = rng.integers(-127, 128, size=(H, I), dtype=np.int8)
    s2 = rng.uniform(0.01, 0.1, size=H).astype(np.float32)
    x = synth.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    xd = bf16_to_f64(x)
    W13 = q13.astype(np.float64) * s13.astype(np.float64)[:, None]
    W2 = q2.astype(np.float64) * s2.astype(np.float64)[:, None]
    for round_h in (False, True):
        z = oracle.shared_ffn(x, q13, s13, q2, s2, round_h=round_h)
        g = xd @ W13[:I].T
        u = xd @ W13[I:].T
        h = np_swiglu(g, u)
        assert (np.abs(g) > 10).any()
        if round_h:
            h = torch_round_bf16(h.astype(np.float32).astype(np.float64))
        want = h @ W2.T
        assert np.allclose(z, want, rtol=1e-12, atol=1e-12 * np.abs(want).max()), round_h


def check_linearity():
    rng = _rng(10)
    E, H, I, T, k = 3, 64, 32, 3, 2
    c13, s13, c2, s2 = _tiny_weights(rng, E, H, I)
    x = synth.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.array([[0, 1], [2, 0], [1, 2]], np.int32)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    a = oracle.expert_ffn(x, ids, w, c13, s13, c2, s2)
    b = oracle.expert_ffn(x, ids, w, c13, s13, c2, (s2 + 1).astype(np.uint8))
    assert np.array_equal(2.0 * a, b)
    q13 = rng.integers(-127, 128, size=(2 * I, H), dtype=np.int8)
    sc13 = rng.uniform(0.01, 0.1, size=2 * I).astype(np.float32)
    q2 = rng.integers(-127, 128, size=(H, I), dtype=np.int8)
    sc2 = rng.uniform(0.01, 0.1, size=H).astype(np.float32)
    z1 = oracle.shared_ffn(x, q13, sc13, q2, sc2)
    z2 = oracle.shared_ffn(x, q13, sc13, q2, (sc2 * 2).astype(np.float32))
    assert np.array_equal(2.0 * z1, z2)


def _layer_from(wl, gate, bias, c13, s13, c2, s2, q13, sc13, q2, sc2, off=None, t2e=None):
    return synth.Layer(wl, gate, bias, off, c13, s13, c2, s2, q13, sc13, q2, sc2, t2e)


def check_special_case_dense():
    """E = 1, k = 1: the layer is 1.5 * MLP_0(x) + shared(x), two dense SwiGLU MLPs."""
    rng = _rng(11)
    H, I, T = 64, 32, 6
    wl = synth.Workload("e1k1", T=T, H=H, E=1, k=1, I=I, V=10)
    c13, s13, c2, s2 = _tiny_weights(rng, 1, H, I)
    q13 = rng.integers(-127, 128, size=(2 * I, H), dtype=np.int8)
    sc13 = rng.uniform(0.01, 0.1, size=2 * I).astype(np.float32)
    q2 = rng.integers(-127, 128, size=(H, I), dtype=np.int8)
    sc2 = rng.uniform(0.01, 0.1, size=H).astype(np.float32)
    gate = (rng.standard_normal((1, H)) * 0.1).astype(np.float32)
    layer = _layer_from(wl, gate, np.zeros(1, np.float32), c13, s13, c2, s2, q13, sc13, q2, sc2)
    x = synth.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    r = oracle.forward(layer, x, round_h=False)
    xd = bf16_to_f64(x)
    W13 = decode_mxfp4_table(c13[0], s13[0])
    W2 = decode_mxfp4_table(c2[0], s2[0])
    S13 = q13.astype(np.float64) * sc13.astype(np.float64)[:, None]
    S2 = q2.astype(np.float64) * sc2.astype(np.float64)[:, None]
    mlp = lambda A, B: np_swiglu(xd @ A[:I].T, xd @ A[I:].T) @ B.T  # noqa: E731
    want = 1.5 * mlp(W13, W2) + mlp(S13, S2)
    assert np.array_equal(r["ids"], np.zeros((T, 1), np.int32))
    assert np.allclose(r["w"], 1.5, rtol=1e-15, atol=0)
    assert np.allclose(r["out"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def check_forward_tiny():
    """The whole tiny layer against a numpy evaluation of the same definition."""
    L = synth.make_layer(synth.WORKLOADS["tiny"])
    wl = L.wl
    x = synth.make_tokens(wl)
    r = oracle.forward(L, x, round_h=False)
    xd = bf16_to_f64(x)
    s = np_score(xd @ L.gate_w.astype(np.float64).T)
    b32 = (s + L.bias.astype(np.float64)).astype(np.float32)
    S13 = L.sh_w13.astype(np.float64) * L.sh_w13_scale.astype(np.float64)[:, None]
    S2 = L.sh_w2.astype(np.float64) * L.sh_w2_scale.astype(np.float64)[:, None]
    I = wl.I
    checked = 0
    for t in range(wl.T):
        srt = np.sort(b32[t])[::-1]
        if srt[wl.k - 1] - srt[wl.k] < 1e-6:
            continue
        ids = np_topk(b32[t], wl.k)
        assert list(r["ids"][t]) == list(ids)
        w = 1.5 * s[t, ids] / s[t, ids].sum()
        out = np.zeros(wl.H)
        for j, e in enumerate(ids):
            y, _, _ = np_expert(xd[t], L.w13_codes[e], L.w13_scales[e], L.w2_codes[e], L.w2_scales[e], False)
            out += w[j] * y
        out += np_swiglu(S13[:I] @ xd[t], S13[I:] @ xd[t]) @ S2.T
        assert np.allclose(r["out"][t], out, rtol=1e-12, atol=1e-12 * np.abs(out).max()), t
        checked += 1
    assert checked >= wl.T - 2
    # a subset of rows reproduces the same rows exactly
    sub = oracle.forward(L, x, rows=np.array([3, 7, 0], np.int32), round_h=False)
    assert np.array_equal(sub["out"], r["out"][[3, 7, 0]])
    assert np.array_equal(sub["ids"], r["ids"][[3, 7, 0]])


def _np_layer_rows(L, xd, ids, w):
    """numpy composition of the layer for given expert ids and weights per row:
    sum_j w_j * expert_{ids_j}(x) + shared(x), h not rounded."""
    I = L.wl.I
    S13 = L.sh_w13.astype(np.float64) * L.sh_w13_scale.astype(np.float64)[:, None]
    S2 = L.sh_w2.astype(np.float64) * L.sh_w2_scale.astype(np.float64)[:, None]
    out = np.zeros((len(ids), L.wl.H))
    for r in range(len(ids)):
        for j, e in enumerate(ids[r]):
            y, _, _ = np_expert(xd[r], L.w13_codes[e], L.w13_scales[e], L.w2_codes[e], L.w2_scales[e], False)
            out[r] += w[r, j] * y
        out[r] += np_swiglu(S13[:I] @ xd[r], S13[I:] @ xd[r]) @ S2.T
    return out


def check_forward_forced_ids():
    """Forced expert ids (used to grade near-tie tokens): the oracle must take
    exactly the given experts, weight them by their own renormalised scores
    (x 1.5), and compose those experts with the shared expert; on a subset of
    rows the forced row r belongs to requested token rows[r]."""
    L = synth.make_layer(synth.WORKLOADS["tiny"])
    wl = L.wl
    x = synth.make_tokens(wl, rep=3)
    rows = np.array([9, 2, 14, 0], np.int32)
    rng = _rng(12)
    full = oracle.forward(L, x, rows=rows, round_h=False)
    forced = np.stack([rng.choice(wl.E, size=wl.k, replace=False) for _ in rows]).astype(np.int32)
    # at least one forced set must differ from the top-k, or the check is empty
    assert any(set(forced[r]) != set(full["ids"][r]) for r in range(len(rows)))
    r = oracle.forward(L, x, rows=rows, force_ids=forced, round_h=False)
    assert np.array_equal(r["ids"], forced)
    xd = bf16_to_f64(x[rows])
    s = np_score(xd @ L.gate_w.astype(np.float64).T)
    w = np.stack([1.5 * s[i, forced[i]] / s[i, forced[i]].sum() for i in range(len(rows))])
    assert np.allclose(r["w"], w, rtol=1e-13, atol=0)
    want = _np_layer_rows(L, xd, forced, w)
    assert np.allclose(r["out"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def check_forward_hash():
    """The whole hash-routed layer: experts are the table row of each token's
    id (table order), weights their renormalised scores x 1.5 with no bias,
    composed with the shared expert; checked on a subset of rows so the row
    of each output is that of the requested token."""
    wl = synth.Workload("tinyhash", T=16, H=256, E=16, k=6, I=128, V=40, hash_layer=True, seed=2)
    L = synth.make_layer(wl)
    x = synth.make_tokens(wl, rep=1)
    tids = synth.make_token_ids(wl, rep=1)
    rows = np.array([11, 3, 7, 15, 0], np.int32)
    assert len(set(tids[rows].tolist())) > 1
    r = oracle.forward(L, x, token_ids=tids, rows=rows, round_h=False)
    assert np.array_equal(r["ids"], L.tid2eid[tids[rows]])
    xd = bf16_to_f64(x[rows])
    s = np_score(xd @ L.gate_w.astype(np.float64).T)
    ids = L.tid2eid[tids[rows]]
    w = np.stack([1.5 * s[i, ids[i]] / s[i, ids[i]].sum() for i in range(len(rows))])
    assert np.allclose(r["w"], w, rtol=1e-13, atol=0)
    want = _np_layer_rows(L, xd, ids, w)
    assert np.allclose(r["out"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def check_linear_w8a16():
    """The int8 per-channel linear against numpy's matmul of the decoded
    weights (q times its row's scale), plain and grouped (block-diagonal):
    each group reads only its own input slice and writes only its own output
    slice; doubling one group's scales doubles exactly that group's outputs."""
    rng = _rng(13)
    for T, K, N, G in ((3, 64, 48, 1), (5, 32, 16, 4), (1, 96, 8, 2)):
        q = rng.integers(-127, 128, size=(G * N, K), dtype=np.int8)
        sc = rng.uniform(0.001, 0.05, size=G * N).astype(np.float32)
        x = synth.f32_to_bf16(rng.standard_normal((T, G * K)).astype(np.float32))
        got = oracle.linear_w8a16(x, q, sc, groups=G)
        xd = bf16_to_f64(x)
        W = q.astype(np.float64) * sc.astype(np.float64)[:, None]
        want = np.concatenate([xd[:, g * K:(g + 1) * K] @ W[g * N:(g + 1) * N].T for g in range(G)], axis=1)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max()), (T, K, N, G)
        if G > 1:
            sc2 = sc.copy()
            sc2[N:2 * N] *= 2
            got2 = oracle.linear_w8a16(x, q, sc2, groups=G)
            assert np.array_equal(got2[:, N:2 * N], 2 * got[:, N:2 * N])
            assert np.array_equal(np.delete(got2, np.s_[N:2 * N], axis=1), np.delete(got, np.s_[N:2 * N], axis=1))


# ------------------------------------------------------------------ 3-bit down experts

def golden_fp16() -> list[tuple[int, float]]:
    out = []
    with open(os.path.join(GOLDEN, "fp16_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, v = line.split()
            out.append((int(b, 16), float(v)))
    return out


def golden_q3_blocks() -> list[tuple[np.ndarray, list[int]]]:
    out = []
    with open(os.path.join(GOLDEN, "q3_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            left, right = line.split("|")
            b = np.array([int(t, 16) for t in left.split()], np.uint8)
            codes = [0] * 32
            for item in right.split():
                i, c = item.split("=")
                codes[int(i)] = int(c)
            out.append((b, codes))
    return out


def check_fp16_values():
    """binary16 scales: the golden IEEE values, and every one of the 65536
    patterns against numpy's float16."""
    for bits, v in golden_fp16():
        got = oracle.fp16_value(bits)
        if math.isnan(v):
            assert math.isnan(got), hex(bits)
        else:
            assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (hex(bits), got, v)
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    lib = oracle.lib()
    for b in range(0, 65536, 7):  # a spread of patterns; the golden list covers the special ones
        got = lib.or_fp16_value(b)
        want = allv[b]
        assert (math.isnan(got) and math.isnan(want)) or got == want, (hex(b), got, want)


def check_q3_codes():
    """The code of every weight of the hand-worked golden blocks."""
    blocks = golden_q3_blocks()
    assert len(blocks) >= 8
    for b, codes in blocks:
        assert [oracle.q3_code(b, i) for i in range(32)] == codes, b


def check_q3_values():
    """Golden blocks decoded with a binary16 scale, uniform (c - 4) and with a
    table of levels: value = scale x level[code]."""
    lv = np.array([-1.5, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 1.5], np.float32)
    blocks = golden_q3_blocks()
    codes = np.stack([b for b, _ in blocks])                       # [n, 12]: row r = block r
    sc_bits = np.array([0x3800, 0xC000, 0x0001, 0x3555] * 4, np.uint16)[: len(blocks)]
    scale = sc_bits.view(np.float16).astype(np.float64)
    uni = oracle.q3_decode(codes, sc_bits[:, None])
    tab = oracle.q3_decode(codes, sc_bits[:, None], lv)
    for r, (_, c) in enumerate(blocks):
        c = np.array(c)
        assert np.array_equal(uni[r], scale[r] * (c - 4.0)), r
        assert np.array_equal(tab[r], scale[r] * lv.astype(np.float64)[c]), r


def check_q3_roundtrip():
    """Weights encoded by the input generator (an encoder written separately)
    decode to the level nearest each weight: |w - decoded| is the distance
    to the nearest of scale x level, for the uniform book and for tables,
    over several rows and blocks (the block and row of each scale)."""
    rng = _rng(14)
    K = 128
    w = (rng.standard_normal((6, K)) * 0.02).astype(np.float32)
    w[2, 40] = 0.5  # a block with an outlier
    tabs = synth.q3_tables(3, 13, 0, 3)
    for tables in (None, tabs):
        codes, scales = synth.quant_q3(w, tables=tables, rows_per_table=2)
        dec = oracle.q3_decode(codes, scales) if tables is None else np.concatenate(
            [oracle.q3_decode(codes[2 * e:2 * e + 2], scales[2 * e:2 * e + 2], tables[e]) for e in range(3)])
        d = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
        for r in range(6):
            lv = np.arange(8.0) - 4 if tables is None else tables[r // 2].astype(np.float64)
            cand = d[r][:, None] * lv[None, :]                        # [K, 8]
            best = np.abs(w[r].astype(np.float64)[:, None] - cand).min(axis=1)
            err = np.abs(w[r].astype(np.float64) - dec[r])
            assert np.allclose(err, best, rtol=0, atol=1e-12), r
        assert np.abs(dec - w).max() < 0.5 * np.abs(w).max()


def _q3_equal_to_mxfp4(rng, E, H, I):
    """w2 weights that both formats hold exactly: 2^x * (c - 4) with c in
    0..7 and a -4 in every block (so both encoders take the scale 2^x)."""
    c = rng.integers(0, 8, size=(E * H, I))
    c[:, ::32] = 0
    x = rng.integers(-9, -5, size=(E * H, I // 32))
    w = (np.repeat(np.ldexp(1.0, x), 32, axis=1) * (c - 4.0)).astype(np.float32)
    qc, qs = synth.quant_q3(w)
    mc, ms = synth.quant_mxfp4(w)
    return (qc.reshape(E, H, -1), qs.reshape(E, H, -1), mc.reshape(E, H, I // 2), ms.reshape(E, H, I // 32), w)


def check_forward_w2q3_equals_mxfp4():
    """With the uniform code book and power-of-two scales the 3-bit w2 holds
    the same numbers as an MXFP4 w2; the two forwards must agree to the bit
    (same experts, same sums in the same order), for learned and hash
    routing, on a subset of rows."""
    rng = _rng(15)
    wl = synth.Workload("q3eq", T=12, H=64, E=8, k=3, I=64, V=30, seed=4)
    L = synth.make_layer(wl)
    qc, qs, mc, ms, w = _q3_equal_to_mxfp4(rng, wl.E, wl.H, wl.I)
    assert np.array_equal(oracle.q3_decode(qc[1], qs[1]), w[wl.H:2 * wl.H].astype(np.float64))
    Lm = synth.Layer(wl, L.gate_w, L.bias, L.logit_offset, L.w13_codes, L.w13_scales, mc, ms, L.sh_w13,
                     L.sh_w13_scale, L.sh_w2, L.sh_w2_scale, synth.tid2eid(1, 9, 0, wl.V, wl.E, wl.k))
    x = synth.make_tokens(wl, rep=2)
    rows = np.array([5, 0, 11, 3], np.int32)
    a = oracle.forward(Lm, x, rows=rows)
    b = oracle.forward_w2q3(Lm, qc, qs, None, x, rows=rows)
    assert len(set(a["ids"].ravel().tolist())) > 3
    assert np.array_equal(a["ids"], b["ids"]) and np.array_equal(a["out"], b["out"])
    tids = rng.integers(0, wl.V, size=wl.T).astype(np.int32)
    a = oracle.forward(Lm, x, token_ids=tids, rows=rows)
    b = oracle.forward_w2q3(Lm, qc, qs, None, x, token_ids=tids, rows=rows)
    assert np.array_equal(a["out"], b["out"])


def check_forward_w2q3_tables():
    """Per-expert tables: the layer against numpy's composition with each
    expert's w2 decoded in numpy from the encoder's inputs (the level nearest
    w / scale in that expert's own table, times the binary16 scale)."""
    rng = _rng(16)
    wl = synth.Workload("q3tab", T=8, H=64, E=6, k=3, I=64, V=30, seed=5)
    L = synth.make_layer(wl)
    E, H, I = wl.E, wl.H, wl.I
    tabs = synth.q3_tables(2, 13, 1, E)
    w = (rng.standard_normal((E * H, I)) * 0.05).astype(np.float32)
    qc, qs = synth.quant_q3(w, tables=tabs, rows_per_table=H)
    d = np.repeat(qs.view(np.float16).astype(np.float64), 32, axis=1)
    W2 = np.empty((E * H, I))
    for r in range(E * H):
        cand = d[r][:, None] * tabs[r // H].astype(np.float64)[None, :]
        W2[r] = cand[np.arange(I), np.abs(w[r].astype(np.float64)[:, None] - cand).argmin(axis=1)]
    W2 = W2.reshape(E, H, I)
    x = synth.make_tokens(wl, rep=1)
    rows = np.array([1, 6, 3], np.int32)
    r = oracle.forward_w2q3(L, qc.reshape(E, H, -1), qs.reshape(E, H, -1), tabs, x, rows=rows, round_h=False)
    xd = bf16_to_f64(x[rows])
    S13 = L.sh_w13.astype(np.float64) * L.sh_w13_scale.astype(np.float64)[:, None]
    S2 = L.sh_w2.astype(np.float64) * L.sh_w2_scale.astype(np.float64)[:, None]
    for i in range(len(rows)):
        out = np.zeros(H)
        for j, e in enumerate(r["ids"][i]):
            W13 = decode_mxfp4_table(L.w13_codes[e], L.w13_scales[e])
            h = np_swiglu(W13[:I] @ xd[i], W13[I:] @ xd[i])
            out += r["w"][i, j] * (W2[e] @ h)
        out += np_swiglu(S13[:I] @ xd[i], S13[I:] @ xd[i]) @ S2.T
        assert np.allclose(r["out"][i], out, rtol=1e-12, atol=1e-12 * np.abs(out).max()), i
    # the forward's experts and weights are those of the MXFP4 layer
    ref = oracle.forward(L, x, rows=rows, round_h=False)
    assert np.array_equal(ref["ids"], r["ids"]) and np.array_equal(ref["w"], r["w"])


ALL_CHECKS = [
    check_e2m1_codes, check_e8m0_bytes, check_mxfp4_layout, check_block_bytes, check_bf16_values,
    check_softplus_score, check_swiglu, check_topk_exhaustive, check_topk_random, check_fp32_decision,
    check_noaux_bias, check_weights_sum, check_hash_route, check_permute, check_expert_ffn,
    check_shared_ffn, check_linearity, check_special_case_dense, check_forward_tiny,
    check_forward_forced_ids, check_forward_hash, check_linear_w8a16, check_fp16_values, check_q3_codes,
    check_q3_values, check_q3_roundtrip, check_forward_w2q3_equals_mxfp4, check_forward_w2q3_tables,
]

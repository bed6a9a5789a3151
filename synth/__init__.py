"""Seeded synthetic workloads for the DeepSeek-V4-Flash MoE layer.

Only inputs are made here (see ``synth.c``): Gaussian weights and their MXFP4 /
int8 encodings, bf16 tokens, Zipf token ids and the token-id -> expert table.
Both the CPU oracle and the GPU library consume these arrays; neither shares
any arithmetic of the layer with this module.

Shapes and constants of the layer come from the checkpoint's ``config.json``
(page "deepseek-v4-mxfp4-int8 config.json": hidden_size 4096,
n_routed_experts 256, num_experts_per_tok 6, moe_intermediate_size 2048,
vocab_size 129280, initializer_range 0.02) and from the export design note
(page "DeepSeek-V4-Flash export design", section "Source configuration").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

# Counter streams: one per tensor kind, so each tensor is regenerable alone.
S_W13, S_W2, S_SH_W13, S_SH_W2, S_GATE, S_BIAS, S_OFFSET, S_TOKENS, S_TIDS, S_TID2EID = range(1, 11)
S_STACK_PERM = 11
S_W2Q3, S_Q3TAB = 12, 13  # routed w2 in 3-bit blocks, their per-expert tables
S_LINEAR = 14  # int8 attention projections (sub-sequence: the projection)  # per-layer expert order of a layer stack

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP, no fast-math)."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
           "-Wall", "-Werror", src, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        L.synth_u64.argtypes = [u64, u64, u64, u64]
        L.synth_u64.restype = u64
        L.synth_normal_at.argtypes = [u64, u64, u64, u64]
        L.synth_normal_at.restype = dbl
        L.synth_normal_f32.argtypes = [u64, u64, u64, dbl, dbl, i64, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, dbl, i64, vp]
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        L.synth_quant_mxfp4.argtypes = [vp, i64, i64, vp, vp]
        L.synth_mxfp4_normal.argtypes = [u64, u64, u64, dbl, i64, i64, vp, vp]
        L.synth_quant_int8.argtypes = [vp, i64, i64, vp, vp]
        L.synth_int8_normal.argtypes = [u64, u64, u64, dbl, i64, i64, vp, vp]
        L.synth_quant_q3.argtypes = [vp, i64, i64, vp, i64, vp, vp]
        L.synth_q3_normal.argtypes = [u64, u64, u64, dbl, i64, i64, vp, i64, vp, vp]
        L.synth_q3_tables.argtypes = [u64, u64, u64, i64, vp]
        L.synth_zipf_ids.argtypes = [u64, u64, u64, dbl, i64, i64, vp]
        L.synth_zipf_ids.restype = ctypes.c_int
        L.synth_tid2eid.argtypes = [u64, u64, u64, i64, i32, i32, vp]
        L.synth_tid2eid.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- primitives

def normal_f32(seed, stream, sub, n, sigma=1.0, mean=0.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(seed, stream, sub, mean, sigma, n, _p(out))
    return out


def normal_bf16(seed, stream, sub, n, sigma=1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32(sigma * N(0,1)), rounded to nearest even."""
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(seed, stream, sub, sigma, n, _p(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(_p(a), a.size, _p(out))
    return out


def quant_mxfp4(w: np.ndarray):
    """Encode fp32 ``w`` [..., K] as (codes uint8 [..., K/2], scales uint8 [..., K/32])."""
    w = np.ascontiguousarray(w, np.float32)
    K = w.shape[-1]
    assert K % 32 == 0
    rows = w.size // K
    codes = np.empty(w.shape[:-1] + (K // 2,), np.uint8)
    scales = np.empty(w.shape[:-1] + (K // 32,), np.uint8)
    lib().synth_quant_mxfp4(_p(w), rows, K, _p(codes), _p(scales))
    return codes, scales


def mxfp4_normal(seed, stream, sub, rows, K, sigma):
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    lib().synth_mxfp4_normal(seed, stream, sub, sigma, rows, K, _p(codes), _p(scales))
    return codes, scales


def quant_int8(w: np.ndarray):
    """Encode fp32 ``w`` [rows, K] as (int8 [rows, K], fp32 scale [rows])."""
    w = np.ascontiguousarray(w, np.float32)
    rows, K = w.shape
    q = np.empty((rows, K), np.int8)
    s = np.empty(rows, np.float32)
    lib().synth_quant_int8(_p(w), rows, K, _p(q), _p(s))
    return q, s


def int8_normal(seed, stream, sub, rows, K, sigma):
    q = np.empty((rows, K), np.int8)
    s = np.empty(rows, np.float32)
    lib().synth_int8_normal(seed, stream, sub, sigma, rows, K, _p(q), _p(s))
    return q, s


def _q3_tables_arg(tables, rows, rows_per_table):
    if tables is None:
        return None, 1
    tables = np.ascontiguousarray(tables, np.float32).reshape(-1, 8)
    if rows_per_table is None:
        rows_per_table = rows // tables.shape[0]
    if rows_per_table <= 0 or (rows - 1) // rows_per_table >= tables.shape[0]:
        raise ValueError("tables do not cover the rows")
    return tables, rows_per_table


def quant_q3(w: np.ndarray, tables=None, rows_per_table=None):
    """Encode fp32 ``w`` [rows, K] as 3-bit blocks: (codes uint8 [rows, K/32*12],
    scales uint16 [rows, K/32] binary16 bits). ``tables`` [n, 8] (row r uses
    table r // rows_per_table) or None for the uniform code book c - 4."""
    w = np.ascontiguousarray(w, np.float32)
    rows, K = w.shape
    assert K % 32 == 0
    t, rpt = _q3_tables_arg(tables, rows, rows_per_table)
    codes = np.empty((rows, K // 32 * 12), np.uint8)
    scales = np.empty((rows, K // 32), np.uint16)
    lib().synth_quant_q3(_p(w), rows, K, None if t is None else _p(t), rpt, _p(codes), _p(scales))
    return codes, scales


def q3_normal(seed, stream, sub, rows, K, sigma, tables=None, rows_per_table=None):
    t, rpt = _q3_tables_arg(tables, rows, rows_per_table)
    codes = np.empty((rows, K // 32 * 12), np.uint8)
    scales = np.empty((rows, K // 32), np.uint16)
    lib().synth_q3_normal(seed, stream, sub, sigma, rows, K, None if t is None else _p(t), rpt, _p(codes),
                          _p(scales))
    return codes, scales


def q3_tables(seed, stream, sub, n) -> np.ndarray:
    """n code books of 8 ascending fp32 levels."""
    out = np.empty((n, 8), np.float32)
    lib().synth_q3_tables(seed, stream, sub, n, _p(out))
    return out


def zipf_ids(seed, stream, sub, n, V, s=1.1) -> np.ndarray:
    out = np.empty(n, np.int32)
    if lib().synth_zipf_ids(seed, stream, sub, s, V, n, _p(out)) != 0:
        raise MemoryError("zipf table")
    return out


def tid2eid(seed, stream, sub, V, E, k) -> np.ndarray:
    out = np.empty((V, k), np.int32)
    if lib().synth_tid2eid(seed, stream, sub, V, E, k, _p(out)) != 0:
        raise ValueError("bad tid2eid shape")
    return out


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    """One synthetic MoE-layer workload (shapes, distributions, seed)."""
    name: str
    T: int
    H: int = 4096
    E: int = 256
    k: int = 6
    I: int = 2048
    V: int = 129280
    weight_sigma: float = 0.02       # initializer_range of config.json
    gate_sigma: float = 0.02
    bias_sigma: float = 0.01
    offset_sigma: float = 0.0        # per-expert logit offset (0 = none)
    hash_layer: bool = False         # token-id table routing instead of the learned router
    zipf_s: float = 1.1
    seed: int = 0
    routed_scaling_factor: float = 1.5
    swiglu_limit: float = 10.0

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS = {
    # tiny layer: T=16, hidden 256, 16 experts, top-6, intermediate 128
    "tiny": Workload("tiny", T=16, H=256, E=16, k=6, I=128, V=1000),
    # full-shape layer, single-token decode
    "decode_t1": Workload("decode_t1", T=1),
    # full-shape layer, 64-token batched decode with a mild expert skew
    "decode_t64": Workload("decode_t64", T=64, bias_sigma=0.05),
    # full-shape layer, 8192-token prefill with imbalanced expert loads
    "prefill_t8192": Workload("prefill_t8192", T=8192, offset_sigma=0.5),
    # full-shape hash-routed layer, 4096 Zipf tokens
    "hash_t4096": Workload("hash_t4096", T=4096, hash_layer=True),
    # the same layers with the routed w2 in 3-bit blocks (per-expert tables)
    "w2q3_t1": Workload("w2q3_t1", T=1),
    "w2q3_t64": Workload("w2q3_t64", T=64, bias_sigma=0.05),
    "w2q3_t8192": Workload("w2q3_t8192", T=8192, offset_sigma=0.5),
    # one token through the 43-layer stack (3 hash-routed layers, then learned-router layers)
    "stack43_t1": Workload("stack43_t1", T=1),
}


@dataclass
class Layer:
    """Host copies of one layer's parameters (numpy)."""
    wl: Workload
    gate_w: np.ndarray          # fp32 [E, H]
    bias: np.ndarray            # fp32 [E]   e_score_correction_bias
    logit_offset: np.ndarray | None  # fp32 [E] or None
    w13_codes: np.ndarray       # uint8 [E, 2I, H/2]
    w13_scales: np.ndarray      # uint8 [E, 2I, H/32]
    w2_codes: np.ndarray        # uint8 [E, H, I/2]
    w2_scales: np.ndarray       # uint8 [E, H, I/32]
    sh_w13: np.ndarray          # int8 [2I, H]
    sh_w13_scale: np.ndarray    # fp32 [2I]
    sh_w2: np.ndarray           # int8 [H, I]
    sh_w2_scale: np.ndarray     # fp32 [H]
    tid2eid: np.ndarray | None = None  # int32 [V, k]
    extra: dict = field(default_factory=dict)


def make_layer(wl: Workload) -> Layer:
    """All parameters of one layer. Expert e of w13/w2 is sub-sequence e."""
    s, H, E, I, k = wl.seed, wl.H, wl.E, wl.I, wl.k
    w13c = np.empty((E, 2 * I, H // 2), np.uint8)
    w13s = np.empty((E, 2 * I, H // 32), np.uint8)
    w2c = np.empty((E, H, I // 2), np.uint8)
    w2s = np.empty((E, H, I // 32), np.uint8)
    L = lib()
    for e in range(E):
        L.synth_mxfp4_normal(s, S_W13, e, wl.weight_sigma, 2 * I, H, _p(w13c[e]), _p(w13s[e]))
        L.synth_mxfp4_normal(s, S_W2, e, wl.weight_sigma, H, I, _p(w2c[e]), _p(w2s[e]))
    sh13, sh13s = int8_normal(s, S_SH_W13, 0, 2 * I, H, wl.weight_sigma)
    sh2, sh2s = int8_normal(s, S_SH_W2, 0, H, I, wl.weight_sigma)
    gate = normal_f32(s, S_GATE, 0, E * H, wl.gate_sigma).reshape(E, H)
    bias = normal_f32(s, S_BIAS, 0, E, wl.bias_sigma)
    off = normal_f32(s, S_OFFSET, 0, E, wl.offset_sigma) if wl.offset_sigma > 0 else None
    t2e = tid2eid(s, S_TID2EID, 0, wl.V, E, k) if wl.hash_layer else None
    return Layer(wl, gate, bias, off, w13c, w13s, w2c, w2s, sh13, sh13s, sh2, sh2s, t2e)


def make_w2q3(wl: Workload, tables: bool):
    """The routed experts' w2 in 3-bit blocks, N(0, weight_sigma^2) like the
    MXFP4 w2: (codes uint8 [E, H, I/32*12], scales uint16 [E, H, I/32]
    binary16 bits, levels fp32 [E, 8] or None for the uniform code book).
    Expert e is sub-sequence e; tables from stream S_Q3TAB."""
    E, H, I = wl.E, wl.H, wl.I
    lv = q3_tables(wl.seed, S_Q3TAB, 0, E) if tables else None
    codes = np.empty((E, H, I // 32 * 12), np.uint8)
    scales = np.empty((E, H, I // 32), np.uint16)
    L = lib()
    for e in range(E):
        L.synth_q3_normal(wl.seed, S_W2Q3, e, wl.weight_sigma, H, I, None if lv is None else _p(lv[e]), H,
                          _p(codes[e]), _p(scales[e]))
    return codes, scales, lv


def make_tokens(wl: Workload, rep: int = 0, T: int | None = None) -> np.ndarray:
    """bf16 bit patterns [T, H] of N(0,1) tokens; ``rep`` selects a fresh batch."""
    T = wl.T if T is None else T
    return normal_bf16(wl.seed, S_TOKENS, rep, T * wl.H).reshape(T, wl.H)


def make_token_ids(wl: Workload, rep: int = 0, T: int | None = None) -> np.ndarray:
    """int32 [T] token ids, Zipf(wl.zipf_s) over the vocabulary."""
    T = wl.T if T is None else T
    return zipf_ids(wl.seed, S_TIDS, rep, T, wl.V, wl.zipf_s)


# ---------------------------------------------------------------- layer stack

# The model's MoE layers: 43, the first 3 routed by the token-id table
# (page "DeepSeek-V4-Flash export design", section "Source configuration";
# page "deepseek-v4-mxfp4-int8 config.json", num_hidden_layers, num_hash_layers).
STACK_LAYERS, STACK_HASH_LAYERS = 43, 3


def stack_expert_order(l: int, E: int) -> np.ndarray:
    """Layer l's routed expert e is expert order[e] of the base layer: a
    seeded permutation (Fisher-Yates on SplitMix64 draws, stream S_STACK_PERM,
    sub-sequence l); layer 0 keeps the base order."""
    order = np.arange(E, dtype=np.int64)
    if l == 0:
        return order
    L = lib()
    for i in range(E - 1, 0, -1):
        j = int(L.synth_u64(0, S_STACK_PERM, l, i) % (i + 1))
        order[i], order[j] = order[j], order[i]
    return order


def make_stack_layer(base: Layer, l: int, n_hash: int = STACK_HASH_LAYERS, routed: bool = True) -> Layer:
    """Layer l of a stack built on ``base`` (its workload's shapes): routed
    experts = the base layer's experts in the seeded order of
    stack_expert_order (1/E of the generation cost per layer, every layer's
    expert tensors in their own memory); router weight, bias, shared expert
    and (layers below n_hash) the token-id table drawn fresh for the layer
    (sub-sequence l + 1 of their streams). Layers below n_hash are hash-routed.
    routed=False leaves the routed expert arrays out (None): the caller
    builds them from the base layer's device copy with the same order."""
    wl = base.wl
    s, H, E, I, k = wl.seed, wl.H, wl.E, wl.I, wl.k
    order = stack_expert_order(l, E)
    hash_layer = l < n_hash
    lw = replace(wl, name=f"{wl.name}_layer{l}", hash_layer=hash_layer)
    sh13, sh13s = int8_normal(s, S_SH_W13, l + 1, 2 * I, H, wl.weight_sigma)
    sh2, sh2s = int8_normal(s, S_SH_W2, l + 1, H, I, wl.weight_sigma)
    gate = normal_f32(s, S_GATE, l + 1, E * H, wl.gate_sigma).reshape(E, H)
    bias = normal_f32(s, S_BIAS, l + 1, E, wl.bias_sigma)
    t2e = tid2eid(s, S_TID2EID, l + 1, wl.V, E, k) if hash_layer else None
    pick = (lambda a: a[order]) if routed else (lambda a: None)
    return Layer(lw, gate, bias, None, pick(base.w13_codes), pick(base.w13_scales), pick(base.w2_codes),
                 pick(base.w2_scales), sh13, sh13s, sh2, sh2s, t2e, extra={"expert_order": order, "layer": l})

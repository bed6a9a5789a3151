"""CPU oracle of the DeepSeek-V4-Flash MoE layer (ctypes binding of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. The product (``mxfp4_moe_expert_amd``) never imports
it, and this module imports nothing from the product.

Every function computes the plain definition of its step in fp64 (see the
header of ``oracle.c`` for the passages of the pages each step follows); the
routing decision is taken on fp32 values, as the GPU takes it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False, src: str | None = None, out: str | None = None) -> str:
    """Compile ``liboracle.so`` with gcc: -O2, no FMA contraction, no fast-math."""
    import subprocess

    src = src or os.path.join(_HERE, "oracle.c")
    out = out or LIB_PATH
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
           "-Wall", "-Werror", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        _lib = _open(LIB_PATH)
    return _lib


def use_library(path: str | None):
    """Point this module at another build of ``oracle.c`` (None = the default).

    Used by the tests that plant a mistake in a copy of the oracle and check
    that the pins catch it."""
    global _lib
    _lib = None if path is None else _open(path)


def _open(path: str):
    L = ctypes.CDLL(path)
    i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    L.or_num_threads.argtypes = []
    L.or_num_threads.restype = i32
    L.or_e2m1.argtypes = [i32]
    L.or_e2m1.restype = dbl
    L.or_e8m0.argtypes = [i32]
    L.or_e8m0.restype = dbl
    L.or_mxfp4_weight.argtypes = [vp, vp, i64, i64, i64]
    L.or_mxfp4_weight.restype = dbl
    L.or_bf16_value.argtypes = [ctypes.c_uint16]
    L.or_bf16_value.restype = dbl
    L.or_round_bf16.argtypes = [dbl]
    L.or_round_bf16.restype = dbl
    L.or_block_bytes.argtypes = [i32, i32, i32]
    L.or_block_bytes.restype = i64
    for f in ("or_softplus", "or_score", "or_silu"):
        getattr(L, f).argtypes = [dbl]
        getattr(L, f).restype = dbl
    L.or_swiglu.argtypes = [dbl, dbl, dbl]
    L.or_swiglu.restype = dbl
    L.or_route.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, dbl, vp, vp, vp, vp]
    L.or_hash_route.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp, dbl, vp, vp]
    L.or_permute.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    L.or_expert_ffn.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, dbl, i32, vp]
    L.or_shared_ffn.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, dbl, i32, vp]
    L.or_forward.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                             vp, vp, vp, vp, dbl, dbl, i32, vp, i32, vp, vp, vp, vp, vp, vp]
    L.or_linear_w8a16.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
    L.or_fp16_value.argtypes = [ctypes.c_uint16]
    L.or_fp16_value.restype = dbl
    L.or_q3_code.argtypes = [vp, i32]
    L.or_q3_code.restype = i32
    L.or_q3_level.argtypes = [vp, i32]
    L.or_q3_level.restype = dbl
    L.or_q3_weight.argtypes = [vp, vp, vp, i64, i64, i64]
    L.or_q3_weight.restype = dbl
    L.or_forward_w2q3.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                  vp, vp, vp, vp, dbl, dbl, i32, vp, i32, vp, vp, vp, vp, vp, vp]
    for f in ("or_route", "or_hash_route", "or_permute", "or_expert_ffn", "or_shared_ffn",
              "or_forward", "or_forward_w2q3", "or_linear_w8a16"):
        getattr(L, f).restype = i32
    return L


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "contiguous numpy array expected"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


# ------------------------------------------------------------------ scalars

def e2m1(code: int) -> float:
    return lib().or_e2m1(code)


def e8m0(byte: int) -> float:
    return lib().or_e8m0(byte)


def bf16_value(bits: int) -> float:
    return lib().or_bf16_value(bits)


def round_bf16(v: float) -> float:
    return lib().or_round_bf16(v)


def block_bytes(bits: int, group: int, scale_bits: int) -> int:
    return lib().or_block_bytes(bits, group, scale_bits)


def softplus(z: float) -> float:
    return lib().or_softplus(z)


def score(logit: float) -> float:
    return lib().or_score(logit)


def silu(z: float) -> float:
    return lib().or_silu(z)


def swiglu(g: float, u: float, limit: float = 10.0) -> float:
    return lib().or_swiglu(g, u, limit)


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode a whole MXFP4 matrix [N, K] (fp64), one weight at a time."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((N, K), np.float64)
    f = lib().or_mxfp4_weight
    pc, ps = _p(codes), _p(scales)
    for n in range(N):
        for k in range(K):
            out[n, k] = f(pc, ps, K, n, k)
    return out


# ------------------------------------------------------------------ layer steps

def route(x, gate_w, bias, offset=None, k=6, scale=1.5):
    """Learned router. Returns (ids int32 [T,k], w fp64 [T,k], gap fp64 [T], next int32 [T])."""
    x = _c(x, np.uint16)
    gate_w = _c(gate_w, np.float32)
    bias = _c(bias, np.float32)
    offset = _c(offset, np.float32)
    T, H = x.shape
    E = gate_w.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    nxt = np.empty(T, np.int32)
    _check(lib().or_route(T, H, E, k, _p(x), _p(gate_w), _p(bias), _p(offset), scale, _p(ids), _p(w),
                          _p(gap), _p(nxt)), "route")
    return ids, w, gap, nxt


def hash_route(x, token_ids, tid2eid, gate_w, scale=1.5):
    x = _c(x, np.uint16)
    token_ids = _c(token_ids, np.int32)
    tid2eid = _c(tid2eid, np.int32)
    gate_w = _c(gate_w, np.float32)
    T, H = x.shape
    V, k = tid2eid.shape
    E = gate_w.shape[0]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check(lib().or_hash_route(T, H, E, k, _p(x), _p(token_ids), _p(tid2eid), V, _p(gate_w), scale,
                               _p(ids), _p(w)), "hash_route")
    return ids, w


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, np.int32)
    sorted_slots = np.empty(T * k, np.int32)
    slot_pos = np.empty(T * k, np.int32)
    _check(lib().or_permute(T, k, E, _p(ids), _p(offsets), _p(sorted_slots), _p(slot_pos)), "permute")
    return offsets, sorted_slots, slot_pos


def expert_ffn(x, ids, w, w13_codes, w13_scales, w2_codes, w2_scales, limit=10.0, round_h=True):
    """Routed experts only: sum_j w[t,j] * expert_{ids[t,j]}(x_t), fp64 [T, H]."""
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T, H = x.shape
    E, twoI = w13_codes.shape[0], w13_codes.shape[1]
    k = ids.shape[1]
    out = np.empty((T, H), np.float64)
    _check(lib().or_expert_ffn(T, H, E, k, twoI // 2, _p(x), _p(ids), _p(w), _p(_c(w13_codes, np.uint8)),
                               _p(_c(w13_scales, np.uint8)), _p(_c(w2_codes, np.uint8)),
                               _p(_c(w2_scales, np.uint8)), limit, int(round_h), _p(out)), "expert_ffn")
    return out


def shared_ffn(x, q13, s13, q2, s2, limit=10.0, round_h=True):
    x = _c(x, np.uint16)
    T, H = x.shape
    I = q13.shape[0] // 2
    z = np.empty((T, H), np.float64)
    _check(lib().or_shared_ffn(T, H, I, _p(x), _p(_c(q13, np.int8)), _p(_c(s13, np.float32)),
                               _p(_c(q2, np.int8)), _p(_c(s2, np.float32)), limit, int(round_h), _p(z)),
           "shared_ffn")
    return z


def forward(layer, x, token_ids=None, rows=None, force_ids=None, round_h=True):
    """Whole layer for the tokens in ``rows`` (all if None).

    ``layer`` is a ``synth.Layer`` (or any object with the same fields).
    Returns dict(ids, w, gap, next, out) with one row per requested token.
    """
    wl = layer.wl
    x = _c(x, np.uint16)
    T, H = x.shape
    E, k, I = wl.E, wl.k, wl.I
    rows_a = None if rows is None else _c(rows, np.int32)
    n = T if rows_a is None else len(rows_a)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    gap = np.empty(n, np.float64)
    nxt = np.empty(n, np.int32)
    out = np.empty((n, H), np.float64)
    tids = _c(token_ids, np.int32)
    t2e = _c(layer.tid2eid, np.int32) if tids is not None else None
    V = t2e.shape[0] if t2e is not None else 0
    _check(lib().or_forward(
        T, H, E, k, I, _p(x), _p(layer.gate_w), _p(layer.bias), _p(layer.logit_offset), _p(tids), _p(t2e), V,
        _p(layer.w13_codes), _p(layer.w13_scales), _p(layer.w2_codes), _p(layer.w2_scales),
        _p(layer.sh_w13), _p(layer.sh_w13_scale), _p(layer.sh_w2), _p(layer.sh_w2_scale),
        wl.routed_scaling_factor, wl.swiglu_limit, int(round_h), _p(rows_a), n,
        _p(_c(force_ids, np.int32)), _p(ids), _p(w), _p(gap), _p(nxt), _p(out)), "forward")
    return dict(ids=ids, w=w, gap=gap, next=nxt, out=out)


def fp16_value(bits: int) -> float:
    return lib().or_fp16_value(bits)


def q3_code(block: np.ndarray, i: int) -> int:
    """3-bit code of weight i of one 12-byte block."""
    b = _c(block, np.uint8)
    assert b.size == 12
    return lib().or_q3_code(_p(b), i)


def q3_decode(codes: np.ndarray, scales: np.ndarray, levels=None) -> np.ndarray:
    """Decode a whole 3-bit matrix [N, K] (fp64), one weight at a time:
    codes [N, K/32*12] u8, scales [N, K/32] binary16 bits, levels [8] or None."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    lv = _c(levels, np.float32)
    N, K = scales.shape[0], scales.shape[1] * 32
    assert codes.shape == (N, K // 32 * 12)
    out = np.empty((N, K), np.float64)
    f = lib().or_q3_weight
    pc, ps, pl = _p(codes), _p(scales), _p(lv)
    for n in range(N):
        for k in range(K):
            out[n, k] = f(pc, ps, pl, K, n, k)
    return out


def forward_w2q3(layer, w2_codes, w2_scales, w2_levels, x, token_ids=None, rows=None, force_ids=None,
                 round_h=True):
    """``forward`` with the routed experts' w2 in 3-bit blocks: w2_codes
    [E, H, I/32*12] u8, w2_scales [E, H, I/32] binary16 bits, w2_levels
    [E, 8] fp32 or None (uniform). ``layer``'s own w2 is not used."""
    wl = layer.wl
    x = _c(x, np.uint16)
    T, H = x.shape
    E, k, I = wl.E, wl.k, wl.I
    c2 = _c(w2_codes, np.uint8)
    s2 = _c(w2_scales, np.uint16)
    lv = _c(w2_levels, np.float32)
    assert c2.size == E * H * (I // 32) * 12 and s2.size == E * H * (I // 32)
    assert lv is None or lv.size == E * 8
    rows_a = None if rows is None else _c(rows, np.int32)
    n = T if rows_a is None else len(rows_a)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    gap = np.empty(n, np.float64)
    nxt = np.empty(n, np.int32)
    out = np.empty((n, H), np.float64)
    tids = _c(token_ids, np.int32)
    t2e = _c(layer.tid2eid, np.int32) if tids is not None else None
    V = t2e.shape[0] if t2e is not None else 0
    _check(lib().or_forward_w2q3(
        T, H, E, k, I, _p(x), _p(layer.gate_w), _p(layer.bias), _p(layer.logit_offset), _p(tids), _p(t2e), V,
        _p(layer.w13_codes), _p(layer.w13_scales), _p(c2), _p(s2), _p(lv),
        _p(layer.sh_w13), _p(layer.sh_w13_scale), _p(layer.sh_w2), _p(layer.sh_w2_scale),
        wl.routed_scaling_factor, wl.swiglu_limit, int(round_h), _p(rows_a), n,
        _p(_c(force_ids, np.int32)), _p(ids), _p(w), _p(gap), _p(nxt), _p(out)), "forward_w2q3")
    return dict(ids=ids, w=w, gap=gap, next=nxt, out=out)


def linear_w8a16(x, q, s, groups=1):
    """int8 per-channel linear (grouped if groups > 1): x [T][groups*K] bf16,
    q [groups*N][K] int8 (group g's rows g*N .. g*N+N-1), s [groups*N] fp32
    -> out [T][groups*N] fp64."""
    x = _c(x, np.uint16)
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    T = x.shape[0]
    K = x.shape[1] // groups
    N = q.shape[0] // groups
    assert q.shape == (groups * N, K) and s.shape == (groups * N,)
    out = np.empty((T, groups * N), np.float64)
    _check(lib().or_linear_w8a16(T, K, N, groups, _p(x), _p(q), _p(s), _p(out)), "linear_w8a16")
    return out

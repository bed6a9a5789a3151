"""Comparison of the GPU layer with the CPU oracle, at the bar the layer is
held to:

  * expert selections equal as sets, except at near-ties, where the k-th and
    (k+1)-th biased scores (oracle, fp32) differ by less than NEAR_TIE; such
    tokens are counted, and a differing set must be the oracle's set with its
    k-th expert swapped for the best unchosen one;
  * routing weights within W_TOL of the oracle's, per expert id;
  * outputs within relative L2 REL_L2 and max abs MAX_ABS_FRAC * rms(oracle).

The tolerance derivation: the GPU sums in fp32 (MFMA) and rounds the
intermediate activation to bf16, like the oracle; the remaining differences
are fp32 summation order (~1e-6 relative) and one-ulp bf16 flips of h
(2^-8 relative on a few elements), both far inside the bar.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_L2 = 5e-3
MAX_ABS_FRAC = 2e-2
NEAR_TIE = 1e-5
W_TOL = 1e-5


def compare_routing(gpu_ids, gpu_w, ora_ids, ora_w, ora_gap, ora_next):
    """Returns dict(near_ties, swapped, alt_rows={row: alt_ids}); raises on a real mismatch."""
    gpu_ids = np.asarray(gpu_ids)
    gpu_w = np.asarray(gpu_w, np.float64)
    T, k = ora_ids.shape
    near = 0
    alt_rows = {}
    for t in range(T):
        gs, os_ = set(gpu_ids[t].tolist()), set(ora_ids[t].tolist())
        if ora_gap[t] < NEAR_TIE:
            near += 1
        if gs == os_:
            gw = dict(zip(gpu_ids[t].tolist(), gpu_w[t].tolist()))
            for e, w in zip(ora_ids[t].tolist(), ora_w[t].tolist()):
                assert abs(gw[e] - w) <= W_TOL, f"token {t}: weight of expert {e}: gpu {gw[e]} oracle {w}"
            continue
        assert ora_gap[t] < NEAR_TIE, (
            f"token {t}: gpu experts {sorted(gs)} != oracle {sorted(os_)} (gap {ora_gap[t]:.3g})")
        alt = list(ora_ids[t])
        alt[k - 1] = int(ora_next[t])
        assert gs == set(alt), f"token {t}: near-tie set {sorted(gs)} is not the one-swap alternative"
        alt_rows[t] = np.array(alt, np.int32)
    return dict(near_ties=near, swapped=len(alt_rows), alt_rows=alt_rows)


def output_errors(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    d = gpu - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    return dict(rel_l2=float(rel), max_abs=float(np.abs(d).max()) if d.size else 0.0, rms=float(rms))


def assert_outputs_close(gpu, ref, what=""):
    e = output_errors(gpu, ref)
    assert e["rel_l2"] <= REL_L2, f"{what}: rel L2 {e['rel_l2']:.3g} > {REL_L2}"
    assert e["max_abs"] <= MAX_ABS_FRAC * e["rms"], (
        f"{what}: max abs {e['max_abs']:.3g} > {MAX_ABS_FRAC} * rms {e['rms']:.3g}")
    return e


def reference_rows(layer, x, rows, token_ids=None, routing=None, fwd=None):
    """Oracle outputs for ``rows``; rows whose GPU selection was a near-tie swap
    are recomputed by the oracle with its own one-swap alternative. ``fwd``
    replaces ``oracle.forward`` (same keyword arguments)."""
    fwd = fwd or oracle.forward
    r = fwd(layer, x, token_ids=token_ids, rows=np.asarray(rows, np.int32))
    out = r["out"]
    if routing is not None:
        for i, t in enumerate(rows):
            if int(t) in routing["alt_rows"]:
                alt = routing["alt_rows"][int(t)][None, :]
                r2 = fwd(layer, x, rows=np.array([t], np.int32), force_ids=alt)
                out[i] = r2["out"][0]
    return r, out


def bf16_bits_to_f64(bits):
    bits = np.asarray(bits).view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(a):
    """Round-to-nearest-even fp32 -> bf16 bit patterns (numpy, finite values)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)

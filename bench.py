#!/usr/bin/env python3
"""Throughput of one full-shape DeepSeek-V4-Flash MoE layer on one MI355X.

A step is one moe_forward call (route, permute, routed MXFP4 experts, int8
shared expert, combine) over one batch of T fresh seeded bf16 tokens, with
every input already resident in HBM. Default workload: single-token decode
(T=1) on the full-shape layer (hidden 4096, 256 experts, top-6, intermediate
2048, MXFP4 routed experts, int8 shared expert), 1000 timed steps after 50
warm-up steps. The weights are replicated ``--copies`` times and the steps
rotate through the copies, so the 256 MB last-level cache cannot keep the
shared expert and router warm from one step to the next.

Prints one JSON line: the throughput (tokens/s), the roofline of the dominant
kernel (its duration measured with HIP events on the launch stream over the
timed region), and the CPU oracle's rate on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at T=1/64/8192; % of HBM BW (decode) / bf16 MFMA peak"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published (5.0 PFLOP/s): the block-scaled fp8 x fp4 rate

DEFAULTS = {  # workload: steps, warmup, copies, dominant kernel (event slot), bound
    "decode_t1": (1000, 50, 12, "routed_w13", "hbm"),
    "decode_t64": (200, 20, 12, "routed_w13", "hbm"),
    "prefill_t8192": (20, 3, 1, "routed_w13", "mfma"),
    "hash_t4096": (20, 3, 1, "routed_w13", "mfma"),
    "stack43_t1": (100, 5, 1, "routed_w13", "hbm"),
    "w2q3_t1": (1000, 50, 12, "routed_w13", "hbm"),
    "w2q3_t64": (200, 20, 12, "routed_w13", "hbm"),
    "w2q3_t8192": (20, 3, 1, "routed_w2", "mfma"),
}
# The kernel that runs in the routed-w13 slot of each schedule, as rocprofv3
# names it, what it does there, and which algorithmic work it is priced on.
DOMINANT = {
    "decode_t1": ("moe::k_layer_small<4, 2, 1, 6, false>",
                  "the whole layer in one launch of one block per CU: router, shared int8 w13, top-6, routed "
                  "MXFP4 w13 + clamped SwiGLU, routed MXFP4 + shared int8 w2 and the weighted combine", "layer"),
    "decode_t64": ("moe::k_stream_fused<8, 4, false>",
                   "both expert stages in one launch: routed MXFP4 + shared int8 w13 with the clamped SwiGLU, "
                   "then routed MXFP4 (x routing weight) + shared int8 w2", "experts"),
    "prefill_t8192": ("moe::k_gemm<0, 0>", "routed w13: MXFP4 grouped GEMM on bf16 MFMA + clamped SwiGLU", "w13"),
    "hash_t4096": ("moe::k_gemm<0, 0>", "routed w13: MXFP4 grouped GEMM on bf16 MFMA + clamped SwiGLU", "w13"),
    "stack43_t1": ("moe::k_layer_stack<4, 2, 1, 6>",
                   "the 43-layer stack (three hash-routed layers, then learned-router layers), up to eight "
                   "single-launch layers per launch, each handing its output rows to the next inside the launch",
                   "layer"),
    "w2q3_t1": ("moe::k_layer_small<4, 2, 1, 6, true>",
                "the whole layer in one launch of one block per CU, the routed w2 in 3-bit blocks (14 B per 32 "
                "weights, per-expert tables)", "layer"),
    "w2q3_t64": ("moe::k_stream_fused<8, 4, true>",
                 "both expert stages in one launch, the routed w2 in 3-bit blocks (14 B per 32 weights, "
                 "per-expert tables)", "experts"),
    "w2q3_t8192": ("moe::k_gemm<2, 1>",
                   "routed w2 in 3-bit blocks (per-expert tables): grouped GEMM on bf16 MFMA, x routing weight",
                   "w2"),
}
# with --prefill-mfma block-scaled (moe_set_option MOE_OPTION_PREFILL_BLOCK_SCALED)
DOMINANT_MX = ("moe::k_gemm_mx<0>",
               "routed w13: MXFP4 grouped GEMM on the block-scaled fp8 x fp4 MFMA (activations split exactly into "
               "hi/lo fp8) + clamped SwiGLU", "w13")


def dominant(workload: str):
    if workload in ("prefill_t8192", "hash_t4096") and PREFILL_MX[0]:
        return DOMINANT_MX
    return DOMINANT[workload]


PREFILL_MX = [False]
COPY_CAL_BYTES = 1 << 28  # the plain copy whose counters calibrate FETCH_SIZE / WRITE_SIZE


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(DEFAULTS),
                    help="all (default): decode_t1 as the headline line, the other workloads under 'workloads'")
    ap.add_argument("--copies", type=int, default=None, help="weight copies rotated through")
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"],
                    help="graph: steps captured in HIP graphs and replayed; eager: one launch sequence per step")
    ap.add_argument("--graph-steps", type=int, default=50, help="steps per captured graph")
    ap.add_argument("--prefill-mfma", default="bf16", choices=["bf16", "block-scaled"],
                    help="routed GEMMs above 64 tokens: bf16 MFMA (default) or the block-scaled fp8 x fp4 MFMA")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample (headline)")
    ap.add_argument("--extra-cpu-seconds", type=float, default=3.0,
                    help="budget of the CPU oracle sample of each further workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--linears", action="store_true",
                    help="also time the int8 attention projections (always with --workload all)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--peaks", action="store_true",
                    help="measure a 1 GiB device copy and a bf16 matmul (denominators beside the published peaks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of %d bytes 5 times (the counters' calibration)"
                    % COPY_CAL_BYTES)
    ap.add_argument("--summarize", metavar="OUTDIR", default=None,
                    help="write the profiles/ summaries of --workload from the rocprofv3 output under OUTDIR "
                    "(kernel_trace/, pmc_read/, pmc_write/, copy_read/, copy_write/) and exit")
    ap.add_argument("--commands", default=None, help="with --summarize: JSON file of the commands that ran")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the benchmark makes itself (events)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        # hipEventDisableSystemFence: a timing-only event; recording it does not
        # write back and invalidate the caches, so it does not perturb the kernel
        ev = ctypes.c_void_p()
        if self.L.hipEventCreateWithFlags(ctypes.byref(ev), 0x20000000) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.L.hipEventDestroy(ev)


def algorithmic(wl, ids_np, w2q3=False):
    """Per-step algorithmic work of the layer and of the routed w13 kernel.

    Bytes: every distinct routed expert's MXFP4 codes + scales (w13 and w2),
    the shared expert's int8 weights + scales, the router weight and bias,
    the tokens in and the output out. Flops: 2 per multiply-add of the
    expert GEMMs (routed slots and shared expert), router separately."""
    H, I, E, k = wl.H, wl.I, wl.E, wl.k
    w13_exp = 2 * I * (H // 2) + 2 * I * (H // 32)
    # routed w2: MXFP4 (16 B of codes + 1 B E8M0 per 32) or 3-bit blocks (12 B + 2 B per 32)
    w2_exp = H * (I // 32) * 14 if w2q3 else H * (I // 2) + H * (I // 32)
    shared = 2 * I * H + 2 * I * 4 + H * I + H * 4
    router = E * H * 4 + E * 4
    T = ids_np.shape[1]
    D = [len(set(s.ravel().tolist())) for s in ids_np]
    Dm = sum(D) / len(D)
    slots = T * k
    layer_bytes = Dm * (w13_exp + w2_exp) + shared + router + T * H * 2 + T * H * 2
    w13_bytes = Dm * w13_exp + slots * H * 2 + slots * I * 2  # weights + gathered x + h out
    # both expert stages: weights + gathered x + h out and back in + weighted y out (fp32)
    experts_bytes = (Dm * (w13_exp + w2_exp) + shared + (slots + T) * H * 2 + 2 * (slots + T) * I * 2
                     + (slots + T) * H * 4)
    flops_w13 = 2.0 * slots * H * 2 * I
    flops_w2 = 2.0 * slots * I * H
    w2_bytes = Dm * w2_exp + slots * I * 2 + slots * H * 2  # weights + h in + weighted y out (bf16)
    flops = 2.0 * slots * (H * 2 * I + I * H) + 2.0 * T * (H * 2 * I + I * H)
    return dict(distinct_experts=Dm, layer_bytes=layer_bytes, w13_bytes=w13_bytes, w13_flops=flops_w13,
                w2_bytes=w2_bytes, w2_flops=flops_w2,
                experts_bytes=experts_bytes,
                layer_flops=flops, router_flops=2.0 * T * E * H)


# Source file of each dominant kernel; its traffic record is keyed on this
# file, the library headers it includes and the launcher (api.cpp, which sets
# its launch configuration), so that a change elsewhere keeps the record.
KERNEL_SOURCE = {"k_layer_small": "fused.hip", "k_stream_fused": "stream.hip", "k_gemm": "gemm.hip",
                 "k_gemm_mx": "gemm_mx.hip"}


def kernel_files(workload: str):
    csrc = os.path.join(ROOT, "mxfp4_moe_expert_amd", "csrc")
    short = dominant(workload)[0].split("::")[1].split("<")[0]
    todo, seen = [KERNEL_SOURCE[short], "api.cpp"], set()
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        with open(os.path.join(csrc, f)) as fh:
            for line in fh:
                m = re.match(r'\s*#include\s+"([^"]+)"', line)
                if m and os.path.exists(os.path.join(csrc, m.group(1))):
                    todo.append(m.group(1))
    return sorted(seen)


def source_hash(workload: str) -> str:
    """Hash of the dominant kernel's sources (kernel_files)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp4_moe_expert_amd", "csrc")
    for f in kernel_files(workload):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch of the dominant kernel from committed counter
    summaries, if they were taken on the current kernel sources."""
    short = dominant(workload)[0].split("::")[1].split("<")[0]
    p = os.path.join(ROOT, "profiles", f"{short}_{workload}_traffic.txt")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(workload):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration():
    """A plain device-to-device copy of COPY_CAL_BYTES, five times: under
    rocprofv3 --pmc its FETCH_SIZE and WRITE_SIZE per dispatch calibrate the
    counters against a known number of bytes read and written."""
    import torch

    src = torch.ones(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    ok = bool(torch.equal(dst[:4096], src[:4096]))
    print(json.dumps({"copy_bytes": COPY_CAL_BYTES, "dispatches": 5, "ok": ok}), flush=True)


def measured_peaks():
    """What plain work reaches on this GPU, as denominators beside the
    published peaks: a 1 GiB device copy (HBM GB/s, read + write bytes), a
    1 GiB read with the library's streaming-read kernel (read bytes; the
    decode paths only read; the best of four grid sizes) and a bf16 8192^3
    matmul (TFLOP/s), each the median of 20 runs timed with events."""
    import mxfp4_moe_expert_amd as mx
    import torch

    def timed(fn, n=20):
        ts = []
        for _ in range(3):
            fn()
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    nb = 1 << 30
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms_copy = timed(lambda: dst.copy_(src))
    del src, dst
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    read_grid = {g: timed(lambda: mx.read_probe(src, g, sink)) for g in (2048, 4096, 8192, 16384)}
    ms_read = min(read_grid.values())
    del src, sink
    n = 8192
    x = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    ms_mm = timed(lambda: torch.matmul(x, y))
    rec = {"copy_bytes_moved": 2 * nb, "copy_ms": round(ms_copy, 4),
           "copy_GBps": round(2 * nb / (ms_copy / 1e3) / 1e9, 1),
           "read_bytes": nb, "read_ms": round(ms_read, 4), "read_GBps": round(nb / (ms_read / 1e3) / 1e9, 1),
           "read_GBps_by_blocks": {str(g): round(nb / (ms / 1e3) / 1e9, 1) for g, ms in read_grid.items()},
           "matmul_bf16_n": n, "matmul_ms": round(ms_mm, 4),
           "matmul_TFLOPs": round(2.0 * n ** 3 / (ms_mm / 1e3) / 1e12, 1),
           "published": {"hbm_GBps": PEAK_HBM_GBS, "bf16_TFLOPs": PEAK_BF16_TFLOPS}}
    print(json.dumps(rec), flush=True)


def _csv_rows(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(outdir, sub, name):
    d = os.path.join(outdir, sub)
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(name):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{name} under {d}")


def _counter_avg(path, counter, match):
    """Mean counter value per dispatch of the kernels whose name holds
    `match`."""
    vals = [float(r["Counter_Value"]) for r in _csv_rows(path)
            if r["Counter_Name"] == counter and match in r["Kernel_Name"]]
    if not vals:
        raise ValueError(f"no {counter} rows for {match} in {path}")
    return sum(vals) / len(vals), len(vals)


# rocprofv3 counter passes (one --pmc run each; at most 4 TCC counters per run)
PMC_READ = ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"]
PMC_WRITE = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
             "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]


def _read_bytes(path, match):
    n = {c: _counter_avg(path, c, match)[0] for c in PMC_READ}
    b = 32 * n["TCC_EA0_RDREQ_32B_sum"] + 64 * n["TCC_EA0_RDREQ_64B_sum"] + 128 * n["TCC_EA0_RDREQ_128B_sum"]
    return b, n


def _write_bytes(path, match):
    n = {c: _counter_avg(path, c, match)[0] for c in PMC_WRITE}
    w64 = n["TCC_EA0_WRREQ_64B_sum"]
    return 32 * (n["TCC_EA0_WRREQ_sum"] - w64) + 64 * w64, n


# Algorithmic flops of the grouped-GEMM launches of the large-batch schedule,
# by the template arguments rocprofv3 prints (<format, mode>: format 0 MXFP4,
# 1 int8, 2 3-bit; mode 0 w13 + SwiGLU, 1 routed w2, 2 shared w2 + combine)
# and the learned router's MFMA launch (three bf16 planes: 3x executed).
def _gemm_flops(kernel, wl):
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    m = re.search(r"k_gemm<(\d), (\d)>", kernel)
    if m:
        fmt, mode = int(m.group(1)), int(m.group(2))
        rows = T * k if fmt != 1 else T  # routed slots or tokens (shared expert)
        return 2.0 * rows * H * 2 * I if mode == 0 else 2.0 * rows * I * H
    if "k_router_mfma" in kernel:
        return 2.0 * T * E * H
    return None


def per_kernel_counters(workload, outdir, r_fac, w_fac, stats, commands):
    """profiles/<workload>_counters_per_kernel.md: for every library kernel of
    the counter runs, the mean per dispatch of MfmaUtil, executed bf16 MFMA
    flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), LDS bank-conflict and active
    cycles and HBM bytes (EA request counts by size, copy-calibrated), with
    the kernel-trace duration and, for the grouped GEMMs and the router, the
    algorithmic TFLOP/s and its fraction of the 2.5 PFLOP/s bf16 peak."""
    import synth

    wl = synth.WORKLOADS[workload]
    rd = _csv_rows(_find(outdir, "pmc_read", "counter_collection.csv"))
    wr = _csv_rows(_find(outdir, "pmc_write", "counter_collection.csv"))
    vals = {}
    for rows in (rd, wr):
        for r in rows:
            if "moe::" in r["Kernel_Name"]:
                vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    dur = {}
    for r in stats or []:
        dur[r["Name"]] = float(r["AverageNs"]) / 1e3
    lines = [f"# Counters per kernel, moe_forward, workload {workload}", "",
             "Mean per dispatch. HBM bytes: 32/64/128-byte EA read requests and 32/64-byte write requests, "
             f"each scaled by what the same counters read for a copy of {COPY_CAL_BYTES} bytes "
             f"(read factor {r_fac:.4f}, write factor {w_fac:.4f}). Executed bf16 flops count every MFMA "
             "the kernel issued (the router's three planes, padded tile positions); algorithmic flops are "
             "the layer's own (2 per multiply-add of the routed slots or tokens).", "",
             "Commands:", "", "```"] + [commands[c] for c in ("pmc_read", "pmc_write", "kernel_trace") if c in commands] + [
             "```", "",
             "| kernel | dispatches | us (trace) | MfmaUtil % | executed bf16 TFLOP/s | algorithmic TFLOP/s | "
             "frac of 2.5 PF | LDS conflict cycles | LDS active cycles | HBM read MB | HBM write MB |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    order = sorted(vals, key=lambda k: -dur.get(k, 0.0))
    for kname in order:
        v = {c: sum(x) / len(x) for c, x in vals[kname].items()}
        n = len(vals[kname].get("MfmaUtil", vals[kname][next(iter(vals[kname]))]))
        us = dur.get(kname)
        rb = (32 * v.get("TCC_EA0_RDREQ_32B_sum", 0) + 64 * v.get("TCC_EA0_RDREQ_64B_sum", 0)
              + 128 * v.get("TCC_EA0_RDREQ_128B_sum", 0)) * r_fac
        w64 = v.get("TCC_EA0_WRREQ_64B_sum", 0)
        wb = (32 * (v.get("TCC_EA0_WRREQ_sum", 0) - w64) + 64 * w64) * w_fac
        ex = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) * 512.0
        alg = _gemm_flops(kname, wl)
        name = kname.split("(")[0].replace("void ", "")
        cells = [f"`{name}`", str(n), f"{us:.1f}" if us else "-", f"{v.get('MfmaUtil', 0):.1f}",
                 f"{ex / (us * 1e6):.1f}" if us and ex else "-",
                 f"{alg / (us * 1e6):.1f}" if us and alg else "-",
                 f"{alg / (us * 1e-6) / (PEAK_BF16_TFLOPS * 1e12):.3f}" if us and alg else "-",
                 f"{v.get('SQ_LDS_BANK_CONFLICT', 0):.0f}", f"{v.get('SQ_LDS_IDX_ACTIVE', 0):.0f}",
                 f"{rb / 1e6:.1f}", f"{wb / 1e6:.1f}"]
        lines.append("| " + " | ".join(cells) + " |")
    with open(os.path.join(ROOT, "profiles", f"{workload}_counters_per_kernel.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize(workload, outdir, commands):
    """Turn one workload's rocprofv3 runs into the committed summaries:
    profiles/moe_forward_<workload>_kernels.md (per-kernel durations) and,
    when the counter runs exist, profiles/<kernel>_<workload>_traffic.txt:
    HBM bytes per launch of the dominant kernel from the EA request counts by
    size (32/64/128-byte reads, 32/64-byte writes), each scaled by what the
    same counters read for a plain copy of known size; MFMA busy fraction,
    executed bf16 MFMA flops and LDS bank-conflict cycles; stamped with the
    hash of the kernel sources."""
    kname, what, _ = dominant(workload)
    short = kname.split("::")[1].split("<")[0]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    try:
        stats = _csv_rows(_find(outdir, "kernel_trace", "kernel_stats.csv"))
    except FileNotFoundError:
        stats = None
    if stats is not None:
        lines = [f"# Kernel durations, moe_forward, workload {workload}", "",
                 f"Source hash of the dominant kernel ({', '.join(kernel_files(workload))}): "
                 f"`{source_hash(workload)}`", "",
                 "Command:", "", "```", commands.get("kernel_trace", "?"), "```", "",
                 f"Dominant kernel: `{kname}` ({what}).", "",
                 "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
        for r in stats:
            nm = r["Name"]
            if len(nm) > 90:
                nm = nm[:87] + "..."
            lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.2f}% |")
        tag = workload + ("_block_scaled" if PREFILL_MX[0] else "")
        with open(os.path.join(ROOT, "profiles", f"moe_forward_{tag}_kernels.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    try:
        rb, rn = _read_bytes(_find(outdir, "pmc_read", "counter_collection.csv"), kname)
        wb, wn = _write_bytes(_find(outdir, "pmc_write", "counter_collection.csv"), kname)
        crb, crn = _read_bytes(_find(outdir, "copy_read", "counter_collection.csv"), "__amd_rocclr_copyBuffer")
        cwb, cwn = _write_bytes(_find(outdir, "copy_write", "counter_collection.csv"), "__amd_rocclr_copyBuffer")
    except (FileNotFoundError, ValueError) as e:
        print(f"no traffic summary: {e}")
        return
    r_fac = COPY_CAL_BYTES / crb
    w_fac = COPY_CAL_BYTES / cwb
    rec = {
        "workload": workload, "kernel": kname, "source_hash": source_hash(workload),
        "source_files": kernel_files(workload),
        "read_requests": {k: round(v, 1) for k, v in rn.items()},
        "write_and_compute": {k: round(v, 3) for k, v in wn.items()},
        "read_bytes_counted": int(rb), "write_bytes_counted": int(wb),
        "copy_bytes": COPY_CAL_BYTES,
        "copy_read_requests": {k: round(v, 1) for k, v in crn.items()},
        "copy_write_requests": {k: round(v, 1) for k in ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")
                                for v in [cwn[k]]},
        "copy_read_bytes_counted": int(crb), "copy_write_bytes_counted": int(cwb),
        "read_factor": round(r_fac, 4), "write_factor": round(w_fac, 4),
        "bytes_per_launch": int(round(rb * r_fac + wb * w_fac)),
        "mfma_busy_pct": round(wn["MfmaUtil"], 2),
        "mfma_bf16_flops_executed": wn["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
        "lds_bank_conflict_cycles": wn["SQ_LDS_BANK_CONFLICT"],
        "lds_active_cycles": wn["SQ_LDS_IDX_ACTIVE"],
        "commands": {k: v for k, v in commands.items() if k != "kernel_trace"},
    }
    with open(os.path.join(ROOT, "profiles", f"{short}_{workload}_traffic.txt"), "w") as f:  # short names the kernel
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    per_kernel_counters(workload, outdir, r_fac, w_fac, stats, commands)


def cpu_leg(layer, batches, tids, budget_s, gpu_out32, gpu_ids, fwd=None):
    """The CPU-oracle leg of one workload: time the oracle, as it stands, on a
    bounded sample of the workload's batches (whole batches at T <= 64,
    sampled rows above), and grade the GPU's first batch against it: routing
    of every token of that batch (sets equal except near-ties, counted) and
    the fp32 outputs of the sampled rows (relative L2, max abs / rms)."""
    import numpy as np

    import oracle

    fwd = fwd or oracle.forward
    threads = oracle.lib().or_num_threads()
    T = batches[0].shape[0]
    rows = None if T <= 64 else np.unique(np.linspace(0, T - 1, 16).astype(np.int32))
    done_tokens, t0, i = 0, time.perf_counter(), 0
    first = None
    while True:
        xb = batches[i % len(batches)]
        tb = None if tids is None else tids[i % len(tids)]
        r = fwd(layer, xb, token_ids=tb, rows=rows)
        if i == 0:
            first = r
        done_tokens += T if rows is None else len(rows)
        i += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    sample = (f"{done_tokens} tokens: {i} batch(es) of T={T}" +
              ("" if rows is None else f", {len(rows)} evenly spaced rows each (route + experts + shared)"))
    base = dict(value=done_tokens / dt, unit="tokens/s", cores=int(threads), kind="oracle", sample=sample,
                seconds=round(dt, 2))

    # grading of batch 0
    near = swapped = 0
    ref = first["out"]
    sel = np.arange(T) if rows is None else rows
    if tids is None:
        oi, _, gap, _ = oracle.route(batches[0], layer.gate_w, layer.bias, layer.logit_offset, k=layer.wl.k)
        near = int(np.sum(gap < 1e-5))
        for j, t in enumerate(sel):
            if set(gpu_ids[t].tolist()) != set(first["ids"][j].tolist()):
                swapped += 1
                r2 = fwd(layer, batches[0], rows=np.array([t], np.int32), force_ids=gpu_ids[t][None, :])
                ref[j] = r2["out"][0]
        # every token of the batch whose set differs (near-ties only, at the bar)
        differ = [t for t in range(T) if set(gpu_ids[t].tolist()) != set(oi[t].tolist())]
        bad = [t for t in differ if gap[t] >= 1e-5]
    else:
        oi, _ = oracle.hash_route(batches[0], tids[0], layer.tid2eid, layer.gate_w)
        differ = [t for t in range(T) if not np.array_equal(gpu_ids[t], oi[t])]
        bad = differ
    g = gpu_out32[sel]
    d = g - ref
    rms = float(np.sqrt(np.mean(ref * ref)))
    check = dict(rows_compared=int(len(sel)), rel_l2=float(np.linalg.norm(d) / np.linalg.norm(ref)),
                 max_abs_over_rms=float(np.abs(d).max() / rms), near_ties=near, routing_sets_differ=len(differ),
                 routing_mismatch_not_near_tie=len(bad),
                 within_bar=bool(np.linalg.norm(d) / np.linalg.norm(ref) <= 5e-3 and np.abs(d).max() <= 2e-2 * rms
                                 and not bad))
    return base, check


def workload_variant(base_host, base_copies, wl):
    """The base layer's expert, shared and router weights with this workload's
    own router bias, logit offset and hash table (host, and each device copy)."""
    import dataclasses

    import torch

    import synth

    bias = synth.normal_f32(wl.seed, synth.S_BIAS, 0, wl.E, wl.bias_sigma)
    off = synth.normal_f32(wl.seed, synth.S_OFFSET, 0, wl.E, wl.offset_sigma) if wl.offset_sigma > 0 else None
    t2e = synth.tid2eid(wl.seed, synth.S_TID2EID, 0, wl.V, wl.E, wl.k) if wl.hash_layer else None
    host = dataclasses.replace(base_host, wl=wl, bias=bias, logit_offset=off, tid2eid=t2e)
    dev = base_copies[0].gate_w.device
    b_d = torch.from_numpy(bias).to(dev)
    o_d = None if off is None else torch.from_numpy(off).to(dev)
    t_d = None if t2e is None else torch.from_numpy(t2e).to(dev)
    copies = [dataclasses.replace(c, bias=b_d, logit_offset=o_d, tid2eid=t_d) for c in base_copies]
    return host, copies


def run_workload(args, name, base_host, base_copies, K, W, C, cpu_budget):
    """Time K steps of one workload (after W warm-up steps) and measure its
    dominant kernel; returns the workload's record."""
    import numpy as np
    import torch

    import mxfp4_moe_expert_amd as mx
    import synth

    _, _, _, kernel, bound = DEFAULTS[name]
    wl = synth.WORKLOADS[name]
    T, H, k = wl.T, wl.H, wl.k
    dev = base_copies[0].gate_w.device
    cfg = mx.config_of(wl)
    layer, copies = workload_variant(base_host, base_copies[:C], wl)
    # the routed w2 in 3-bit blocks (per-expert tables): host once, C device copies
    q3 = name.startswith("w2q3_")
    q3_host = q3_dev = None
    if q3:
        if "w2q3" not in _Q3:
            t = time.perf_counter()
            _Q3["w2q3"] = synth.make_w2q3(synth.WORKLOADS["decode_t1"], True)
            print(f"[bench] 3-bit w2 generated in {time.perf_counter() - t:.1f} s", file=sys.stderr, flush=True)
        q3_host = _Q3["w2q3"]
        c0 = torch.from_numpy(q3_host[0]).to(dev)
        s0 = torch.from_numpy(q3_host[1].view(np.int16)).to(dev)
        l0 = torch.from_numpy(q3_host[2]).to(dev)
        q3_dev = [(c0, s0, l0)] + [(c0.clone(), s0.clone(), l0.clone()) for _ in range(C - 1)]
    sched = mx.forward_schedule(cfg, T, hash_layer=wl.hash_layer)
    nb = min(K + W, max(2, (1 << 27) // (T * H)))
    batches = [synth.make_tokens(wl, rep=r) for r in range(nb)]
    tids = [synth.make_token_ids(wl, rep=r) for r in range(nb)] if wl.hash_layer else None
    x_dev = torch.stack([mx.bf16_from_numpy(b, dev) for b in batches])
    t_dev = torch.stack([torch.from_numpy(t).to(dev) for t in tids]) if tids else None
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    ids_all = torch.empty(K, T, k, dtype=torch.int32, device=dev)
    w_all = torch.empty(K, T, k, dtype=torch.float32, device=dev)
    ws = mx.Workspace(dev)
    buf = ws.get(cfg, T)
    L = mx.lib()
    stream = torch.cuda.current_stream(dev)

    def call_args(s, st):
        D = copies[s % C]
        xb = x_dev[s % nb]
        tb = None if t_dev is None else t_dev[s % nb]
        P = mx._ptr
        w2 = (P(D.w2_codes), P(D.w2_scales)) if not q3 else tuple(P(t) for t in q3_dev[s % C])
        return (ctypes.byref(cfg), T, P(xb), P(D.gate_w), P(D.bias), P(D.logit_offset), P(tb),
                P(D.tid2eid if tb is not None else None), 0 if D.tid2eid is None else D.tid2eid.shape[0],
                P(D.w13_codes), P(D.w13_scales), *w2, P(D.sh_w13), P(D.sh_w13_scale),
                P(D.sh_w2), P(D.sh_w2_scale), P(out), 0, P(ids_all[s % K]), P(w_all[s % K]), P(buf), buf.numel(),
                ctypes.c_void_p(st))

    argv = [call_args(s, stream.cuda_stream) for s in range(max(K, W))]
    entry = L.moe_forward_w2q3 if q3 else L.moe_forward

    def step(s):
        rc = entry(*argv[s])
        if rc != 0:
            raise mx.MoEError(rc, "moe_forward")

    hip = Hip()
    ev_a = [hip.event() for _ in range(K)]
    ev_b = [hip.event() for _ in range(K)]
    for s in range(W):
        step(s)
    torch.cuda.synchronize(dev)

    # eager pass: timing-only events bracket the dominant kernel on its launch stream, every step
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s in range(K):
        mx.set_kernel_events(kernel, ev_a[s], ev_b[s])
        step(s)
    t1.record(stream)
    mx.set_kernel_events(None)
    torch.cuda.synchronize(dev)
    eager_ms = t0.elapsed_time(t1)
    kern_ms = [hip.elapsed_ms(ev_a[s], ev_b[s]) for s in range(K)]
    for e in ev_a + ev_b:
        hip.destroy(e)

    graph_ms = None
    if args.mode == "graph":
        G = max(1, min(args.graph_steps, K))
        graphs = []
        cs = torch.cuda.Stream(dev)
        argv_g = [call_args(s, cs.cuda_stream) for s in range(K)]
        with torch.cuda.stream(cs):
            for g0 in range(0, K, G):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=cs):
                    for s in range(g0, min(K, g0 + G)):
                        rc = entry(*argv_g[s])
                        if rc != 0:
                            raise mx.MoEError(rc, "moe_forward (capture)")
                graphs.append(gr)
        torch.cuda.synchronize(dev)
        graphs[0].replay()  # warm replay
        torch.cuda.synchronize(dev)
        t0.record(stream)
        for gr in graphs:
            gr.replay()
        t1.record(stream)
        torch.cuda.synchronize(dev)
        graph_ms = t0.elapsed_time(t1)
        del graphs

    total_ms = graph_ms if graph_ms is not None else eager_ms
    ms_step = total_ms / K
    ids_np = ids_all.cpu().numpy()
    alg = algorithmic(wl, ids_np, w2q3=q3)
    # The dominant kernel's average duration: in the single-launch schedule
    # the kernel is the whole step, so it is the timed region over K steps
    # (the event pair around each eager launch adds its own recording time);
    # otherwise the mean of the per-launch event pairs of the eager pass.
    if sched == "single":
        kern_avg_ms = ms_step
        ksrc = ("timed region / steps (one launch per step, events on the launch stream around "
                + ("the graph replays)" if graph_ms is not None else "the eager steps)"))
    else:
        kern_avg_ms = sum(kern_ms) / K
        ksrc = "mean of per-launch event pairs on the launch stream (eager pass)"
    scope = dominant(name)[2]
    if bound == "hbm":
        achieved = alg[scope + "_bytes"] / (kern_avg_ms / 1e3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), algorithmic=int(alg[scope + "_bytes"]))
    elif "k_gemm_mx" in dominant(name)[0]:
        # block-scaled fp8 x fp4 MFMA: every bf16 activation is split into two fp8 halves, so the
        # matrix cores execute twice the method's flops at the fp8 rate; the fraction of the fp8
        # peak equals the method's flops over the bf16 peak (the metric's definition)
        algo = alg[scope + "_flops"]
        achieved = 2.0 * algo / (kern_avg_ms / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_FP8_TFLOPS, 4), algorithmic=algo, executed=2.0 * algo,
                    dtype="fp8 x fp4 (block-scaled; activations as exact hi + lo fp8)",
                    bf16_equivalent_TFLOPs=round(achieved / 2.0, 2),
                    bf16_equivalent_frac=round(achieved / 2.0 / PEAK_BF16_TFLOPS, 4))
    else:
        achieved = alg[scope + "_flops"] / (kern_avg_ms / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4), algorithmic=alg[scope + "_flops"])
    roof["traffic"] = traffic_from_profiles(name)
    roof["kernel"] = dominant(name)[0]
    roof["kernel_avg_us"] = round(kern_avg_ms * 1e3, 2)
    roof["kernel_time"] = ksrc
    ks = sorted(kern_ms)
    roof["kernel_event_p50_us"] = round(ks[len(ks) // 2] * 1e3, 2)
    roof["kernel_event_p99_us"] = round(ks[min(len(ks) - 1, (len(ks) * 99) // 100)] * 1e3, 2)
    if kern_avg_ms > ms_step * 1.001:
        print(f"warning: {name}: kernel time {kern_avg_ms * 1e3:.2f} us exceeds the step {ms_step * 1e3:.2f} us",
              file=sys.stderr, flush=True)
        roof["warning"] = "kernel time exceeds the timed step"
    layer_bw = alg["layer_bytes"] / (ms_step / 1e3) / 1e9
    layer_tf = alg["layer_flops"] / (ms_step / 1e3) / 1e12
    rec = {
        "T": T, "schedule": sched, "steps": K, "warmup": W, "weight_copies": C, "mode": args.mode,
        "ms_per_step": round(ms_step, 5), "tokens_per_s": round(T * K / (total_ms / 1e3), 1),
        "roofline": roof,
        "layer": {"bytes_per_step": int(alg["layer_bytes"]), "hbm_GBps": round(layer_bw, 1),
                  "hbm_frac": round(layer_bw / PEAK_HBM_GBS, 4), "flops_per_step": alg["layer_flops"],
                  "mfma_TFLOPs": round(layer_tf, 2), "mfma_frac": round(layer_tf / PEAK_BF16_TFLOPS, 4),
                  "distinct_experts": round(alg["distinct_experts"], 2),
                  "eager_ms_per_step": round(eager_ms / K, 5),
                  "graph_ms_per_step": None if graph_ms is None else round(graph_ms / K, 5)},
    }
    if cpu_budget > 0:
        import oracle

        tb0 = None if t_dev is None else t_dev[0]
        if q3:
            o32 = mx.forward_w2q3(cfg, x_dev[0], copies[0], *q3_dev[0], token_ids=tb0, out_fp32=True, ws=ws)
            ids0 = mx.forward_w2q3(cfg, x_dev[0], copies[0], *q3_dev[0], token_ids=tb0, return_routing=True,
                                   ws=ws)[1][0]
            c2, s2, l2 = q3_host
            fwd = lambda lay, xb, **kw: oracle.forward_w2q3(lay, c2, s2, l2, xb, **kw)  # noqa: E731
        else:
            o32 = mx.forward(cfg, x_dev[0], copies[0], token_ids=tb0, out_fp32=True, ws=ws)
            ids0 = mx.forward(cfg, x_dev[0], copies[0], token_ids=tb0, return_routing=True, ws=ws)[1][0]
            fwd = None
        torch.cuda.synchronize(dev)
        cb, check = cpu_leg(layer, batches, tids, cpu_budget, o32.cpu().double().numpy(), ids0.cpu().numpy(),
                            fwd=fwd)
        rec["cpu_baseline"] = cb
        rec["parity"] = check
    if q3:
        rec["w2_format"] = "3-bit blocks: 12 B codes + binary16 scale per 32 weights, per-expert tables of 8 levels"
    del x_dev, t_dev, out, ids_all, w_all, ws, buf, q3_dev
    torch.cuda.empty_cache()
    return rec


def stack_cpu_leg(base_host, base_copies, layers_dev, budget_s):
    """The oracle on the stack: checked layers (0, 1, 3 and the last) each on
    its own seeded token against the GPU, the first two layers chained
    (the oracle's layer 1 reads its own layer 0's bf16 output) against the
    GPU stack, and the oracle's rate per token through all layers from its
    time per layer."""
    import numpy as np
    import torch

    import mxfp4_moe_expert_amd as mx
    import oracle
    import synth

    wl = base_host.wl
    cfg = mx.config_of(wl)
    dev = base_copies[0].gate_w.device
    nl = len(layers_dev)
    checked = [0, 1, 3, nl - 1]
    hosts = {l: synth.make_stack_layer(base_host, l) for l in checked}
    tz = synth.WORKLOADS["hash_t4096"]
    worst, times = 0.0, []
    for l in checked:
        L = hosts[l]
        xh = synth.make_tokens(wl, rep=900 + l, T=1)
        tid_h = synth.make_token_ids(tz, rep=900 + l, T=1)
        hsh = L.wl.hash_layer
        out = mx.forward(cfg, mx.bf16_from_numpy(xh, dev), layers_dev[l],
                         token_ids=torch.from_numpy(tid_h).to(dev) if hsh else None, out_fp32=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = oracle.forward(L, xh, token_ids=tid_h if hsh else None)
        times.append(time.perf_counter() - t0)
        d = out.cpu().double().numpy() - r["out"]
        worst = max(worst, float(np.linalg.norm(d) / np.linalg.norm(r["out"])))
    # the first two layers chained
    xh = synth.make_tokens(wl, rep=950, T=1)
    tid_h = synth.make_token_ids(tz, rep=950, T=1)
    r0 = oracle.forward(hosts[0], xh, token_ids=tid_h)
    x1 = synth.f32_to_bf16(r0["out"].astype(np.float32))
    r1 = oracle.forward(hosts[1], x1, token_ids=tid_h)
    out = mx.forward_stack(cfg, mx.bf16_from_numpy(xh, dev), layers_dev[:2],
                           token_ids=torch.from_numpy(tid_h).to(dev), out_fp32=True)
    torch.cuda.synchronize()
    d = out.cpu().double().numpy() - r1["out"]
    chain = float(np.linalg.norm(d) / np.linalg.norm(r1["out"]))
    per_layer = sum(times) / len(times)
    threads = oracle.lib().or_num_threads()
    cb = dict(value=1.0 / (nl * per_layer), unit="tokens/s", cores=int(threads), kind="oracle",
              sample=f"{len(checked)} of {nl} layers at T=1 (layers {checked}), rate = 1 / ({nl} x mean layer time)",
              seconds=round(sum(times), 2))
    check = dict(layers_checked=checked, rel_l2_max=worst, chain_layers_0_1_rel_l2=chain,
                 within_bar=bool(worst <= 5e-3 and chain <= 5e-3))
    return cb, check


def run_stack(args, name, base_host, base_copies, K, W, cpu_budget):
    """K steps of one token through the 43-layer stack (moe_forward_stack),
    every layer's weights in their own device memory (about 147 GB)."""
    import torch

    import mxfp4_moe_expert_amd as mx
    import synth

    wl = base_host.wl
    cfg = mx.config_of(wl)
    dev = base_copies[0].gate_w.device
    nl = synth.STACK_LAYERS
    t0 = time.perf_counter()
    layers = []
    for l in range(nl):
        Lh = synth.make_stack_layer(base_host, l, routed=False)
        order = torch.from_numpy(Lh.extra["expert_order"]).to(dev)
        b = base_copies[0]
        pick = (lambda t: t.index_select(0, order)) if l else (lambda t: t)

        def d(a):
            return None if a is None else torch.from_numpy(a).to(dev)
        layers.append(mx.DeviceLayer(d(Lh.gate_w), d(Lh.bias), None, pick(b.w13_codes), pick(b.w13_scales),
                                     pick(b.w2_codes), pick(b.w2_scales), d(Lh.sh_w13), d(Lh.sh_w13_scale),
                                     d(Lh.sh_w2), d(Lh.sh_w2_scale), d(Lh.tid2eid)))
    torch.cuda.synchronize(dev)
    t_build = time.perf_counter() - t0
    print(f"[bench] {name}: {nl} layers built in {t_build:.1f} s", file=sys.stderr, flush=True)
    weights = (mx.MoeLayerWeights * nl)(*[mx.layer_weights(L) for L in layers])
    nb = min(K + W, 256)
    xs = torch.stack([mx.bf16_from_numpy(synth.make_tokens(wl, rep=r, T=1), dev) for r in range(nb)])
    tz = synth.WORKLOADS["hash_t4096"]
    tids = torch.stack([torch.from_numpy(synth.make_token_ids(tz, rep=r, T=1)) for r in range(nb)]).to(dev)
    act = torch.empty(2, 1, wl.H, dtype=torch.bfloat16, device=dev)
    out = torch.empty(1, wl.H, dtype=torch.bfloat16, device=dev)
    ws = mx.Workspace(dev)
    buf = ws.get(cfg, 1)
    L = mx.lib()

    def args_of(s, st):
        P = mx._ptr
        return (ctypes.byref(cfg), nl, weights, 1, P(xs[s % nb]), P(tids[s % nb]), P(act), P(out), 0, P(buf),
                buf.numel(), ctypes.c_void_p(st))

    stream = torch.cuda.current_stream(dev)
    for s in range(W):
        rc = L.moe_forward_stack(*args_of(s, stream.cuda_stream))
        if rc != 0:
            raise mx.MoEError(rc, "moe_forward_stack")
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(K):
        rc = L.moe_forward_stack(*args_of(s, stream.cuda_stream))
        if rc != 0:
            raise mx.MoEError(rc, "moe_forward_stack")
    e1.record(stream)
    torch.cuda.synchronize(dev)
    eager_ms = e0.elapsed_time(e1)
    graph_ms = None
    if args.mode == "graph":
        G = max(1, min(10, K))
        cs = torch.cuda.Stream(dev)
        graphs = []
        with torch.cuda.stream(cs):
            for g0 in range(0, K, G):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=cs):
                    for s in range(g0, min(K, g0 + G)):
                        rc = L.moe_forward_stack(*args_of(s, cs.cuda_stream))
                        if rc != 0:
                            raise mx.MoEError(rc, "moe_forward_stack (capture)")
                graphs.append(gr)
        torch.cuda.synchronize(dev)
        graphs[0].replay()
        torch.cuda.synchronize(dev)
        e0.record(stream)
        for gr in graphs:
            gr.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        graph_ms = e0.elapsed_time(e1)
        del graphs
    total_ms = graph_ms if graph_ms is not None else eager_ms
    ms_step = total_ms / K
    import numpy as np
    per_layer = algorithmic(wl, np.arange(wl.k, dtype=np.int32).reshape(1, 1, wl.k))  # 6 distinct experts per layer
    layer_ms = ms_step / nl
    achieved = per_layer["layer_bytes"] / (layer_ms / 1e3) / 1e9
    roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(achieved / PEAK_HBM_GBS, 4), algorithmic=int(per_layer["layer_bytes"]), traffic=None,
                kernel=DOMINANT[name][0], kernel_avg_us=round(layer_ms * 1e3, 2),
                kernel_time=f"timed region / (steps x {nl} layers): launches of up to 8 layers each, "
                            "back to back")
    rec = {"T": 1, "layers": nl, "hash_layers": synth.STACK_HASH_LAYERS,
           "schedule": "single-launch layers, up to 8 per launch",
           "steps": K, "warmup": W, "weight_copies": "one per layer", "mode": args.mode,
           "ms_per_step": round(ms_step, 5), "tokens_per_s": round(1e3 / ms_step, 1),
           "roofline": roof,
           "stack": {"bytes_per_step": int(nl * per_layer["layer_bytes"]),
                     "hbm_GBps": round(nl * per_layer["layer_bytes"] / (ms_step / 1e3) / 1e9, 1),
                     "eager_ms_per_step": round(eager_ms / K, 5),
                     "graph_ms_per_step": None if graph_ms is None else round(graph_ms / K, 5),
                     "build_seconds": round(t_build, 1), "device_bytes_of_weights": int(nl * 3422552064)}}
    if cpu_budget > 0:
        cb, check = stack_cpu_leg(base_host, base_copies, layers, cpu_budget)
        rec["cpu_baseline"] = cb
        rec["parity"] = check
    del layers, weights, xs, tids, act, out, ws, buf
    torch.cuda.empty_cache()
    return rec


# The model's int8 attention projections (page "deepseek-v4-mxfp4-int8 config.json", config group
# linears_w8a16) as (K, N, groups); the pages name them, the shapes are readings of the model's sizes.
LINEARS = {"fused_wqa_wkv": (4096, 1536, 1), "wq_b": (1024, 32768, 1), "wo_a": (4096, 1024, 8),
           "wo_b": (8192, 4096, 1), "indexer_wq_b": (1024, 8192, 1), "indexer_compressor_wkv": (4096, 256, 1)}


def run_linears(reps=40, copies=4):
    """moe_linear_w8a16 on each projection at T = 1, 64 (bound by the int8
    weights' bytes) and 8192 (bf16 MFMA), weights rotated through `copies`
    copies (together beyond the last-level cache): `reps` calls captured in
    one HIP graph, replayed between events on the launch stream (so that the
    host's call overhead is not timed); the mean per call."""
    import torch

    import mxfp4_moe_expert_amd as mx
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    res = {}
    for i, (name, (K, N, G)) in enumerate(LINEARS.items()):
        q, sc = synth.int8_normal(0, synth.S_LINEAR, i, G * N, K, 0.02)
        qs = [torch.from_numpy(q).to(dev) for _ in range(copies)]
        ss = [torch.from_numpy(sc).to(dev) for _ in range(copies)]
        wbytes = G * N * K + G * N * 4
        res[name] = {"K": K, "N": N, "groups": G}
        for T in (1, 64, 8192):
            x = mx.bf16_from_numpy(synth.normal_bf16(0, synth.S_TOKENS, 800 + T, T * G * K).reshape(T, G * K), dev)
            out = torch.empty(T, G * N, dtype=torch.bfloat16, device=dev)
            n = reps if T <= 64 else 10
            for r in range(3):
                mx.linear_w8a16(x, qs[r % copies], ss[r % copies], groups=G, out=out)
            torch.cuda.synchronize(dev)
            cs = torch.cuda.Stream(dev)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cs):
                with torch.cuda.graph(gr, stream=cs):
                    for r in range(n):
                        mx.linear_w8a16(x, qs[r % copies], ss[r % copies], groups=G, out=out)
            torch.cuda.synchronize(dev)
            gr.replay()  # warm replay
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize(dev)
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            us = e0.elapsed_time(e1) * 1e3 / n
            del gr
            if T <= 64:
                b = wbytes + T * G * (K + N) * 2
                res[name][f"T{T}"] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1),
                                      "hbm_frac": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
            else:
                f = 2.0 * T * G * N * K
                res[name][f"T{T}"] = {"us": round(us, 2), "TFLOPs": round(f / us / 1e6, 1),
                                      "mfma_frac": round(f / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
        del qs, ss
    torch.cuda.empty_cache()
    return res


ORDER = ["decode_t1", "decode_t64", "prefill_t8192", "hash_t4096", "w2q3_t1", "w2q3_t64", "stack43_t1"]
_Q3 = {}  # the 3-bit w2 of the base layer (host), generated once


def main():
    args = parse()
    if args.summarize:
        PREFILL_MX[0] = args.prefill_mfma == "block-scaled"
        cmds = {}
        if args.commands:
            with open(args.commands) as f:
                cmds = json.load(f)
        summarize(args.workload, args.summarize, cmds)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on a single GPU: --gpus must be 1 (there is no multi-GPU path)"}))
        sys.exit(2)
    if args.peaks:
        measured_peaks()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import mxfp4_moe_expert_amd as mx
    import synth

    if args.prefill_mfma == "block-scaled":
        PREFILL_MX[0] = True
        mx.set_option("prefill_block_scaled", 1)
    names = ORDER if args.workload == "all" else [args.workload]
    main_name = names[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    plan = {}
    for i, n in enumerate(names):
        steps0, warm0, copies0, _, _ = DEFAULTS[n]
        K = args.steps if (args.steps is not None and i == 0) else steps0
        W = args.warmup if (args.warmup is not None and i == 0) else warm0
        C = max(1, args.copies if args.copies is not None else copies0)
        plan[n] = (K, W, C)
    t_gen = time.perf_counter()
    base_host = synth.make_layer(synth.WORKLOADS["decode_t1"])  # seed 0: the same weights for every workload
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] layer generated in {t_gen:.1f} s", file=sys.stderr, flush=True)
    base = mx.DeviceLayer.from_host(base_host, dev)
    Cmax = max(c for _, _, c in plan.values())
    base_copies = [base] + [mx.DeviceLayer(*[None if t is None else t.clone() for t in vars(base).values()])
                            for _ in range(Cmax - 1)]
    recs = {}
    for i, n in enumerate(names):
        K, W, C = plan[n]
        budget = 0.0 if args.no_cpu_baseline else (args.cpu_seconds if i == 0 else args.extra_cpu_seconds)
        print(f"[bench] {n}: {K} steps after {W} warm-up, {C} weight copies", file=sys.stderr, flush=True)
        if n == "stack43_t1":
            del base_copies[1:]  # the stack's layers take their own copies
            torch.cuda.empty_cache()
            recs[n] = run_stack(args, n, base_host, base_copies, K, W, budget)
        else:
            recs[n] = run_workload(args, n, base_host, base_copies, K, W, C, budget)
        print(f"[bench] {n}: {recs[n]['ms_per_step']} ms/step, {recs[n]['tokens_per_s']} tokens/s",
              file=sys.stderr, flush=True)
    m = recs[main_name]
    wl = synth.WORKLOADS[main_name]
    rec = {
        "metric": METRIC, "value": m["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": m["steps"],
        "warmup": m["warmup"], "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": main_name, "T": wl.T, "hidden_size": wl.H, "n_routed_experts": wl.E,
                   "top_k": wl.k, "moe_intermediate": wl.I, "routed": "mxfp4 (E2M1 + E8M0/32)",
                   "shared": "int8 per-channel", "weight_copies": m["weight_copies"], "mode": args.mode,
                   "prefill_mfma": args.prefill_mfma,
                   "schedule": m["schedule"], "parallelism": "single GPU"},
        "roofline": m["roofline"],
        "layer": m.get("layer", m.get("stack")),
        "cpu_baseline": m.get("cpu_baseline"),
        "parity": m.get("parity"),
        "gen_seconds": round(t_gen, 1),
        "workloads": {n: r for n, r in recs.items() if n != main_name},
    }
    if args.workload == "all" or args.linears:
        print("[bench] w8a16 linears", file=sys.stderr, flush=True)
        rec["w8a16_linears"] = run_linears()
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()

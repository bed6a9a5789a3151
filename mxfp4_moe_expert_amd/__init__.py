"""Python binding of ``libmoe.so`` — a DeepSeek-V4-Flash MoE layer for MI355X.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``csrc/`` behind the C ABI of ``include/moe.h``. PyTorch provides device
memory and the current stream. There is no CPU fallback: if the library is
not built, or a call fails, an exception is raised.

Entry points (same names as the C ABI): ``route``, ``hash_route``,
``permute``, ``expert_ffn``, ``forward``; plus ``workspace_size``,
``Workspace`` and ``DeviceLayer`` (device copies of one layer's parameters).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
KERNELS = {"router": 1, "permute": 2, "routed_w13": 3, "routed_w2": 4, "shared_w13": 5, "shared_w2": 6,
           "combine": 7}


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class MoeLayerWeights(ctypes.Structure):
    """Mirror of ``moe_layer_weights`` (device pointers of one layer)."""
    _fields_ = [("gate_w", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("logit_offset", ctypes.c_void_p),
                ("tid2eid", ctypes.c_void_p), ("V", ctypes.c_int32), ("w13_codes", ctypes.c_void_p),
                ("w13_scales", ctypes.c_void_p), ("w2_codes", ctypes.c_void_p), ("w2_scales", ctypes.c_void_p),
                ("sh_w13", ctypes.c_void_p), ("sh_w13_scale", ctypes.c_void_p), ("sh_w2", ctypes.c_void_p),
                ("sh_w2_scale", ctypes.c_void_p)]


class MoeConfig(ctypes.Structure):
    """Mirror of ``moe_config`` (names of the checkpoint's config.json)."""
    _fields_ = [("hidden_size", ctypes.c_int32), ("n_routed_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("moe_intermediate", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("swiglu_limit", ctypes.c_float),
                ("norm_topk_prob", ctypes.c_int32)]


def config(hidden_size=4096, n_routed_experts=256, top_k=6, moe_intermediate=2048,
           routed_scaling_factor=1.5, swiglu_limit=10.0, norm_topk_prob=1) -> MoeConfig:
    return MoeConfig(hidden_size, n_routed_experts, top_k, moe_intermediate, routed_scaling_factor,
                     swiglu_limit, norm_topk_prob)


def config_of(wl) -> MoeConfig:
    """Config of a workload description with fields H, E, k, I (e.g. ``synth.Workload``)."""
    return config(wl.H, wl.E, wl.k, wl.I, wl.routed_scaling_factor, wl.swiglu_limit)


_lib = None
_VP, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_CFGP = ctypes.POINTER(MoeConfig)

_SIGNATURES = {
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_version": ([], ctypes.c_char_p),
    "moe_workspace_size": ([_CFGP, _I32], _SZ),
    "moe_workspace_init": ([_VP, _SZ, _VP], ctypes.c_int),
    "moe_route": ([_CFGP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "moe_hash_route": ([_CFGP, _I32, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP], ctypes.c_int),
    "moe_permute": ([_CFGP, _I32, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "moe_expert_ffn": ([_CFGP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
                       ctypes.c_int),
    "moe_set_kernel_events": ([_I32, _VP, _VP], ctypes.c_int),
    "moe_device_flags": ([ctypes.POINTER(ctypes.c_uint32), _I32, _VP], ctypes.c_int),
    "moe_read_probe": ([_VP, _SZ, _I32, _VP, _VP], ctypes.c_int),
    "moe_set_option": ([_I32, _I32], ctypes.c_int),
    "moe_get_option": ([_I32], ctypes.c_int),
    "moe_forward_schedule": ([_CFGP, _I32, _I32], ctypes.c_int),
    "moe_noalloc_max_bytes": ([], _SZ),
    "moe_linear_workspace_size": ([_I32, _I32, _I32, _I32], _SZ),
    "moe_linear_w8a16": ([_I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _VP, _SZ, _VP], ctypes.c_int),
    "moe_forward_stack": ([_CFGP, _I32, _VP, _I32, _VP, _VP, _VP, _VP, _I32, _VP, _SZ, _VP], ctypes.c_int),
    "moe_forward_noalloc": ([_CFGP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP,
                             _VP, _VP, _VP, _I32, _VP, _VP, _VP], ctypes.c_int),
    "moe_forward": ([_CFGP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP,
                     _VP, _VP, _VP, _I32, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "moe_forward_w2q3": ([_CFGP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                          _VP, _VP, _VP, _I32, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
}


def lib():
    """The loaded ``libmoe.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with mxfp4_moe_expert_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def version() -> str:
    return lib().moe_version().decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoEError(status, what)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: torch.Tensor expected")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device (cuda/hip) tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def set_kernel_events(kernel: str | None, start_event=None, stop_event=None):
    """Bracket every launch of ``kernel`` (a KERNELS name) with the given
    hipEvent_t handles (ints or c_void_p); None stops. Measurement only."""
    kid = 0 if kernel is None else KERNELS[kernel]
    _check(lib().moe_set_kernel_events(kid, start_event, stop_event), "moe_set_kernel_events")


OPTIONS = {"prefill_block_scaled": 1}


def set_option(name: str, value: int):
    """Set a process-wide option (``OPTIONS``); returns the previous value."""
    prev = lib().moe_get_option(OPTIONS[name])
    _check(lib().moe_set_option(OPTIONS[name], int(value)), "moe_set_option")
    return prev


FLAGS = {"token_id": 1, "table_entry": 2, "expert_id": 4, "wait_expired": 8, "permutation": 16}


def read_probe(buf, blocks: int, sink, device=None) -> None:
    """Queues the library's streaming-read kernel over all of ``buf`` (a
    contiguous device tensor, 16-byte multiple) with ``blocks`` blocks on the
    current stream; ``sink`` is an int32/uint32 device tensor of at least
    ``blocks`` words (a measurement aid: time it to get the read rate)."""
    if not (buf.is_cuda and sink.is_cuda and buf.is_contiguous()):
        raise ValueError("read_probe: contiguous device tensors expected")
    if sink.numel() * sink.element_size() < 4 * blocks:
        raise ValueError("read_probe: sink smaller than one word per block")
    _check(lib().moe_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), int(blocks), sink.data_ptr(),
                                _stream(device)), "moe_read_probe")


def device_flags(clear: bool = False, device=None) -> set:
    """Names of the device error flags (``FLAGS``) set on the current device
    by work queued so far on the current stream; waits for that stream.
    ``clear`` resets them afterwards."""
    v = ctypes.c_uint32(0)
    _check(lib().moe_device_flags(ctypes.byref(v), 1 if clear else 0, _stream(device)), "moe_device_flags")
    return {name for name, bit in FLAGS.items() if v.value & bit}


SCHEDULES = {1: "single", 2: "tiny", 3: "decode", 4: "large"}


def forward_schedule(cfg: MoeConfig, T: int, hash_layer: bool = False) -> str:
    """Which launch sequence ``forward`` takes for T tokens on the current
    device: "single" (the whole layer in one launch), "tiny", "decode" or
    "large"."""
    rc = lib().moe_forward_schedule(ctypes.byref(cfg), T, 1 if hash_layer else 0)
    if rc < 0:
        raise MoEError(rc, "moe_forward_schedule")
    return SCHEDULES[rc]


def workspace_size(cfg: MoeConfig, T: int) -> int:
    n = lib().moe_workspace_size(ctypes.byref(cfg), T)
    if n == 0:
        raise MoEError(MOE_EUNSUPPORTED, "moe_workspace_size")
    return n


class Workspace:
    """Zero-initialised device scratch, grown on demand (one per device/stream user)."""

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf = None

    def get(self, cfg: MoeConfig, T: int) -> torch.Tensor:
        need = workspace_size(cfg, T)
        if self.buf is None or self.buf.numel() < need:
            self.buf = torch.zeros(need, dtype=torch.uint8, device=self.device)
            if self.buf.data_ptr() % 256:
                raise RuntimeError("workspace allocation is not 256-byte aligned")
        return self.buf


_default_ws: dict = {}


def _ws(cfg, T, device, ws):
    if ws is None:
        key = torch.device(device).index or 0
        ws = _default_ws.setdefault(key, Workspace(device))
    buf = ws.get(cfg, T)
    return buf, buf.numel()


# ------------------------------------------------------------------ device layer

@dataclass
class DeviceLayer:
    """Device tensors of one layer (layouts as in include/moe.h)."""
    gate_w: torch.Tensor
    bias: torch.Tensor
    logit_offset: torch.Tensor | None
    w13_codes: torch.Tensor
    w13_scales: torch.Tensor
    w2_codes: torch.Tensor
    w2_scales: torch.Tensor
    sh_w13: torch.Tensor
    sh_w13_scale: torch.Tensor
    sh_w2: torch.Tensor
    sh_w2_scale: torch.Tensor
    tid2eid: torch.Tensor | None = None

    @staticmethod
    def from_host(layer, device="cuda") -> "DeviceLayer":
        """Copy a host layer (numpy arrays with the same field names) to the device."""
        def d(a):
            return None if a is None else torch.from_numpy(a).to(device)
        return DeviceLayer(d(layer.gate_w), d(layer.bias), d(layer.logit_offset), d(layer.w13_codes),
                           d(layer.w13_scales), d(layer.w2_codes), d(layer.w2_scales), d(layer.sh_w13),
                           d(layer.sh_w13_scale), d(layer.sh_w2), d(layer.sh_w2_scale), d(layer.tid2eid))


def bf16_from_numpy(a, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> a torch.bfloat16 device tensor."""
    import numpy as np

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


# ------------------------------------------------------------------ entry points

def route(cfg: MoeConfig, x, gate_w, bias, logit_offset=None, ws=None, out=None):
    """Learned router -> (topk_ids int32 [T,k], topk_w fp32 [T,k])."""
    T, H, E, k = x.shape[0], cfg.hidden_size, cfg.n_routed_experts, cfg.top_k
    _need(x, _BF16, (T, H), "x")
    _need(gate_w, torch.float32, (E, H), "gate_w")
    _need(bias, torch.float32, (E,), "bias")
    if logit_offset is not None:
        _need(logit_offset, torch.float32, (E,), "logit_offset")
    ids, w = out if out is not None else (torch.empty(T, k, dtype=torch.int32, device=x.device),
                                          torch.empty(T, k, dtype=torch.float32, device=x.device))
    buf, nb = _ws(cfg, T, x.device, ws)
    _check(lib().moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(gate_w), _ptr(bias), _ptr(logit_offset),
                           _ptr(ids), _ptr(w), _ptr(buf), nb, _stream(x.device)), "moe_route")
    return ids, w


def hash_route(cfg: MoeConfig, x, token_ids, tid2eid, gate_w, out=None):
    """Hash-layer router -> (topk_ids, topk_w)."""
    T, H, E, k = x.shape[0], cfg.hidden_size, cfg.n_routed_experts, cfg.top_k
    _need(x, _BF16, (T, H), "x")
    _need(token_ids, torch.int32, (T,), "token_ids")
    _need(tid2eid, torch.int32, None, "tid2eid")
    if tid2eid.dim() != 2 or tid2eid.shape[1] != k:
        raise ValueError("tid2eid: shape [V, top_k] expected")
    _need(gate_w, torch.float32, (E, H), "gate_w")
    ids, w = out if out is not None else (torch.empty(T, k, dtype=torch.int32, device=x.device),
                                          torch.empty(T, k, dtype=torch.float32, device=x.device))
    _check(lib().moe_hash_route(ctypes.byref(cfg), T, _ptr(x), _ptr(token_ids), _ptr(tid2eid),
                                tid2eid.shape[0], _ptr(gate_w), _ptr(ids), _ptr(w), _stream(x.device)),
           "moe_hash_route")
    return ids, w


def permute(cfg: MoeConfig, topk_ids, ws=None):
    """Stable sort of slots by expert -> (expert_offsets [E+1], sorted_slots [T*k], slot_pos [T*k])."""
    T, k, E = topk_ids.shape[0], cfg.top_k, cfg.n_routed_experts
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    dev = topk_ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_slots = torch.empty(T * k, dtype=torch.int32, device=dev)
    slot_pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    buf, nb = _ws(cfg, T, dev, ws)
    _check(lib().moe_permute(ctypes.byref(cfg), T, _ptr(topk_ids), _ptr(offsets), _ptr(sorted_slots),
                             _ptr(slot_pos), _ptr(buf), nb, _stream(dev)), "moe_permute")
    return offsets, sorted_slots, slot_pos


def expert_ffn(cfg: MoeConfig, x, expert_offsets, sorted_slots, topk_w, w13_codes, w13_scales, w2_codes,
               w2_scales, ws=None):
    """Routed experts only -> routed_out fp32 [T, H]."""
    T, H, E, k, I = x.shape[0], cfg.hidden_size, cfg.n_routed_experts, cfg.top_k, cfg.moe_intermediate
    _need(x, _BF16, (T, H), "x")
    _need(expert_offsets, torch.int32, (E + 1,), "expert_offsets")
    _need(sorted_slots, torch.int32, (T * k,), "sorted_slots")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(w13_codes, torch.uint8, (E, 2 * I, H // 2), "w13_codes")
    _need(w13_scales, torch.uint8, (E, 2 * I, H // 32), "w13_scales")
    _need(w2_codes, torch.uint8, (E, H, I // 2), "w2_codes")
    _need(w2_scales, torch.uint8, (E, H, I // 32), "w2_scales")
    out = torch.empty(T, H, dtype=torch.float32, device=x.device)
    buf, nb = _ws(cfg, T, x.device, ws)
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), T, _ptr(x), _ptr(expert_offsets), _ptr(sorted_slots),
                                _ptr(topk_w), _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes),
                                _ptr(w2_scales), _ptr(out), _ptr(buf), nb, _stream(x.device)),
           "moe_expert_ffn")
    return out


def forward(cfg: MoeConfig, x, layer: DeviceLayer, token_ids=None, out_fp32=False, return_routing=False,
            ws=None, out=None, routing_out=None):
    """The whole layer -> out [T, H] (bf16, or fp32 if out_fp32) [, (topk_ids, topk_w)]."""
    T, H, E, k, I = x.shape[0], cfg.hidden_size, cfg.n_routed_experts, cfg.top_k, cfg.moe_intermediate
    dev = x.device
    _need(x, _BF16, (T, H), "x")
    _need(layer.gate_w, torch.float32, (E, H), "gate_w")
    _need(layer.w13_codes, torch.uint8, (E, 2 * I, H // 2), "w13_codes")
    _need(layer.w13_scales, torch.uint8, (E, 2 * I, H // 32), "w13_scales")
    _need(layer.w2_codes, torch.uint8, (E, H, I // 2), "w2_codes")
    _need(layer.w2_scales, torch.uint8, (E, H, I // 32), "w2_scales")
    _need(layer.sh_w13, torch.int8, (2 * I, H), "sh_w13")
    _need(layer.sh_w13_scale, torch.float32, (2 * I,), "sh_w13_scale")
    _need(layer.sh_w2, torch.int8, (H, I), "sh_w2")
    _need(layer.sh_w2_scale, torch.float32, (H,), "sh_w2_scale")
    V = 0
    if token_ids is not None:
        _need(token_ids, torch.int32, (T,), "token_ids")
        if layer.tid2eid is None:
            raise ValueError("hash layer needs layer.tid2eid")
        _need(layer.tid2eid, torch.int32, None, "tid2eid")
        V = layer.tid2eid.shape[0]
    else:
        _need(layer.bias, torch.float32, (E,), "bias")
    if out is None:
        out = torch.empty(T, H, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=dev)
    ids = w = None
    if return_routing:
        ids, w = routing_out if routing_out is not None else (
            torch.empty(T, k, dtype=torch.int32, device=dev), torch.empty(T, k, dtype=torch.float32, device=dev))
    buf, nb = _ws(cfg, T, dev, ws)
    _check(lib().moe_forward(
        ctypes.byref(cfg), T, _ptr(x), _ptr(layer.gate_w), _ptr(layer.bias), _ptr(layer.logit_offset),
        _ptr(token_ids), _ptr(layer.tid2eid if token_ids is not None else None), V, _ptr(layer.w13_codes),
        _ptr(layer.w13_scales), _ptr(layer.w2_codes), _ptr(layer.w2_scales), _ptr(layer.sh_w13),
        _ptr(layer.sh_w13_scale), _ptr(layer.sh_w2), _ptr(layer.sh_w2_scale), _ptr(out), int(out_fp32),
        _ptr(ids), _ptr(w), _ptr(buf), nb, _stream(dev)), "moe_forward")
    if return_routing:
        return out, (ids, w)
    return out


def forward_w2q3(cfg: MoeConfig, x, layer: DeviceLayer, w2_codes, w2_scales, w2_levels=None, token_ids=None,
                 out_fp32=False, return_routing=False, ws=None, out=None):
    """``forward`` with the routed experts' w2 in 3-bit blocks (moe_forward_w2q3):
    w2_codes uint8 [E, H, I/32*12], w2_scales int16/uint16 [E, H, I/32]
    (binary16 bits), w2_levels fp32 [E, 8] or None (the uniform code book).
    ``layer``'s own w2 tensors are not used."""
    T, H, E, k, I = x.shape[0], cfg.hidden_size, cfg.n_routed_experts, cfg.top_k, cfg.moe_intermediate
    dev = x.device
    _need(x, _BF16, (T, H), "x")
    _need(layer.gate_w, torch.float32, (E, H), "gate_w")
    _need(layer.w13_codes, torch.uint8, (E, 2 * I, H // 2), "w13_codes")
    _need(layer.w13_scales, torch.uint8, (E, 2 * I, H // 32), "w13_scales")
    _need(w2_codes, torch.uint8, (E, H, I // 32 * 12), "w2_codes")
    _need(w2_scales, (torch.int16, torch.uint16), (E, H, I // 32), "w2_scales")
    if w2_levels is not None:
        _need(w2_levels, torch.float32, (E, 8), "w2_levels")
    _need(layer.sh_w13, torch.int8, (2 * I, H), "sh_w13")
    _need(layer.sh_w2, torch.int8, (H, I), "sh_w2")
    V = 0
    if token_ids is not None:
        _need(token_ids, torch.int32, (T,), "token_ids")
        if layer.tid2eid is None:
            raise ValueError("hash layer needs layer.tid2eid")
        V = layer.tid2eid.shape[0]
    else:
        _need(layer.bias, torch.float32, (E,), "bias")
    if out is None:
        out = torch.empty(T, H, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=dev)
    ids = w = None
    if return_routing:
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
        w = torch.empty(T, k, dtype=torch.float32, device=dev)
    buf, nb = _ws(cfg, T, dev, ws)
    _check(lib().moe_forward_w2q3(
        ctypes.byref(cfg), T, _ptr(x), _ptr(layer.gate_w), _ptr(layer.bias), _ptr(layer.logit_offset),
        _ptr(token_ids), _ptr(layer.tid2eid if token_ids is not None else None), V, _ptr(layer.w13_codes),
        _ptr(layer.w13_scales), _ptr(w2_codes), _ptr(w2_scales), _ptr(w2_levels), _ptr(layer.sh_w13),
        _ptr(layer.sh_w13_scale), _ptr(layer.sh_w2), _ptr(layer.sh_w2_scale), _ptr(out), int(out_fp32),
        _ptr(ids), _ptr(w), _ptr(buf), nb, _stream(dev)), "moe_forward_w2q3")
    if return_routing:
        return out, (ids, w)
    return out


def forward_noalloc(cfg: MoeConfig, x, layer: DeviceLayer, token_ids=None, out_fp32=False, out=None,
                    routing_out=None):
    """``forward`` through moe_forward_noalloc (no workspace: the library's
    fixed per-GPU scratch). ``out`` and ``routing_out`` may be preallocated
    so that the call itself allocates nothing."""
    T, H, E, k, I = x.shape[0], cfg.hidden_size, cfg.n_routed_experts, cfg.top_k, cfg.moe_intermediate
    dev = x.device
    _need(x, _BF16, (T, H), "x")
    _need(layer.w13_codes, torch.uint8, (E, 2 * I, H // 2), "w13_codes")
    _need(layer.w2_codes, torch.uint8, (E, H, I // 2), "w2_codes")
    _need(layer.sh_w13, torch.int8, (2 * I, H), "sh_w13")
    _need(layer.sh_w2, torch.int8, (H, I), "sh_w2")
    V = 0
    if token_ids is not None:
        _need(token_ids, torch.int32, (T,), "token_ids")
        V = layer.tid2eid.shape[0]
    if out is None:
        out = torch.empty(T, H, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=dev)
    ids, w = routing_out if routing_out is not None else (None, None)
    _check(lib().moe_forward_noalloc(
        ctypes.byref(cfg), T, _ptr(x), _ptr(layer.gate_w), _ptr(layer.bias), _ptr(layer.logit_offset),
        _ptr(token_ids), _ptr(layer.tid2eid if token_ids is not None else None), V, _ptr(layer.w13_codes),
        _ptr(layer.w13_scales), _ptr(layer.w2_codes), _ptr(layer.w2_scales), _ptr(layer.sh_w13),
        _ptr(layer.sh_w13_scale), _ptr(layer.sh_w2), _ptr(layer.sh_w2_scale), _ptr(out), int(out_fp32),
        _ptr(ids), _ptr(w), _stream(dev)), "moe_forward_noalloc")
    return out


def layer_weights(layer: DeviceLayer) -> MoeLayerWeights:
    """The ``moe_layer_weights`` of a device layer (hash layer if it has a tid2eid table)."""
    def p(t):
        return None if t is None else t.data_ptr()
    V = 0 if layer.tid2eid is None else layer.tid2eid.shape[0]
    return MoeLayerWeights(p(layer.gate_w), p(layer.bias), p(layer.logit_offset), p(layer.tid2eid), V,
                           p(layer.w13_codes), p(layer.w13_scales), p(layer.w2_codes), p(layer.w2_scales),
                           p(layer.sh_w13), p(layer.sh_w13_scale), p(layer.sh_w2), p(layer.sh_w2_scale))


def forward_stack(cfg: MoeConfig, x, layers, token_ids=None, out_fp32=False, ws=None, act=None, out=None,
                  weights=None):
    """MoE layers back to back (moe_forward_stack): layer l + 1 reads layer l's
    bf16 output. ``layers``: DeviceLayers (hash layers carry tid2eid);
    ``weights``: their prebuilt ctypes array (optional, for repeated calls)."""
    T, H = x.shape[0], cfg.hidden_size
    dev = x.device
    _need(x, _BF16, (T, H), "x")
    n = len(layers)
    if weights is None:
        weights = (MoeLayerWeights * n)(*[layer_weights(L) for L in layers])
    if token_ids is not None:
        _need(token_ids, torch.int32, (T,), "token_ids")
    if act is None:
        act = torch.empty(2, T, H, dtype=torch.bfloat16, device=dev)
    if out is None:
        out = torch.empty(T, H, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=dev)
    buf, nb = _ws(cfg, T, dev, ws)
    _check(lib().moe_forward_stack(ctypes.byref(cfg), n, weights, T, _ptr(x), _ptr(token_ids), _ptr(act),
                                   _ptr(out), int(out_fp32), _ptr(buf), nb, _stream(dev)), "moe_forward_stack")
    return out


_linear_ws: dict = {}


def linear_w8a16(x, q, scale, groups=1, out_fp32=False, out=None, ws=None):
    """int8 per-channel linear (moe_linear_w8a16): x [T][groups*K] bf16, q
    [groups*N][K] int8, scale [groups*N] f32 -> [T][groups*N] (bf16 or f32)."""
    T = x.shape[0]
    dev = x.device
    _need(x, _BF16, None, "x")
    _need(q, torch.int8, None, "q")
    _need(scale, torch.float32, None, "scale")
    if x.dim() != 2 or q.dim() != 2 or x.shape[1] % groups or q.shape[0] % groups:
        raise ValueError("x [T][groups*K], q [groups*N][K] expected")
    K, N = x.shape[1] // groups, q.shape[0] // groups
    if q.shape[1] != K or scale.shape != (groups * N,):
        raise ValueError("shapes of q / scale do not match x")
    need = lib().moe_linear_workspace_size(T, K, N, groups)
    if need == 0:
        raise MoEError(MOE_EUNSUPPORTED, "moe_linear_workspace_size")
    if ws is None:
        key = torch.device(dev).index or 0
        ws = _linear_ws.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=dev)
            _linear_ws[key] = ws
    if out is None:
        out = torch.empty(T, groups * N, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=dev)
    _check(lib().moe_linear_w8a16(T, K, N, groups, _ptr(x), _ptr(q), _ptr(scale), _ptr(out), int(out_fp32),
                                  _ptr(ws), ws.numel(), _stream(dev)), "moe_linear_w8a16")
    return out

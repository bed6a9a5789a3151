"""The C ABI on the CPU: libmoe.so loads, exports every function include/moe.h
declares, and its host-side checks return the documented status codes
before anything is launched (no GPU is touched here)."""
import ctypes
import os
import re

import pytest

mx = pytest.importorskip("mxfp4_moe_expert_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_header_declares_the_five_entry_points():
    names = _declared_functions()
    for n in ("moe_route", "moe_hash_route", "moe_permute", "moe_expert_ffn", "moe_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = mx.lib()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    assert mx.version().count(".") == 2


def _cfg(**kw):
    return mx.config(**kw)


def test_workspace_size_host_logic():
    cfg = _cfg()
    L = mx.lib()
    n1 = L.moe_workspace_size(ctypes.byref(cfg), 1)
    n64 = L.moe_workspace_size(ctypes.byref(cfg), 64)
    n8k = L.moe_workspace_size(ctypes.byref(cfg), 8192)
    assert 0 < n1 < n64 < n8k and n8k % 256 == 0
    # dominated by the per-slot fp32 expert outputs and bf16 activations
    slots = 8192 * 6
    assert n8k >= slots * (4096 * 4 + 2048 * 2)
    assert n8k < slots * (4096 * 4 + 2048 * 2) * 1.3
    # invalid configurations and sizes
    for bad in (dict(hidden_size=100), dict(moe_intermediate=96), dict(top_k=0), dict(top_k=9),
                dict(n_routed_experts=5, top_k=6), dict(n_routed_experts=512)):
        assert L.moe_workspace_size(ctypes.byref(_cfg(**bad)), 1) == 0, bad
    assert L.moe_workspace_size(ctypes.byref(cfg), -1) == 0
    assert L.moe_workspace_size(ctypes.byref(cfg), 65537) == 0
    assert L.moe_workspace_size(None, 1) == 0
    # norm_topk_prob: only the model's renormalised weights are supported
    assert L.moe_workspace_size(ctypes.byref(_cfg(norm_topk_prob=0)), 1) == 0


def test_invalid_arguments_are_rejected_before_launch():
    L = mx.lib()
    cfg = _cfg()
    p = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails a host check
    nb = L.moe_workspace_size(ctypes.byref(cfg), 4)
    # null config
    assert L.moe_route(None, 4, p, p, p, None, p, p, p, nb, None) == mx.MOE_EINVAL
    # unsupported shape
    bad = _cfg(hidden_size=100)
    assert L.moe_route(ctypes.byref(bad), 4, p, p, p, None, p, p, p, nb, None) == mx.MOE_EUNSUPPORTED
    assert L.moe_forward(ctypes.byref(cfg), 70000, p, p, p, None, None, None, 0, p, p, p, p, p, p, p, p, p, 0,
                         None, None, p, nb, None) == mx.MOE_EUNSUPPORTED
    # negative T
    assert L.moe_route(ctypes.byref(cfg), -1, p, p, p, None, p, p, p, nb, None) == mx.MOE_EINVAL
    # null required pointers
    assert L.moe_route(ctypes.byref(cfg), 4, None, p, p, None, p, p, p, nb, None) == mx.MOE_EINVAL
    assert L.moe_hash_route(ctypes.byref(cfg), 4, p, None, p, 10, p, p, p, None) == mx.MOE_EINVAL
    assert L.moe_hash_route(ctypes.byref(cfg), 4, p, p, p, 0, p, p, p, None) == mx.MOE_EINVAL
    assert L.moe_permute(ctypes.byref(cfg), 4, p, None, p, p, p, nb, None) == mx.MOE_EINVAL
    assert L.moe_expert_ffn(ctypes.byref(cfg), 4, p, p, p, p, None, p, p, p, p, p, nb, None) == mx.MOE_EINVAL
    assert L.moe_forward(ctypes.byref(cfg), 4, p, p, p, None, None, None, 0, p, p, p, p, None, p, p, p, p, 0,
                         None, None, p, nb, None) == mx.MOE_EINVAL
    # a hash layer needs its table
    assert L.moe_forward(ctypes.byref(cfg), 4, p, p, None, None, p, None, 0, p, p, p, p, p, p, p, p, p, 0,
                         None, None, p, nb, None) == mx.MOE_EINVAL
    # misaligned pointers
    q = ctypes.c_void_p(0x100004)
    assert L.moe_route(ctypes.byref(cfg), 4, q, p, p, None, p, p, p, nb, None) == mx.MOE_EINVAL
    # workspace: null, misaligned, too small
    assert L.moe_route(ctypes.byref(cfg), 4, p, p, p, None, p, p, None, nb, None) == mx.MOE_EINVAL
    assert L.moe_route(ctypes.byref(cfg), 4, p, p, p, None, p, p, ctypes.c_void_p(0x100010), nb,
                       None) == mx.MOE_EINVAL
    assert L.moe_route(ctypes.byref(cfg), 4, p, p, p, None, p, p, p, nb - 1, None) == mx.MOE_EWORKSPACE
    assert L.moe_forward(ctypes.byref(cfg), 4, p, p, p, None, None, None, 0, p, p, p, p, p, p, p, p, p, 0,
                         None, None, p, 100, None) == mx.MOE_EWORKSPACE


def test_w2q3_host_checks():
    """moe_forward_w2q3: shapes without a 3-bit path are refused, and the
    usual pointer checks apply, before anything is launched."""
    L = mx.lib()
    p = ctypes.c_void_p(0x100000)
    q = ctypes.c_void_p(0x100004)
    small = _cfg(hidden_size=512, moe_intermediate=256, n_routed_experts=16)
    cfg = _cfg()
    for c, T, want in ((small, 4, mx.MOE_EUNSUPPORTED), (cfg, 70000, mx.MOE_EUNSUPPORTED)):
        nb = L.moe_workspace_size(ctypes.byref(c), min(T, 64))
        assert L.moe_forward_w2q3(ctypes.byref(c), T, p, p, p, None, None, None, 0, p, p, p, p, None, p, p, p, p,
                                  p, 0, None, None, p, nb, None) == want
    nb = L.moe_workspace_size(ctypes.byref(cfg), 4)
    # misaligned levels, null codes, too small a workspace
    assert L.moe_forward_w2q3(ctypes.byref(cfg), 4, p, p, p, None, None, None, 0, p, p, p, p, q, p, p, p, p, p, 0,
                              None, None, p, nb, None) == mx.MOE_EINVAL
    assert L.moe_forward_w2q3(ctypes.byref(cfg), 4, p, p, p, None, None, None, 0, p, p, None, p, None, p, p, p, p,
                              p, 0, None, None, p, nb, None) == mx.MOE_EINVAL
    assert L.moe_forward_w2q3(ctypes.byref(cfg), 4, p, p, p, None, None, None, 0, p, p, p, p, None, p, p, p, p, p,
                              0, None, None, p, 100, None) == mx.MOE_EWORKSPACE
    assert L.moe_forward_w2q3(ctypes.byref(cfg), 0, None, None, None, None, None, None, 0, None, None, None, None,
                              None, None, None, None, None, None, 0, None, None, None, 0, None) == mx.MOE_OK


def test_empty_batch_is_a_no_op():
    L = mx.lib()
    cfg = _cfg()
    assert L.moe_route(ctypes.byref(cfg), 0, None, None, None, None, None, None, None, 0, None) == mx.MOE_OK
    assert L.moe_forward(ctypes.byref(cfg), 0, None, None, None, None, None, None, 0, None, None, None, None,
                         None, None, None, None, None, 0, None, None, None, 0, None) == mx.MOE_OK


def test_status_strings():
    for s in (mx.MOE_OK, mx.MOE_EINVAL, mx.MOE_EUNSUPPORTED, mx.MOE_EWORKSPACE, mx.MOE_EHIP):
        assert mx.status_string(s)
    assert mx.status_string(12345) == "unknown status"


def test_binding_refuses_host_tensors():
    import torch

    cfg = _cfg(hidden_size=256, n_routed_experts=16, moe_intermediate=128)
    x = torch.zeros(2, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mx.route(cfg, x, torch.zeros(16, 256), torch.zeros(16))


def test_forward_schedule_host_logic():
    """The schedule query's argument checks and the choices that need no
    device (hash layers, batches past the single-launch sizes)."""
    L = mx.lib()
    cfg = _cfg()
    assert L.moe_forward_schedule(None, 1, 0) == mx.MOE_EINVAL
    assert L.moe_forward_schedule(ctypes.byref(cfg), -1, 0) == mx.MOE_EINVAL
    assert L.moe_forward_schedule(ctypes.byref(cfg), 65537, 0) == mx.MOE_EUNSUPPORTED
    assert L.moe_forward_schedule(ctypes.byref(_cfg(top_k=9)), 1, 0) == mx.MOE_EUNSUPPORTED
    small = _cfg(hidden_size=1024, moe_intermediate=512, n_routed_experts=32)
    assert mx.forward_schedule(small, 1, hash_layer=True) == "decode"  # no single-launch kernel at hidden 1024
    assert mx.forward_schedule(cfg, 17, hash_layer=True) == "decode"
    assert mx.forward_schedule(cfg, 65, hash_layer=True) == "large"
    assert mx.forward_schedule(cfg, 3) == "decode"
    assert mx.forward_schedule(cfg, 64) == "decode"
    assert mx.forward_schedule(cfg, 65) == "large"
    # hidden 1024 has no single-launch kernel: the three-launch schedule
    assert mx.forward_schedule(_cfg(hidden_size=1024, moe_intermediate=512, n_routed_experts=32), 1) == "tiny"


def test_read_probe_host_checks():
    """The measurement aid refuses bad arguments before launching anything."""
    L = mx.lib()
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    p16 = (p + 15) & ~15
    EINVAL = -1
    assert L.moe_read_probe(None, 16, 1, p16, None) == EINVAL
    assert L.moe_read_probe(p16, 16, 1, None, None) == EINVAL
    assert L.moe_read_probe(p16, 16, 0, p16, None) == EINVAL
    assert L.moe_read_probe(p16, 0, 1, p16, None) == EINVAL
    assert L.moe_read_probe(p16 + 4, 16, 1, p16, None) == EINVAL
    assert L.moe_read_probe(p16, 24, 1, p16, None) == EINVAL


def test_shape_cap_and_schedules():
    """H and I up to 8192 are accepted, larger ones rejected up front; where
    the tiny schedule's w2 launch would not fit a block's LDS (large I with
    several columns) the decode schedule is taken instead."""
    L = mx.lib()
    for H, I, ok in ((8192, 8192, True), (8192 + 128, 256, False), (256, 8192 + 128, False),
                     (16384, 256, False), (256, 16384, False)):
        cfg = _cfg(hidden_size=H, moe_intermediate=I, n_routed_experts=8, top_k=2)
        assert (L.moe_workspace_size(ctypes.byref(cfg), 5) > 0) == ok, (H, I)
        if not ok:
            assert L.moe_forward_schedule(ctypes.byref(cfg), 5, 0) == mx.MOE_EUNSUPPORTED
    small = _cfg(hidden_size=256, moe_intermediate=256, n_routed_experts=8, top_k=2)
    big_i = _cfg(hidden_size=256, moe_intermediate=8192, n_routed_experts=8, top_k=2)
    assert mx.forward_schedule(small, 5) == "tiny"
    assert mx.forward_schedule(big_i, 1) == "tiny"   # 3 columns of 16 KB fit
    assert mx.forward_schedule(big_i, 5) == "decode"  # 15 columns do not

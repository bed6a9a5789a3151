"""moe_forward_noalloc (the entry point without a workspace argument, for
callers that cannot allocate) against moe_forward, through the C ABI: the
same kernels on the same inputs, so the outputs must be bit-identical. Two
calls in a row on the one per-GPU scratch, the second with a smaller batch
(the decode schedule, then the single-launch one), then the same pair again;
a batch whose workspace exceeds the scratch is rejected before any launch."""
import numpy as np
import pytest
import torch

import synth
from parity import assert_outputs_close, reference_rows

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"
LAY = synth.Workload("lay", T=2, H=2048, E=64, k=6, I=1024, V=5000, bias_sigma=0.05, seed=7)


@pytest.fixture(scope="module")
def lay():
    L = synth.make_layer(LAY)
    return LAY, L, mx.DeviceLayer.from_host(L, DEV), mx.config_of(LAY)


def test_noalloc_matches_forward(lay):
    wl, L, D, cfg = lay
    for rnd in range(2):
        for T, sched in ((40, "decode"), (1, "single")):
            print(f"[noalloc round {rnd} T={T} {sched}]", flush=True)
            assert mx.forward_schedule(cfg, T) == sched
            xh = synth.make_tokens(wl, rep=300 + 10 * rnd + T, T=T)
            x = mx.bf16_from_numpy(xh, DEV)
            out = torch.empty(T, wl.H, dtype=torch.float32, device=DEV)
            got = mx.forward_noalloc(cfg, x, D, out_fp32=True, out=out)
            ref = mx.forward(cfg, x, D, out_fp32=True)
            torch.cuda.synchronize()
            assert got.data_ptr() == out.data_ptr()
            assert torch.isfinite(got).all()
            assert torch.equal(got, ref), f"T={T}: differs from moe_forward"
            if rnd == 0:
                _, o = reference_rows(L, xh, np.arange(T, dtype=np.int32))
                assert_outputs_close(got.cpu().numpy(), o, f"noalloc T={T}")


def test_noalloc_rejects_batches_beyond_the_scratch(lay):
    wl, L, D, cfg = lay
    cap = mx.lib().moe_noalloc_max_bytes()
    T = 64
    while mx.workspace_size(cfg, T) <= cap:
        T *= 2
    x = torch.zeros(T, wl.H, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mx.MoEError) as ei:
        mx.forward_noalloc(cfg, x, D)
    assert ei.value.status == mx.MOE_EWORKSPACE

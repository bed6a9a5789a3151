"""GPU parity of the int8 per-channel ("w8a16") linear layers of the model's
attention (page "deepseek-v4-mxfp4-int8 config.json", quantization_config,
config group linears_w8a16) through moe_linear_w8a16, against the oracle.
The pages give the layer names and the model's sizes, not the matrix shapes;
the shapes taken (hidden 4096, q_lora_rank 1024, 64 heads of head_dim 512, one
KV head, o_groups 8 of o_lora_rank 1024, 64 indexer heads of 128):
  fused_wqa_wkv  4096 -> 1024 + 512
  wq_b           1024 -> 64 x 512
  wo_a           8 groups of 4096 -> 1024 (grouped)
  wo_b           8192 -> 4096
  indexer.wq_b   1024 -> 64 x 128
  indexer.compressor.wkv 4096 -> 256
Weights are N(0, 0.02) quantised per row to int8; tokens N(0, 1) bf16. At
T <= 64 the streaming pass runs, above it the grouped GEMM; outputs of every
row (T <= 64) or of 24 sampled rows, rel L2 <= 5e-3, max abs <= 2e-2 rms."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_outputs_close

pytestmark = pytest.mark.gpu
mx = pytest.importorskip("mxfp4_moe_expert_amd")
DEV = "cuda"

SHAPES = {  # name: (K, N, groups)
    "fused_wqa_wkv": (4096, 1536, 1),
    "wq_b": (1024, 32768, 1),
    "wo_a": (4096, 1024, 8),
    "wo_b": (8192, 4096, 1),
    "indexer_wq_b": (1024, 8192, 1),
    "indexer_compressor_wkv": (4096, 256, 1),
}
_W = {}


def _weights(name):
    if name not in _W:
        K, N, G = SHAPES[name]
        sub = list(SHAPES).index(name)
        q, s = synth.int8_normal(0, synth.S_LINEAR, sub, G * N, K, 0.02)
        _W[name] = (q, s, torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV))
    return _W[name]


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("T", [1, 17, 64, 300])
def test_linear_w8a16_matches_oracle(name, T):
    K, N, G = SHAPES[name]
    q, s, qd, sd = _weights(name)
    print(f"[linear {name} T={T}]", flush=True)
    xh = synth.normal_bf16(0, synth.S_TOKENS, 700 + T, T * G * K).reshape(T, G * K)
    x = mx.bf16_from_numpy(xh, DEV)
    out = mx.linear_w8a16(x, qd, sd, groups=G, out_fp32=True)
    out_bf = mx.linear_w8a16(x, qd, sd, groups=G)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 64 else np.unique(np.linspace(0, T - 1, 24).astype(np.int64))
    ref = oracle.linear_w8a16(xh[rows], q, s, groups=G)
    assert_outputs_close(out.cpu().numpy()[rows], ref, f"{name} T={T}")
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


def test_linear_w8a16_arguments():
    L = mx.lib()
    assert L.moe_linear_workspace_size(4, 100, 256, 1) == 0    # K not a multiple of 128
    assert L.moe_linear_workspace_size(4, 128, 100, 1) == 0    # N not a multiple of 256
    assert L.moe_linear_workspace_size(4, 128, 256, 0) == 0
    assert L.moe_linear_workspace_size(0, 128, 256, 1) > 0
    x = torch.zeros(0, 128, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros(256, 128, dtype=torch.int8, device=DEV)
    sc = torch.ones(256, dtype=torch.float32, device=DEV)
    assert mx.linear_w8a16(x, q, sc).shape == (0, 256)


def test_linear_w8a16_interleaved_and_repeatable():
    """At decode sizes the split-K pass counts each row block's slices in
    arrival words that every call leaves at zero: calls of different shapes
    (split 16, 1 and 4 slices, grouped and plain) interleaved on one
    workspace give the same bits as the same calls alone, twice over."""
    cases = [("fused_wqa_wkv", 1), ("wq_b", 1), ("wo_a", 1), ("indexer_compressor_wkv", 5), ("wo_b", 33)]
    xs, first = {}, {}
    for name, T in cases:
        K, N, G = SHAPES[name]
        xs[name] = mx.bf16_from_numpy(
            synth.normal_bf16(0, synth.S_TOKENS, 750 + T, T * G * K).reshape(T, G * K), DEV)
    for rep in range(2):
        for name, T in cases:
            K, N, G = SHAPES[name]
            _, _, qd, sd = _weights(name)
            out = mx.linear_w8a16(xs[name], qd, sd, groups=G, out_fp32=True)
            torch.cuda.synchronize()
            if rep == 0:
                first[name] = out.clone()
            else:
                assert torch.equal(out, first[name]), name

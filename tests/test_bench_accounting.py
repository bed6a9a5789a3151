"""The benchmark's algorithmic work per step (the numerator of every roofline
figure it reports) against the byte and flop counts derived independently
from the layer's shapes: per expert, MXFP4 codes (half a byte per weight)
plus one E8M0 byte per 32 weights; the shared expert as int8 plus one fp32
scale per row; the fp32 router and its bias; bf16 tokens in and out; 2 flop
per multiply-add of the expert GEMMs."""
import numpy as np

import bench
import synth

H, I, E, K = 4096, 2048, 256, 6
W13_EXPERT = 2 * I * H // 2 + 2 * I * H // 32      # 8,912,896 B
W2_EXPERT = H * I // 2 + H * I // 32               # 4,456,448 B
SHARED = 2 * I * H + 2 * I * 4 + H * I + H * 4      # 25,198,592 B
ROUTER = E * H * 4 + E * 4                          # 4,195,328 B


def test_expert_and_shared_sizes():
    assert W13_EXPERT + W2_EXPERT == 13_369_344
    assert SHARED == 25_198_592
    assert ROUTER == 4_195_328


def test_decode_t1_bytes():
    """Six distinct experts, one token: 109,626,368 B."""
    ids = np.arange(K, dtype=np.int32).reshape(1, 1, K)
    a = bench.algorithmic(synth.WORKLOADS["decode_t1"], ids)
    assert a["distinct_experts"] == 6
    assert a["layer_bytes"] == 6 * (W13_EXPERT + W2_EXPERT) + SHARED + ROUTER + 1 * H * 2 * 2
    assert a["layer_bytes"] == 109_626_368


def test_decode_t64_bytes_count_distinct_experts():
    """The routed bytes scale with the distinct experts a batch touches (each
    read once), not with its T*k slots."""
    rng = np.random.default_rng(0)
    ids = np.stack([rng.choice(40, size=(64, K)) for _ in range(3)]).astype(np.int32)
    d = [len(set(s.ravel().tolist())) for s in ids]
    a = bench.algorithmic(synth.WORKLOADS["decode_t64"], ids)
    assert a["distinct_experts"] == sum(d) / 3
    want = sum(d) / 3 * (W13_EXPERT + W2_EXPERT) + SHARED + ROUTER + 64 * H * 2 * 2
    assert abs(a["layer_bytes"] - want) < 1e-6 * want


def test_prefill_and_hash_flops():
    """2 flop per multiply-add over every slot's w13 (H x 2I) and w2 (I x H)
    and every token's shared expert, 7 expert passes per token:
    2 * T * 7 * (H*2I + I*H) = 2,886,218,022,912 flop at T=8192 and
    1,443,109,011,456 at T=4096."""
    for name, T, want in (("prefill_t8192", 8192, 2_886_218_022_912), ("hash_t4096", 4096, 1_443_109_011_456)):
        ids = np.zeros((1, T, K), dtype=np.int32)
        a = bench.algorithmic(synth.WORKLOADS[name], ids)
        assert a["layer_flops"] == 2 * T * (K + 1) * (H * 2 * I + I * H)
        assert a["layer_flops"] == want
        assert a["w13_flops"] == 2 * T * K * H * 2 * I


def test_per_kernel_gemm_flops_sum_to_the_layer():
    """The per-kernel counter table prices each grouped GEMM of the large-batch
    schedule by its template arguments (format, mode): routed w13 and w2 over
    T*k slots, shared w13 and w2 + combine over T tokens. Their sum is the
    layer's expert flops, and the routed w13 figure is the dominant kernel's;
    the router is 2 flop per multiply-add of T x E x H."""
    wl = synth.WORKLOADS["prefill_t8192"]
    T = wl.T
    ids = np.zeros((1, T, K), dtype=np.int32)
    a = bench.algorithmic(wl, ids)
    names = {k: f"void moe::k_gemm<{k[0]}, {k[1]}>(moe::GemmArgs)" for k in ((0, 0), (0, 1), (1, 0), (1, 2))}
    f = {k: bench._gemm_flops(n, wl) for k, n in names.items()}
    assert f[(0, 0)] == a["w13_flops"] == 2.0 * T * K * H * 2 * I
    assert f[(0, 1)] == a["w2_flops"] == 2.0 * T * K * I * H
    assert f[(1, 0)] == 2.0 * T * H * 2 * I
    assert f[(1, 2)] == 2.0 * T * I * H
    assert sum(f.values()) == a["layer_flops"]
    assert bench._gemm_flops("moe::k_router_mfma(moe::RouterMfmaArgs)", wl) == a["router_flops"]
    # the 3-bit routed w2 GEMM (format 2) is priced as the MXFP4 one
    assert bench._gemm_flops("void moe::k_gemm<2, 1>(moe::GemmArgs)", wl) == f[(0, 1)]
    assert bench._gemm_flops("moe::k_perm_count(moe::PermArgs)", wl) is None

"""The streaming-read measurement kernel (moe_read_probe) on the GPU: it
reads buffers of several sizes, including a size that leaves a tail after
the unrolled loop, and leaves the sink untouched for buffers whose folded
words never take the marker value (all ones, all zeros)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mxfp4_moe_expert_amd")


@pytest.mark.parametrize("nbytes,blocks", [(64 << 20, 1024), ((1 << 20) + 16, 2048), (4096, 1)])
def test_read_probe_reads_and_leaves_sink(nbytes, blocks):
    print(f"[read probe {nbytes} B, {blocks} blocks]", flush=True)
    for fill in (1, 0):
        buf = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        sink = torch.full((blocks,), 7, dtype=torch.int32, device="cuda")
        mx.read_probe(buf, blocks, sink)
        torch.cuda.synchronize()
        assert torch.all(sink == 7)

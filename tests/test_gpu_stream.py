"""GPU check of the streaming-read measurement aid (moe_verify_stream_read):
it reads every 16-byte piece of the buffer at sizes that do not divide
evenly over its workgroups, and a thread stores to the sink only when the
XOR of what it read equals the kernel's fixed marker."""
import pytest
import torch

from speculative_block_verify_amd import api
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"
MARK = 0x9E3779B9  # the kernel's sink marker


def _sink(v):
    return torch.tensor([v], dtype=torch.int64).to(torch.int32).to(DEV)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 << 20, (64 << 20) + 48])
def test_zero_data_leaves_the_sink(nbytes):
    print("case: stream read of %d zero bytes" % nbytes, flush=True)
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    sink = _sink(12345)
    api.moe_verify_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 12345


def test_a_piece_whose_xor_is_the_marker_reaches_the_sink():
    """One 16-byte piece: the first thread of the one workgroup whose range
    holds it reads it alone; words (MARK, 0, 0, 0) XOR to the marker."""
    print("case: stream read marker piece", flush=True)
    words = torch.tensor([MARK, 0, 0, 0], dtype=torch.int64).to(torch.int32)
    buf = words.view(torch.uint8).to(DEV)
    sink = _sink(7)
    api.moe_verify_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MARK

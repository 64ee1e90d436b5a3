"""GPU: the streaming-read probe (a measurement aid) runs to completion and
leaves its sink untouched on ordinary data."""
import pytest
import torch

from decode_attention_paged_06_amd.ops import stream_read_probe
from gpu_util import device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,run_bytes", [(16, 0), (4096, 0), (1000 * 16, 0), (64 << 20, 0),
                                              (1024, 1024), (64 << 20, 8192), (64 << 20, 1 << 20)])
def test_stream_read_probe(nbytes, run_bytes):
    dev = device()
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    sink = torch.full((16 * 4096,), 7, dtype=torch.uint8, device=dev)
    stream_read_probe(src, sink, run_bytes=run_bytes)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())

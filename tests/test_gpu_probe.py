"""The streaming-read probe runs and writes nothing (its sink is stored only
when the folded data equals a constant that all-zero data cannot give)."""
import pytest
import torch

import decode_attention_paged_amd as pa

pytestmark = pytest.mark.gpu


def test_stream_read_writes_nothing():
    src = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")   # 4 MiB
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    pa.stream_read(src, sink)
    pa.stream_read(src[:1000].contiguous(), sink)                    # a ragged tail
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
    with pytest.raises(pa.PaError):
        pa.stream_read(src[:3], sink)                                # 12 bytes: not 16-byte rows

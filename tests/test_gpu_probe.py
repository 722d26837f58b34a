"""wsl_stream_read (the streaming-read ceiling probe used by bench.py): every 16-byte
word of the buffer is read, including the words past the last full pass of the grid."""

import pytest

import weight_streaming_linear_amd as wsl
from gpu_common import say

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("words,pos", [(1, 0), (256, 255), (65536 + 3, 65538), (8 * 524288 + 5, 8 * 524288 + 4),
                                       (8 * 524288 + 5, 3 * 524288 + 17), (20 * 524288, 20 * 524288 - 1),
                                       (262151, 262150), (262151, 131072)])
def test_stream_read_reads_every_word(words, pos):
    """A buffer of zeros with the magic value in one 16-byte word: the lane that reads
    that word XORs to the magic value and writes it to the sink.  Sizes from one word to
    160 MB reach every part of the kernel: no whole 1 KB unit per wave (word loop only),
    fewer rounds than loads in flight, the pipelined rounds with their remainder, and
    the units and words past the last whole round; without the plant the sink stays
    untouched."""
    import torch
    say(f"stream_read {words} words, plant at {pos}")
    buf = torch.zeros(words * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsl.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    buf[4 * pos + (pos % 4)] = MAGIC - (1 << 32)
    wsl.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC

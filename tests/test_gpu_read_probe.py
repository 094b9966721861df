"""The read-stream probe (a measurement aid of the benchmark, not a step of
the method) reads every 16-byte word of its buffer: a buffer of zeros whose
first or last word carries the marker makes the probe store the marker, and a
buffer of zeros leaves the sink alone, at sizes below, at and above one grid
stride and for several launch widths."""

import pytest
import torch

import int8_group_quantized_amd as q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [1, 3, 257, 4 * 256 * 7 + 5, (1 << 20) + 3])
@pytest.mark.parametrize("wgs", [1, 7, 2048, 65536])
@pytest.mark.parametrize("where", ["none", "first", "last"])
def test_probe_reads_every_word(words, wgs, where):
    print("read probe: words=%d workgroups=%d marker=%s" % (words, wgs, where), flush=True)
    buf = torch.zeros((words, 4), dtype=torch.int32, device="cuda")
    mark = q.READ_PROBE_MARK - (1 << 32)          # the same 32 bits as a signed int32
    if where == "first":
        buf[0, 0] = mark
    elif where == "last":
        buf[-1, 0] = mark
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    q.read_stream(buf, wgs, sink)
    torch.cuda.synchronize()
    got = int(sink[0].item()) & 0xFFFFFFFF
    assert got == (0 if where == "none" else q.READ_PROBE_MARK)

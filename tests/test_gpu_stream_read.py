"""The streaming-read probe reads every 16-byte word: a single word equal to the probe's
fixed value, anywhere in an otherwise zero buffer, makes the thread that read it store the
value; a zero buffer leaves the sink alone."""
import pytest
import torch

pytestmark = pytest.mark.gpu

MAGIC = 0x9e3779b9


@pytest.mark.parametrize("n_words,where", [(4, 0), (4 * 1000, 3999), (4 * 1_000_003, 4_000_004),
                                           (1 << 26, (1 << 26) - 1)])
def test_stream_read_sees_every_word(n_words, where):
    import long_context_decode_kvq_amd as kvq
    buf = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvq.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    buf[where] = MAGIC - (1 << 32)  # the same 32 bits as a signed int32
    kvq.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xffffffff == MAGIC

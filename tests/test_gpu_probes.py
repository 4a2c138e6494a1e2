"""The streaming-read ceiling probe (jq4k_probe_stream) reads every byte it
is given, in its documented pattern: thread t of workgroup w XORs the 16-byte
chunks 2304 w + 256 k + t, k = 0..8, and writes sink[t] only when that XOR
has the magic value.  A buffer that plants the value in exactly one thread's
chunks (split over several of them) shows each of them is read; a ragged
tail (the last workgroup's loads past the end repeat the last chunk) and the
argument checks are covered too."""
import numpy as np
import pytest

from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAGIC = 0x9E3779B9
NOT_WRITTEN = 0xDEADBEEF


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import q4_weight_only_amd as jq4k
    jq4k.raw()
    return jq4k


def _run(gpu, words):
    buf = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.full((256,), NOT_WRITTEN - (1 << 32), dtype=torch.int32, device="cuda:0")
    rc = gpu.raw().jq4k_probe_stream(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), None)
    assert rc == 0
    torch.cuda.synchronize()
    return sink.cpu().numpy().view(np.uint32)


def test_probe_stream_reads_every_chunk(gpu):
    # two workgroups; thread 37 of the second: its nine chunks carry three
    # words whose XOR is the magic value, every other chunk is zero
    chunks = np.zeros((2 * 2304, 4), np.uint32)
    parts = [0x12345678, 0x0F0F0F0F]
    parts.append(MAGIC ^ parts[0] ^ parts[1])
    for k, v in zip((0, 4, 8), parts):
        chunks[2304 + 256 * k + 37, k % 4] = v
    announce("probe_stream: planted value in one thread's chunks")
    sink = _run(gpu, chunks.reshape(-1))
    assert sink[37] == MAGIC
    assert all(sink[t] == NOT_WRITTEN for t in range(256) if t != 37)


def test_probe_stream_ragged_tail_and_checks(gpu):
    # 2304 + 5 chunks, the last one holding the magic value: the second
    # workgroup's loads past the end repeat that chunk, so threads 4 .. 255
    # read it nine times (XOR: the value) and threads 0 .. 3, whose first
    # load is one of the zero chunks 2304 .. 2307, eight times (XOR: zero)
    chunks = np.zeros((2304 + 5, 4), np.uint32)
    chunks[-1, 2] = MAGIC
    announce("probe_stream: ragged tail")
    sink = _run(gpu, chunks.reshape(-1))
    assert all(sink[t] == NOT_WRITTEN for t in range(4))
    assert all(sink[t] == MAGIC for t in range(4, 256))
    L = gpu.raw()
    buf = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    assert L.jq4k_probe_stream(buf.data_ptr(), 20, sink.data_ptr(), None) == -1   # not 16 B
    assert L.jq4k_probe_stream(buf.data_ptr() + 4, 16, sink.data_ptr(), None) == -1
    assert L.jq4k_probe_stream(None, 16, sink.data_ptr(), None) == -1
    assert L.jq4k_probe_stream(buf.data_ptr(), 0, sink.data_ptr(), None) == 0

"""The streaming-read probe (the achievable-bandwidth yardstick of the benchmark) reads every byte it is
given: its only store fires when a thread's sixteen words XOR to a marker value, so a buffer holding the
marker in exactly one word makes the sink receive it, and an all-zero buffer leaves the sink alone."""
import pytest

import verify_attention_loop_amd as vla

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MARKER = 0x9E3779B9


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    vla.load()


def _run(words):
    buf = words.view(torch.uint8)
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    print(f"probe read of {buf.numel()} bytes", flush=True)
    vla.lkv_probe_read(buf, buf.numel(), sink)
    torch.cuda.synchronize()
    return int(sink.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("chunks", [1, 3, 64])
def test_probe_reads_every_chunk(chunks):
    n_words = chunks * vla.PROBE_CHUNK // 4
    zeros = torch.zeros(n_words, dtype=torch.int32, device="cuda")
    assert _run(zeros) == 7
    # the marker in the last word of the buffer (last chunk, last thread, last load)
    w = torch.zeros(n_words, dtype=torch.int32)
    w[-1] = MARKER - (1 << 32)
    assert _run(w.cuda()) == MARKER
    # and in a word of the first chunk's second load (thread 1's words 1028..1031)
    w = torch.zeros(n_words, dtype=torch.int32)
    w[256 * 4 + 5] = MARKER - (1 << 32)
    assert _run(w.cuda()) == MARKER

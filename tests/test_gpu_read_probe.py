"""The plain streaming-read probe (osx_read_probe) reads every 32-bit word of its buffer exactly once.

Checked through its fold: the XOR of the sink words must equal the XOR of all
words of the buffer, computed on the host (a word skipped or read twice
changes it).  Sizes: below one load per thread, ragged against the grid and
the unroll, and the 2 GiB buffer the benchmark reads.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def xor_all(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.view(np.uint32)))


@pytest.mark.parametrize("n_words", [4, 4 * 1000, 4 * (2048 * 256 * 8 + 2048 * 256 * 3 + 17), 4 * (1 << 22) + 8])
def test_read_probe_reads_every_word_once(osx, n_words):
    print(f"case read probe {n_words} words", flush=True)
    host = np.random.default_rng(n_words).integers(0, 2 ** 32, n_words, dtype=np.uint64).astype(np.uint32)
    x = torch.from_numpy(host.view(np.int32)).cuda()
    sink = osx.read_probe(x)
    torch.cuda.synchronize()
    assert xor_all(sink.cpu().numpy()) == xor_all(host)


def test_read_probe_benchmark_size(osx):
    """2 GiB of int32 words w[i] = i: the XOR of 0 .. 2^29 - 1 is 0 (every run of 4 from a multiple of 4 cancels)."""
    n = 1 << 29
    print("case read probe 2 GiB", flush=True)
    x = torch.arange(n, dtype=torch.int32, device="cuda")
    sink = osx.read_probe(x)
    torch.cuda.synchronize()
    assert xor_all(sink.cpu().numpy()) == 0
    x[12345] = 0  # one word changed: the fold changes by exactly that word
    sink = osx.read_probe(x)
    torch.cuda.synchronize()
    assert xor_all(sink.cpu().numpy()) == 12345

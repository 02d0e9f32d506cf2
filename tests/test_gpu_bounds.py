"""GPU checks that the attention kernels touch nothing outside their tensors.

Q, K and V are views at the front of larger buffers whose tails (well over
five key blocks) hold NaN, and O and the log-sum-exp sit at the front of
buffers whose tails hold a sentinel pattern.  Rows past the end of a head
(the ragged last key block, the blocks the bf16 prefill's load stream runs
through after a workgroup's last tile, query rows past the last tile) must
read as zeros without touching that memory: a NaN read into K is masked,
but a NaN read into V turns 0 * NaN into NaN in the P V product, so any
out-of-range read shows up as a non-finite output.  Outputs must match the
oracle, and the sentinel tails must be unchanged (nothing is written past
O or the log-sum-exp).  Covers bf16 and fp32 prefill, causal and not, with
ragged key counts and padded head dimensions, and decode with one and with
several key splits.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TAIL_ROWS = 1024  # rows of NaN after each input: 16 bf16 blocks of 64 keys, 32 fp32 blocks of 32


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def front_view(t, tail_elems, fill):
    """A copy of tensor t at the front of a buffer with `tail_elems` more elements set to `fill`."""
    n = t.numel()
    buf = torch.empty(n + tail_elems, dtype=t.dtype, device=t.device)
    buf[n:] = fill
    buf[:n] = t.reshape(-1)
    return buf[:n].view(t.shape), buf


CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, D, causal
    ("bf16", 1, 4, 1, 200, 200, 128, True),
    ("bf16", 2, 4, 2, 150, 333, 128, False),
    ("bf16", 1, 2, 2, 100, 100, 64, False),
    ("bf16", 2, 8, 2, 97, 97, 48, True),       # padded head dimension
    ("bf16", 1, 4, 4, 70, 130, 112, False),    # padded head dimension
    ("bf16", 20, 32, 8, 100, 100, 64, True),   # persistent walk over 320 tiles
    ("f32", 1, 1, 1, 64, 100, 48, False),
    ("f32", 1, 2, 1, 100, 100, 128, True),
    ("f32", 1, 1, 1, 600, 600, 64, True),      # key slices + combine
    ("bf16", 3, 8, 2, 1, 77, 128, False),      # decode, one split
    ("bf16", 2, 16, 4, 1, 3001, 80, False),    # decode, key splits, padded head dimension
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_no_reads_or_writes_outside_the_tensors(osx, case):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case bounds {case}", flush=True)
    t = synth.random_attn(Sq * 7 + Sk, dtype, B, Hq, Hkv, Sq, Sk, D)
    nan = float("nan")
    q, _ = front_view(to_dev(t["q"]), TAIL_ROWS * D, nan)
    k, _ = front_view(to_dev(t["k"]), TAIL_ROWS * D, nan)
    v, _ = front_view(to_dev(t["v"]), TAIL_ROWS * D, nan)
    sentinel = -12288.0  # -3 * 2^12: exact in bf16 and fp32
    o, obuf = front_view(torch.full_like(q, nan), TAIL_ROWS * D, sentinel)
    lse, lbuf = front_view(torch.full(q.shape[:3], nan, dtype=torch.float32, device="cuda"), 4096, sentinel)
    osx.attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    got = to_f64(o)
    assert np.isfinite(got).all(), f"{case}: non-finite output (an out-of-range read)"
    check(got, oracle.attention(t["q"], t["k"], t["v"], causal=causal), dtype, f"bounds {case}")
    assert torch.isfinite(lse).all()
    n = q.numel()
    assert (obuf[n:].float() == sentinel).all(), f"{case}: written past the end of O"
    assert (lbuf[lse.numel():] == sentinel).all(), f"{case}: written past the end of the log-sum-exp"

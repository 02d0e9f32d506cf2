"""The debug build (extra full waits and workgroup barriers at every LDS stage
boundary, ``OSX_DEBUG_SYNC=1``) against the default build, bit for bit.

Only the timing differs between the two libraries: every wavefront runs the
same instructions on the same data in the same order.  A stage read before its
loads were complete, or overwritten while another wavefront still read it,
would give the default build different values on some run, so any difference
here names a missing wait or barrier.  Each case also meets the oracle's bar,
so the two builds cannot agree on a wrong answer.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def osx():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import online_softmax_02_amd as osx
    assert os.path.exists(osx.DEBUG_SYNC_LIB_PATH), \
        f"{osx.DEBUG_SYNC_LIB_PATH} is missing: build with `python -m online_softmax_02_amd.build`"
    return osx


def _both(osx, fn):
    """fn() through the default library, then through the debug build."""
    import torch
    a = fn()
    torch.cuda.synchronize()
    with osx.using_library(osx.DEBUG_SYNC_LIB_PATH):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    import torch
    a = a if isinstance(a, (tuple, list)) else (a,)
    b = b if isinstance(b, (tuple, list)) else (b,)
    for x, y in zip(a, b):
        xv = x.contiguous().view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32)
        yv = y.contiguous().view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)
        n = int((xv != yv).sum())
        assert n == 0, f"{what}: {n} of {xv.numel()} values differ between the default and the debug build"


ATTN_CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, d, causal
    ("bf16", 1, 8, 2, 700, 700, 128, True),     # several tiles, diagonal and ragged blocks
    ("bf16", 2, 4, 4, 333, 333, 64, False),     # d64, ragged tail
    ("bf16", 1, 4, 1, 257, 257, 80, True),      # padded head dim, G = 4
    ("f32", 1, 1, 1, 1024, 1024, 128, False),   # key split + combine
    ("f32", 2, 4, 2, 300, 300, 48, True),       # padded d, causal, GQA
    ("bf16", 4, 8, 2, 1, 5000, 128, False),     # decode
    ("bf16", 2, 8, 2, 1, 70000, 128, False),    # decode with key splits + combine
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_attention_debug_sync_bit_identical(osx, case):
    dtype, B, Hq, Hkv, Sq, Sk, d, causal = case
    print(f"debug-sync attention {case}", flush=True)
    t = synth.random_attn(41, dtype, B, Hq, Hkv, Sq, Sk, d)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    a, b = _both(osx, lambda: osx.attn_fwd(q, k, v, causal=causal, return_lse=True))
    _same(a, b, f"attention {case}")
    ref = oracle.attention(t["q"], t["k"], t["v"], causal=causal)
    check(to_f64(a[0]), ref, dtype, f"attention {case}")


def test_normalised_debug_sync_bit_identical(osx):
    t = synth.random_attn(42, "f32", 1, 2, 1, 1024, 1024, 128)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    a, b = _both(osx, lambda: osx.attn_fwd_normalised(q, k, v))
    _same(a, b, "normalised-output recurrence")
    check(to_f64(a), oracle.attention(t["q"], t["k"], t["v"]), "f32", "normalised")


@pytest.mark.parametrize("rows,cols", [(64, 200), (8, 3000), (1, 200000)], ids=["wave", "row", "split"])
def test_softmax_debug_sync_bit_identical(osx, rows, cols):
    import torch
    rng = np.random.default_rng([43, rows, cols])
    x = torch.from_numpy(rng.normal(0.0, 2.0, (rows, cols)).astype(np.float32)).cuda()
    a, b = _both(osx, lambda: osx.softmax_rows(x))
    _same(a, b, f"softmax {rows}x{cols}")
    y = a.cpu().numpy().astype(np.float64)
    assert np.abs(y - oracle.softmax_rows(x.cpu().numpy())).max() <= 1e-5

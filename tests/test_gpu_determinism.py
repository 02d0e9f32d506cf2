"""Run-to-run determinism: the same call twice, on two streams, gives identical bits.

Every kernel combines its partial results in a fixed order (no atomics on
values), so results must not depend on timing.  Covered: decode with one
split and with key splits (combine kernel), fp32 prefill with and without a
key split, the normalised-output recurrence, the row softmax's wavefront,
workgroup and split kernels (fp32, and bf16 with the causal mask), the
stash three-pass comparator and the unfused comparator.  (The atomic
three-pass comparator adds its partial sums in arrival order by design, so
its last bits may differ between runs; it is left out.)
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def twice(fn):
    """fn() on the current stream and on a second stream; both results, as raw bits."""
    a = fn()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b = fn()
    s.synchronize()
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    return bits(a), bits(b)


ATTN = [
    # dtype, B, Hq, Hkv, Sq, Sk, D, causal
    ("bf16", 64, 32, 8, 1, 2000, 128, False),   # decode, one split
    ("bf16", 2, 16, 4, 1, 5000, 128, False),    # decode, key splits + combine
    ("bf16", 1, 8, 2, 1, 3000, 48, False),      # decode, splits, padded head dim
    ("f32", 1, 1, 1, 1024, 1024, 128, False),   # fp32, key splits + combine
    ("f32", 4, 32, 8, 256, 256, 64, True),      # fp32, no split
    ("bf16", 2, 32, 8, 1024, 1024, 80, True),   # bf16 prefill, padded head dim
]


@pytest.mark.parametrize("case", ATTN, ids=lambda c: "-".join(map(str, c)))
def test_attention_deterministic(osx, case):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case determinism {case}", flush=True)
    t = synth.random_attn(3, dtype, B, Hq, Hkv, Sq, Sk, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    a, b = twice(lambda: osx.attn_fwd(q, k, v, causal=causal, return_lse=True)[0])
    assert torch.equal(a, b)
    if dtype == "f32":
        a, b = twice(lambda: osx.attn_fwd_normalised(q, k, v, causal=causal))
        assert torch.equal(a, b)


@pytest.mark.parametrize("shape,dtype,period", [((1000, 700), "f32", 0), ((300, 5000), "f32", 0),
                                                ((3, 300000), "f32", 0), ((4096, 2048), "bf16", 2048),
                                                ((2, 100000), "bf16", 0)],
                         ids=lambda c: str(c))
def test_softmax_deterministic(osx, shape, dtype, period):
    print(f"case softmax determinism {shape} {dtype} {period}", flush=True)
    x = np.random.default_rng(shape[1]).normal(0, 3, shape).astype(np.float32)
    xd = to_dev(synth.round_to_bf16_bits(x) if dtype == "bf16" else x)
    a, b = twice(lambda: osx.softmax_rows(xd, causal_period=period, scale=0.5))
    assert torch.equal(a, b)


def test_comparators_deterministic(osx):
    x = to_dev(np.random.default_rng(9).normal(0, 3, (2, 200000)).astype(np.float32))
    a, b = twice(lambda: osx.softmax_rows_3pass(x, osx.OSX_3PASS_STASH))
    assert torch.equal(a, b)
    t = synth.random_attn(4, "bf16", 1, 8, 2, 300, 300, 128)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    a, b = twice(lambda: osx.attn_fwd_unfused(q, k, v, causal=True))
    assert torch.equal(a, b)

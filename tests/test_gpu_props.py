"""Randomised GPU parity sweeps (hypothesis, derandomised so every run draws the same cases).

Small shapes drawn over the whole argument space of each entry point --
dtypes, GQA group sizes, causal or not, ragged sequence lengths, every head
dim of each dtype, column counts that take each softmax kernel (wavefront,
workgroup, split), causal periods and scales, the fp32 normalised-output
variant with and without key splits -- against the fp64 oracle at the
same bars as the fixed cases.  Outputs start NaN-poisoned, so every element
must be written.
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from tests.gpu_util import F32_ATOL, SOFTMAX_BF16_ATOL, SOFTMAX_BF16_RTOL, check, to_dev, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SWEEP = settings(max_examples=30, deadline=None, derandomize=True, print_blob=True)


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


@st.composite
def attn_cases(draw):
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    batch = draw(st.integers(1, 2))
    hkv = draw(st.integers(1, 2))
    groups = draw(st.sampled_from([1, 2, 3, 4, 8]))
    d = 16 * draw(st.integers(1, 8)) if dtype == "bf16" else 4 * draw(st.integers(1, 32))
    causal = draw(st.booleans())
    sq = draw(st.sampled_from([1, draw(st.integers(2, 160))]))
    sk = sq if (causal and sq > 1) else draw(st.integers(1, 200))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return dtype, batch, hkv * groups, hkv, sq, sk, d, causal, seed


@SWEEP
@given(case=attn_cases())
def test_attention_sweep(osx, case):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal, seed = case
    print(f"case sweep attn {case}", flush=True)
    t = synth.random_attn(seed, dtype, B, Hq, Hkv, Sq, Sk, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    osx.attn_fwd(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    check(to_f64(out), oracle.attention(t["q"], t["k"], t["v"], causal=causal), dtype, str(case))


@st.composite
def softmax_cases(draw):
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    rows = draw(st.integers(1, 40))
    cols = draw(st.sampled_from([draw(st.integers(1, 2048)), draw(st.integers(2049, 8192)),
                                 draw(st.integers(8193, 40000))]))
    period = draw(st.sampled_from([0, draw(st.integers(1, rows))]))
    scale = draw(st.sampled_from([1.0, draw(st.floats(0.05, 4.0))]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return dtype, rows, cols, period, scale, seed


@SWEEP
@given(case=softmax_cases())
def test_softmax_options_sweep(osx, case):
    dtype, rows, cols, period, scale, seed = case
    print(f"case sweep softmax {case}", flush=True)
    x = np.random.default_rng(seed).normal(0.0, 3.0, (rows, cols)).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_to_bf16_bits(x)
    xd = to_dev(x)
    y = torch.full_like(xd, float("nan"))
    osx.softmax_rows(xd, out=y, causal_period=period, scale=scale)
    torch.cuda.synchronize()
    got, ref = to_f64(y), oracle.softmax_rows(x, causal_period=period, scale=scale)
    assert np.isfinite(got).all(), case
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= F32_ATOL, (case, err.max())
    else:
        assert (err <= SOFTMAX_BF16_ATOL + SOFTMAX_BF16_RTOL * np.abs(ref)).all(), (case, err.max())


@SWEEP
@given(rows=st.integers(1, 6), cols=st.integers(1, 40000), method=st.sampled_from([1, 2]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_softmax_3pass_sweep(osx, rows, cols, method, seed):
    print(f"case sweep 3pass {(rows, cols, method, seed)}", flush=True)
    x = np.random.default_rng(seed).normal(0.0, 3.0, (rows, cols)).astype(np.float32)
    xd = to_dev(x)
    y = torch.full_like(xd, float("nan"))
    osx.softmax_rows_3pass(xd, method, out=y)
    torch.cuda.synchronize()
    check(to_f64(y), oracle.softmax_rows(x), "f32", f"3pass {(rows, cols, method)}")


@settings(max_examples=15, deadline=None, derandomize=True, print_blob=True)
@given(hkv=st.integers(1, 2), groups=st.sampled_from([1, 2, 4]), sq=st.integers(1, 140), sk=st.integers(1, 180),
       d=st.sampled_from([64, 128]), causal=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_unfused_sweep(osx, hkv, groups, sq, sk, d, causal, seed):
    if causal and sq > 1:
        sk = sq
    case = (hkv, groups, sq, sk, d, causal, seed)
    print(f"case sweep unfused {case}", flush=True)
    t = synth.random_attn(seed, "bf16", 1, hkv * groups, hkv, sq, sk, d)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    osx.attn_fwd_unfused(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    check(to_f64(out), oracle.attention(t["q"], t["k"], t["v"], causal=causal), "bf16", str(case))


@settings(max_examples=15, deadline=None, derandomize=True, print_blob=True)
@given(batch=st.integers(1, 2), hkv=st.integers(1, 2), groups=st.sampled_from([1, 2, 4]), sq=st.integers(1, 300),
       sk=st.integers(1, 700), d=st.integers(1, 32), causal=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_normalised_sweep(osx, batch, hkv, groups, sq, sk, d, causal, seed):
    if causal and sq > 1:
        sk = sq
    d *= 4
    case = (batch, hkv, groups, sq, sk, d, causal, seed)
    print(f"case sweep normalised {case}", flush=True)
    t = synth.random_attn(seed, "f32", batch, hkv * groups, hkv, sq, sk, d)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    osx.attn_fwd_normalised(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    check(to_f64(out), oracle.attention(t["q"], t["k"], t["v"], causal=causal), "f32", str(case))

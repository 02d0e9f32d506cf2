"""GPU parity where the running max moves mid-stream, and with explicit scales.

The online recurrence rescales the accumulator and the denominator by
2^(m_old - m_new) whenever a later block of keys raises a row's max (page
"softmax_attention", section 实现思路: after the block [1, 2, 3] the block
[4, 5, 10] multiplies everything kept so far by e^(3 - 10)).  The bf16 prefill
kernel moves its reference max only when a block's max exceeds it by more
than 8 log2 units, so N(0, 1) inputs never reach that branch after the first
block.  These cases are built so that they do: keys in late blocks scaled by
8 (exact in bf16: a power of two), inputs with standard deviation 4, and an
explicit scale of 1.0.  Each test first checks, on the fp64 inputs, that some
row's max over its later keys exceeds its max over the first key block by
more than 8 log2 units -- the kernel's trigger -- then compares the output
(and the log-sum-exp) element by element with the oracle.

Explicit ``scale`` values other than 1/sqrt(d) (0.3 and 1.0; page
"从零开始写Qwen3（五-其一）使用Triton实现自注意力", section 自注意力原理, scales
the scores by d^-1/2, which the argument replaces) go through every fused
path: bf16 prefill, fp32 prefill with and without a key split, decode with
one split and with several, the log-sum-exp output and the
normalised-output recurrence.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import LSE_BF16_ATOL, LSE_F32_ATOL, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RESCALE_SLACK_LOG2 = 8.0  # the bf16 prefill kernel's lazy-rescale threshold, in log2 units


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def _f64(a):
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def late_max_rise(q, k, block_n, causal, scale=None, heads=None):
    """Per (b, h, row): (max scaled score over visible keys >= block_n) - (max over keys < block_n), in log2 units.

    Computed in fp64 from the inputs; -inf where a row sees no later key."""
    q, k = _f64(q), _f64(k)
    B, Hq, Sq, D = q.shape
    G = Hq // k.shape[1]
    sc = (1.0 / math.sqrt(D) if scale is None else scale) * math.log2(math.e)
    out = {}
    for b, h in (heads or [(b, h) for b in range(B) for h in range(Hq)]):
        s = (q[b, h] @ k[b, h // G].T) * sc
        if causal and Sq > 1:
            s = np.where(np.tril(np.ones(s.shape, dtype=bool)), s, -np.inf)
        first = s[:, :block_n].max(axis=1)
        later = s[:, block_n:].max(axis=1) if s.shape[1] > block_n else np.full(Sq, -np.inf)
        out[(b, h)] = later - first
    return out


def assert_rescale_fires(osx, t, causal, scale=None, min_rows=1, heads=None):
    B, Hq, Sq, D = t["q"].shape
    _, Hkv, Sk, _ = t["k"].shape
    bn = osx.attn_plan(osx.OSX_BF16, B, Hq, Hkv, Sq, Sk, D, causal)["block_n"]
    rise = late_max_rise(t["q"], t["k"], bn, causal, scale, heads)
    n = sum(int((r > RESCALE_SLACK_LOG2).sum()) for r in rise.values())
    top = max(float(r.max()) for r in rise.values())
    print(f"rows whose max rises > {RESCALE_SLACK_LOG2} log2 units after block 0: {n} (largest rise {top:.1f})")
    assert n >= min_rows, "the inputs do not reach the mid-stream rescale"


def late_dominant_keys(seed, B, Hq, Hkv, S, D, boost=8.0, start=None):
    """N(0, 1) q, k, v with every key row from `start` (default S // 2) on multiplied by `boost`, rounded to bf16."""
    t = synth.random_attn(seed, "f32", B, Hq, Hkv, S, S, D)
    k = t["k"].copy()
    k[:, :, (S // 2 if start is None else start):, :] *= np.float32(boost)
    return {"q": synth.round_to_bf16_bits(t["q"]), "k": synth.round_to_bf16_bits(k),
            "v": synth.round_to_bf16_bits(t["v"])}


def _run(osx, t, causal, scale=None, lse=False, fn=None):
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    fn = fn or osx.attn_fwd
    if lse:
        l = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        fn(q, k, v, causal=causal, scale=scale, out=out, lse=l)
        torch.cuda.synchronize()
        return to_f64(out), l.cpu().numpy().astype(np.float64)
    fn(q, k, v, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    return to_f64(out)


def _check_lse(got, ref, dtype, what):
    assert np.isfinite(got).all(), f"{what}: non-finite lse"
    err = float(np.abs(got - ref).max())
    bar = LSE_F32_ATOL if dtype == "f32" else LSE_BF16_ATOL
    print(f"{what}: lse max abs err {err:.3e} (bar {bar})")
    assert err <= bar, f"{what}: lse max abs error {err:.3e} > {bar}"


# Multi-tile shapes: more row tiles than the GPU has workgroups, so every
# persistent workgroup walks several tiles (the running state restarts per tile).
PREFILL_SHAPES = [
    # B, Hq, Hkv, S, D, causal
    (2, 32, 8, 2048, 128, True),   # G = 4, 512 tiles of 64 rows
    (4, 16, 8, 1500, 64, False),   # G = 2, 384 tiles of 128 rows, ragged last block
    (2, 32, 8, 1100, 64, True),    # G = 4, d = 64, ragged
    (4, 16, 8, 1000, 128, False),  # G = 2, d = 128
]


@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_bf16_late_dominant_keys(osx, shape):
    B, Hq, Hkv, S, D, causal = shape
    print(f"case late keys x8 {shape}", flush=True)
    t = late_dominant_keys(sum(shape), B, Hq, Hkv, S, D)
    assert_rescale_fires(osx, t, causal, min_rows=S // 4, heads=[(0, 0), (B - 1, Hq - 1)])
    got, lse = _run(osx, t, causal, lse=True)
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], causal=causal, with_lse=True)
    err = check(got, ref, "bf16", f"late keys {shape}")
    print(f"{shape}: {got.size} elements, max abs err {err:.3e}")
    _check_lse(lse, ref_lse, "bf16", f"late keys {shape}")


@pytest.mark.parametrize("shape", [(2, 32, 8, 2048, 128, True), (4, 16, 8, 1500, 64, False)],
                         ids=lambda c: "-".join(map(str, c)))
def test_prefill_bf16_sigma4_inputs(osx, shape):
    """q, k ~ N(0, 16): scaled scores of standard deviation ~16 move most rows' max long after block 0.  v stays
    N(0, 1), so the bar's absolute term keeps its meaning (the output error scales with v)."""
    B, Hq, Hkv, S, D, causal = shape
    print(f"case sigma 4 {shape}", flush=True)
    t = synth.random_attn(sum(shape) + 1, "bf16", B, Hq, Hkv, S, S, D, scale_std=4.0)
    t["v"] = synth.random_attn(sum(shape) + 2, "bf16", B, Hq, Hkv, S, S, D)["v"]
    assert_rescale_fires(osx, t, causal, min_rows=S // 8, heads=[(0, 0), (B - 1, Hq - 1)])
    got, lse = _run(osx, t, causal, lse=True)
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], causal=causal, with_lse=True)
    err = check(got, ref, "bf16", f"sigma 4 {shape}")
    print(f"{shape}: max abs err {err:.3e}")
    _check_lse(lse, ref_lse, "bf16", f"sigma 4 {shape}")


def test_prefill_bf16_workload_shape_with_late_dominant_keys(osx):
    """The causal GQA prefill workload's shape (B 2, Hq 32, Hkv 8, S 4096, d 128) with keys 3072.. scaled by 8:
    every one of the 262144 output rows and its log-sum-exp against the oracle."""
    w = synth.WORKLOADS["gqa_prefill_bf16"]
    print("case workload shape, late keys x8", flush=True)
    t = late_dominant_keys(55, w.batch, w.heads_q, w.heads_kv, w.seq_q, w.head_dim, start=3072)
    assert_rescale_fires(osx, t, True, min_rows=512, heads=[(0, 0), (1, 31)])
    got, lse = _run(osx, t, True, lse=True)
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], causal=True, with_lse=True)
    err = check(got, ref, "bf16", "workload shape, late keys")
    print(f"workload shape, late keys: {got.size} elements, max abs err {err:.3e}")
    _check_lse(lse, ref_lse, "bf16", "workload shape, late keys")


# ------------------------------------------------------------------ explicit scales
SCALE_CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, D, causal, input std
    ("bf16", 2, 32, 8, 1100, 1100, 128, True, 1.0),   # prefill, multi-tile
    ("bf16", 1, 8, 2, 300, 333, 64, False, 1.0),      # prefill, ragged
    ("f32", 1, 1, 1, 1024, 1024, 64, True, 0.35),     # fp32, keys split over workgroups
    ("f32", 2, 64, 16, 256, 300, 32, False, 0.35),    # fp32, no split, ragged
    ("bf16", 64, 32, 8, 1, 1500, 128, False, 1.0),    # decode, one split
    ("bf16", 2, 16, 4, 1, 3000, 128, False, 1.0),     # decode, key splits + combine
]


@pytest.mark.parametrize("scale", [0.3, 1.0])
@pytest.mark.parametrize("case", SCALE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_explicit_scale(osx, case, scale):
    """O and the log-sum-exp with an explicit scale, against the oracle at the same scale.  fp32 inputs are drawn
    with a small standard deviation so the scaled scores stay O(1) and the 1e-5 bar measures the kernel, not fp32
    rounding of large scores."""
    dtype, B, Hq, Hkv, Sq, Sk, D, causal, std = case
    print(f"case scale {scale} {case}", flush=True)
    t = synth.random_attn(int(scale * 10) + Sq + Sk, dtype, B, Hq, Hkv, Sq, Sk, D, scale_std=std)
    got, lse = _run(osx, t, causal, scale=scale, lse=True)
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], causal=causal, scale=scale, with_lse=True)
    # the default scale would give a different answer: the argument is really used
    if scale != 1.0 / math.sqrt(D):
        dflt = oracle.attention_heads(t["q"], t["k"], t["v"], causal=causal, heads=[(0, 0)])
        assert np.abs(dflt[0, 0] - ref[0, 0]).max() > 1e-3
    err = check(got, ref, dtype, f"scale {scale} {case}")
    print(f"scale {scale} {case}: max abs err {err:.3e}")
    _check_lse(lse, ref_lse, dtype, f"scale {scale} {case}")
    if dtype == "bf16" and Sq > 1 and scale == 1.0:
        assert_rescale_fires(osx, t, causal, scale=scale, min_rows=1, heads=[(0, 0)])


@pytest.mark.parametrize("scale", [0.3, 1.0])
@pytest.mark.parametrize("case", [(1, 1, 1, 1024, 1024, 64, True), (2, 8, 2, 100, 150, 48, False)],
                         ids=lambda c: "-".join(map(str, c)))
def test_explicit_scale_normalised(osx, case, scale):
    """The normalised-output recurrence with an explicit scale (with a key split in the first case)."""
    B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case normalised scale {scale} {case}", flush=True)
    t = synth.random_attn(Sq + int(10 * scale), "f32", B, Hq, Hkv, Sq, Sk, D, scale_std=0.35)
    got, lse = _run(osx, t, causal, scale=scale, lse=True, fn=osx.attn_fwd_normalised)
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], causal=causal, scale=scale, with_lse=True)
    err = check(got, ref, "f32", f"normalised scale {scale} {case}")
    print(f"normalised scale {scale} {case}: max abs err {err:.3e}")
    _check_lse(lse, ref_lse, "f32", f"normalised scale {scale} {case}")

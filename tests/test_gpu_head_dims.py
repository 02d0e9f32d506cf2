"""GPU parity for every bf16 head dimension the ABI accepts: 16 k <= 128.

Head dims other than 64 and 128 run in the 64- or 128-wide kernels with the
missing columns read as zeros and never stored (page "softmax_attention",
section 实现思路, pads the head dimension up to the block width and masks the
padded lanes).  The prefill kernel (GQA, causal and not, ragged keys, a
persistent walk over more tiles than the GPU has workgroups) and the decode
kernel (one split, and key splits merged by the combine kernel) are compared
with the oracle element by element, with the log-sum-exp.  Outputs start
NaN-poisoned, so every element of the true width must be written.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import LSE_BF16_ATOL, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PADDED = [16, 32, 48, 80, 96, 112]


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def _run_and_check(osx, case, t):
    _, B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    osx.attn_fwd(q, k, v, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], causal=causal, with_lse=True)
    err = check(to_f64(out), ref, "bf16", str(case))
    lerr = float(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse).max())
    print(f"{case}: max abs err {err:.3e}, lse {lerr:.3e}")
    assert lerr <= LSE_BF16_ATOL


@pytest.mark.parametrize("d", PADDED)
@pytest.mark.parametrize("shape", [(1, 4, 1, 200, 200, True), (2, 4, 2, 130, 333, False),
                                   (8, 32, 8, 257, 257, True)],
                         ids=lambda c: "-".join(map(str, c)))
def test_prefill_bf16_padded_head_dims(osx, shape, d):
    B, Hq, Hkv, Sq, Sk, causal = shape
    case = ("bf16", B, Hq, Hkv, Sq, Sk, d, causal)
    print(f"case head dim {case}", flush=True)
    assert osx.attn_plan(osx.OSX_BF16, B, Hq, Hkv, Sq, Sk, d, causal)["kernel_name"] == "prefill_bf16"
    _run_and_check(osx, case, synth.random_attn(d + Sq, "bf16", B, Hq, Hkv, Sq, Sk, d))


@pytest.mark.parametrize("d", PADDED)
@pytest.mark.parametrize("shape", [(64, 8, 8, 1, 100), (4, 16, 4, 1, 1000), (2, 10, 2, 1, 33)],
                         ids=lambda c: "-".join(map(str, c)))
def test_decode_bf16_padded_head_dims(osx, shape, d):
    B, Hq, Hkv, Sq, Sk = shape
    case = ("bf16", B, Hq, Hkv, Sq, Sk, d, False)
    print(f"case decode head dim {case}", flush=True)
    p = osx.attn_plan(osx.OSX_BF16, B, Hq, Hkv, Sq, Sk, d)
    assert p["kernel_name"] == "decode_bf16"
    _run_and_check(osx, case, synth.random_attn(d + Sk, "bf16", B, Hq, Hkv, Sq, Sk, d))


def test_padded_head_dim_gqa_index_map_exact(osx):
    """V[b, kv] = 8b + kv gives O[b, h] = 8b + h // G exactly, at d = 48 (prefill) and d = 80 (decode)."""
    for Sq, D in ((70, 48), (1, 80)):
        B, Hq, Hkv, Sk = 2, 16, 4, 90
        rng = np.random.default_rng(D)
        q = rng.normal(size=(B, Hq, Sq, D)).astype(np.float32)
        k = rng.normal(size=(B, Hkv, Sk, D)).astype(np.float32)
        v = np.empty((B, Hkv, Sk, D), np.float32)
        for b in range(B):
            for kv in range(Hkv):
                v[b, kv] = 8 * b + kv
        q, k, v = (synth.round_to_bf16_bits(a) for a in (q, k, v))
        out = osx.attn_fwd(to_dev(q), to_dev(k), to_dev(v))
        torch.cuda.synchronize()
        got = to_f64(out)
        for b in range(B):
            for h in range(Hq):
                np.testing.assert_array_equal(got[b, h], 8 * b + h // (Hq // Hkv))

"""GPU parity of the normalised-output recurrence (osx_attn_fwd_normalised) against the fp64 oracle.

The kernel keeps O normalised after every block of keys (page "Puzzle 9:
Simple FlashAttention", the recurrence under its scalar FlashAttention spec).
Its result is the same attention output, so besides the per-key recurrence of
``oracle.recurrence.attention_normalised`` on the small ragged workload, the
plain definition is the oracle.  Cases: one head with a ragged key tail and
d = 48, GQA with and without the causal mask, key splits merged by the
normalised combine (one long head, an fp32 decode shape), the full-size fp32
workload with its planted key, and the log-sum-exp the same call writes.
Outputs start NaN-poisoned.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import recurrence
from tests.gpu_util import LSE_F32_ATOL, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def _run(osx, t, causal, want_lse=False):
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    if want_lse:
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        osx.attn_fwd_normalised(q, k, v, causal=causal, out=out, lse=lse)
        torch.cuda.synchronize()
        return to_f64(out), lse.cpu().numpy().astype(np.float64)
    osx.attn_fwd_normalised(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    return to_f64(out)


def test_normalised_small_ragged_matches_the_per_key_recurrence(osx):
    w = synth.WORKLOADS["attn_f32_m64_n100_d48"]
    t = synth.attn_inputs(w)
    print(f"case normalised {w.name}", flush=True)
    got = _run(osx, t, False)
    ref, _, _ = recurrence.attention_normalised(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0])
    check(got[0, 0], ref, "f32", f"normalised {w.name} vs recurrence")
    check(got, oracle.attention(t["q"], t["k"], t["v"]), "f32", f"normalised {w.name} vs definition")


CASES = [  # B, Hq, Hkv, Sq, Sk, D, causal
    (2, 4, 2, 130, 130, 64, True),
    (1, 3, 1, 257, 300, 128, False),
    (1, 1, 1, 600, 600, 64, True),    # keys split across workgroups, causal
    (1, 1, 1, 1000, 1000, 96, False),  # keys split, no mask
    (3, 4, 4, 1, 777, 32, False),     # one query row per head: split keys, ragged
    (1, 2, 1, 33, 5, 4, False),       # fewer keys than one block
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_normalised_matches_oracle(osx, case):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case normalised {case} plan {osx.attn_plan(osx.OSX_F32, B, Hq, Hkv, Sq, Sk, D, causal)}", flush=True)
    t = synth.random_attn(11, "f32", B, Hq, Hkv, Sq, Sk, D)
    got, lse = _run(osx, t, causal, want_lse=True)
    check(got, oracle.attention(t["q"], t["k"], t["v"], causal=causal), "f32", f"normalised {case}")
    err = float(np.abs(lse - oracle.attention_lse(t["q"], t["k"], causal=causal)).max())
    assert err <= LSE_F32_ATOL, f"{case}: lse max abs error {err:.3e}"


def test_normalised_full_size_planted_key(osx):
    """4096 x 4096, d = 128 with one dominant late key; 16 key slices merged by the normalised combine."""
    w = synth.WORKLOADS["attn_f32_4k_d128"]
    t = synth.attn_inputs(w)
    print(f"case normalised {w.name}", flush=True)
    assert osx.attn_plan(osx.OSX_F32, w.batch, w.heads_q, w.heads_kv, w.seq_q, w.seq_k, w.head_dim)["splits"] > 1
    got = _run(osx, t, False)
    err = check(got, oracle.attention(t["q"], t["k"], t["v"]), "f32", f"normalised {w.name}")
    print(f"normalised {w.name}: max abs err {err:.3e}")


def test_normalised_constant_values_and_single_key(osx):
    """V constant: every normalised step keeps O = that constant; one visible key (causal row 0): O = V[0].

    (Up to rounding: the weight of the lone key is 2^(fma(s, c, -m)) with m = s c rounded, so within
    an ulp or two of 1, and O = V[0] p / d' with d' = p.)"""
    S, D = 300, 64
    q = torch.randn(1, 2, S, D, device="cuda")
    k = torch.randn(1, 1, S, D, device="cuda") * 3.0
    v = torch.full((1, 1, S, D), 0.375, device="cuda")
    out = osx.attn_fwd_normalised(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert float((out - 0.375).abs().max()) <= 1e-6
    v2 = torch.randn(1, 1, S, D, device="cuda")
    out2 = osx.attn_fwd_normalised(q, k, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.allclose(out2[0, :, 0], v2[0, 0, 0][None].expand(2, D), rtol=1e-6, atol=0)

"""GPU parity of the log-sum-exp output (osx_attn_fwd_lse) against the fp64 oracle.

Every kernel path that can write it: bf16 prefill (4, 2 and 1 query heads per
workgroup, ragged and causal), fp32 prefill without and with a key split (the
combine kernel writes it), and decode (written by its combine kernel).  The
output O of the same call must equal osx_attn_fwd's bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import LSE_BF16_ATOL, LSE_F32_ATOL, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [  # dtype, B, Hq, Hkv, Sq, Sk, D, causal
    ("bf16", 1, 4, 1, 200, 200, 128, True),
    ("bf16", 2, 4, 2, 130, 130, 128, True),
    ("bf16", 1, 2, 2, 300, 333, 64, False),
    ("bf16", 1, 3, 1, 257, 257, 64, True),
    ("f32", 1, 1, 1, 600, 600, 64, True),     # keys split across workgroups
    ("f32", 2, 4, 2, 64, 100, 48, False),
    ("bf16", 4, 8, 2, 1, 1000, 128, False),   # decode
    ("bf16", 3, 16, 4, 1, 77, 64, False),     # decode, ragged
]


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_lse_matches_oracle(osx, case):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case lse {case}", flush=True)
    t = synth.random_attn(7, dtype, B, Hq, Hkv, Sq, Sk, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
    out, lse = osx.attn_fwd(q, k, v, causal=causal, return_lse=True, lse=lse)
    plain = osx.attn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if dtype == "bf16" else out, plain.view(torch.int16) if dtype == "bf16" else plain)
    check(to_f64(out), oracle.attention(t["q"], t["k"], t["v"], causal=causal), dtype, f"O {case}")
    ref = oracle.attention_lse(t["q"], t["k"], causal=causal)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    bar = LSE_F32_ATOL if dtype == "f32" else LSE_BF16_ATOL
    print(f"lse max abs err {err:.3e} (bar {bar})")
    assert err <= bar, f"{case}: lse max abs error {err:.3e} > {bar}"


def test_lse_of_constant_keys_is_log_count(osx):
    """K = 0: every score is 0, so LSE = log(number of visible keys) = log(i + 1) under the causal mask."""
    B, Hq, Hkv, S, D = 1, 4, 1, 300, 128
    q = torch.randn(B, Hq, S, D, device="cuda").bfloat16()
    k = torch.zeros(B, Hkv, S, D, device="cuda").bfloat16()
    v = torch.randn(B, Hkv, S, D, device="cuda").bfloat16()
    _, lse = osx.attn_fwd(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    want = np.log(np.arange(1, S + 1, dtype=np.float64))
    err = float(np.abs(lse.cpu().numpy()[0] - want[None, :]).max())
    assert err <= 1e-5, err  # P = 1 exactly in bf16: only fp32 rounding of the count remains


def test_lse_full_size_prefill_sampled_heads(osx):
    """The causal GQA prefill workload at full size: LSE of two (batch, head) slices against the oracle."""
    w = synth.WORKLOADS["gqa_prefill_bf16"]
    t = synth.attn_inputs(w)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    _, lse = osx.attn_fwd(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    got = lse.cpu().numpy()
    G = w.heads_q // w.heads_kv
    for b, h in [(0, 5), (1, 30)]:
        ref = oracle.attention_lse(t["q"][b:b + 1, h:h + 1], t["k"][b:b + 1, h // G:h // G + 1], causal=True)[0, 0]
        err = float(np.abs(got[b, h] - ref).max())
        print(f"b{b} h{h}: lse max abs err {err:.3e}")
        assert err <= LSE_BF16_ATOL

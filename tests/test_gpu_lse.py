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


@pytest.mark.parametrize("case", [("bf16", 2, 16, 4, 1, 5000, 128, False), ("f32", 1, 1, 1, 600, 600, 64, True)],
                         ids=lambda c: "-".join(map(str, c)))
def test_binding_allocated_workspace_and_lse(osx, case):
    """Problems that need a workspace (decode key splits, fp32 key splits), with the workspace and the log-sum-exp
    both allocated by the binding: the workspace must stay allocated until the launch (it once was freed first, and
    the log-sum-exp tensor then took its memory), also when the call runs on a side stream."""
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case binding workspace {case}", flush=True)
    assert osx.attn_fwd_workspace(osx.OSX_BF16 if dtype == "bf16" else osx.OSX_F32, B, Hq, Hkv, Sq, Sk, D,
                                  causal) > 0
    t = synth.random_attn(17, dtype, B, Hq, Hkv, Sq, Sk, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    ref = oracle.attention(t["q"], t["k"], t["v"], causal=causal)
    ref_lse = oracle.attention_lse(t["q"], t["k"], causal=causal)
    bar = LSE_F32_ATOL if dtype == "f32" else LSE_BF16_ATOL
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for stream in (None, s):
        out, lse = osx.attn_fwd(q, k, v, causal=causal, return_lse=True, stream=stream)
        torch.cuda.synchronize()
        check(to_f64(out), ref, dtype, f"binding workspace {case} stream={stream}")
        assert float(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse).max()) <= bar

"""osx_attn_fwd_noalloc: the attention call that allocates nothing and uses the library's static scratch.

Its output must equal osx_attn_fwd's (same plan, same kernels; the partial
states go to the static scratch instead of a caller's workspace) and meet the
oracle's bars, on two calls in a row, the second with a smaller problem (the
scratch keeps the first call's contents).  Problems that need more scratch
than the array holds are rejected on the host before anything is launched.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import LSE_BF16_ATOL, LSE_F32_ATOL, check, to_dev, to_f64

torch = pytest.importorskip("torch")

import online_softmax_02_amd as osx  # noqa: E402

F32, BF16 = osx.OSX_F32, osx.OSX_BF16


def test_noalloc_rejects_problems_beyond_the_scratch():
    """One fp32 head of 65408 queries and keys, d = 128: the key split needs 68 MB of partial states, more than the
    64 MiB scratch -> OSX_EWORKSPACE, decided on the host (no device call is made)."""
    need = osx.attn_plan(F32, 1, 1, 1, 65408, 65408, 128)["workspace_bytes"]
    assert need > osx.NOALLOC_SCRATCH_BYTES
    a, b, c, o = (ctypes.c_void_p(x) for x in (0x100000, 0x200000, 0x300000, 0x400000))
    st = osx.lib.osx_attn_fwd_noalloc(a, b, c, o, None, F32, 1, 1, 1, 65408, 65408, 128, 0, 0.0, None)
    assert st == osx.OSX_EWORKSPACE
    assert "static scratch" in osx.last_error() and str(need) in osx.last_error()
    # argument errors are reported as by osx_attn_fwd
    st = osx.lib.osx_attn_fwd_noalloc(a, b, c, o, None, BF16, 1, 6, 4, 8, 8, 64, 0, 0.0, None)
    assert st == osx.OSX_EINVAL
    # the largest split plans of the benchmark workloads fit
    assert osx.attn_plan(F32, 1, 1, 1, 4096, 4096, 128)["workspace_bytes"] <= osx.NOALLOC_SCRATCH_BYTES


PAIRS = [
    # (first, second): dtype, B, Hq, Hkv, Sq, Sk, D, causal -- the second problem is smaller
    (("f32", 1, 1, 1, 4096, 4096, 128, False), ("f32", 1, 1, 1, 600, 600, 64, True)),
    (("bf16", 2, 16, 4, 1, 5000, 128, False), ("bf16", 1, 8, 2, 1, 1000, 48, False)),
    (("bf16", 2, 32, 8, 512, 512, 128, True), ("bf16", 1, 4, 1, 200, 200, 64, True)),
]


def _call_both(case, seed):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    t = synth.random_attn(seed, dtype, B, Hq, Hkv, Sq, Sk, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    osx.attn_fwd_noalloc(q, k, v, out, causal=causal, lse=lse)
    ref_out, ref_lse = osx.attn_fwd(q, k, v, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    return t, out, lse, ref_out, ref_lse


@pytest.mark.gpu
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}-{p[0][4]}x{p[0][5]}")
def test_noalloc_matches_the_workspace_call_twice(pair):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    for i, case in enumerate(pair):
        print(f"case noalloc call {i + 1} {case}", flush=True)
        dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
        t, out, lse, ref_out, ref_lse = _call_both(case, 31 + i)
        bits = (lambda x: x.view(torch.int16)) if dtype == "bf16" else (lambda x: x.view(torch.int32))
        assert torch.equal(bits(out), bits(ref_out)), f"{case}: differs from osx_attn_fwd"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        check(to_f64(out), oracle.attention(t["q"], t["k"], t["v"], causal=causal), dtype, f"noalloc {case}")
        err = float(np.abs(lse.cpu().numpy().astype(np.float64) - oracle.attention_lse(t["q"], t["k"],
                                                                                      causal=causal)).max())
        assert err <= (LSE_F32_ATOL if dtype == "f32" else LSE_BF16_ATOL)

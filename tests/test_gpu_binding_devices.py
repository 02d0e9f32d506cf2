"""The binding's device handling: every tensor of a call must be on one CUDA
device, which is made current for the call (the C ABI plans and launches on the
current device).  A tensor elsewhere -- out, lse or a workspace in host memory
-- is rejected on the host before anything is launched, so no kernel ever sees
a host pointer.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def _qkv(dtype="f32", Sq=64, Sk=100, d=64):
    t = synth.random_attn(7, dtype, 1, 2, 1, Sq, Sk, d)
    return t, to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])


def test_host_out_is_rejected_before_launch(osx):
    t, q, k, v = _qkv()
    with pytest.raises(ValueError, match="one CUDA device"):
        osx.attn_fwd(q, k, v, out=torch.empty(q.shape, dtype=q.dtype))
    with pytest.raises(ValueError, match="one CUDA device"):
        osx.attn_fwd_normalised(q, k, v, out=torch.empty(q.shape, dtype=q.dtype))
    x = torch.randn(4, 300, device="cuda")
    with pytest.raises(ValueError, match="one CUDA device"):
        osx.softmax_rows(x, out=torch.empty(4, 300))
    with pytest.raises(ValueError, match="one CUDA device"):
        osx.softmax_rows_3pass(x, osx.OSX_3PASS_STASH, out=torch.empty(4, 300))
    with pytest.raises(ValueError, match="out must be a contiguous 4-D"):
        osx.attn_fwd_noalloc(q, k, v, torch.empty(q.shape, dtype=q.dtype))


def test_host_lse_and_workspace_are_rejected_before_launch(osx):
    t, q, k, v = _qkv()
    with pytest.raises(ValueError, match="one CUDA device"):
        osx.attn_fwd(q, k, v, return_lse=True, lse=torch.empty(q.shape[:3], dtype=torch.float32))
    need = osx.attn_fwd_workspace(osx.OSX_F32, 1, 2, 1, 64, 100, 64)
    with pytest.raises(ValueError, match="one CUDA device"):
        osx.attn_fwd(q, k, v, workspace=torch.empty(max(need, 16), dtype=torch.uint8))
    x = torch.randn(1, 300000, device="cuda")
    need = osx.softmax_rows_workspace(1, 300000)
    assert need > 0
    with pytest.raises(ValueError, match="one CUDA device"):
        osx.softmax_rows(x, workspace=torch.empty(need, dtype=torch.uint8))


def test_calls_after_a_rejected_call_are_unaffected(osx):
    t, q, k, v = _qkv()
    with pytest.raises(ValueError):
        osx.attn_fwd(q, k, v, out=torch.empty(q.shape, dtype=q.dtype))
    o = osx.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    check(to_f64(o), oracle.attention(t["q"], t["k"], t["v"]), "f32", "after a rejected call")


@pytest.mark.skipif(not torch.cuda.is_available() or torch.cuda.device_count() < 2, reason="needs two GPUs")
def test_tensors_on_a_device_that_is_not_current(osx):
    t = synth.random_attn(8, "bf16", 1, 4, 2, 300, 300, 128)
    dev = torch.device("cuda", 1)
    q, k, v = (to_dev(t[n], dev) for n in ("q", "k", "v"))
    with torch.cuda.device(0):
        o = osx.attn_fwd(q, k, v, causal=True)
        x = torch.randn(2, 200000, device=dev)
        y = osx.softmax_rows(x)
    torch.cuda.synchronize(dev)
    assert o.device == dev and y.device == dev
    check(to_f64(o), oracle.attention(t["q"], t["k"], t["v"], causal=True), "bf16", "device 1")
    assert np.abs(y.cpu().numpy().astype(np.float64) - oracle.softmax_rows(x.cpu().numpy())).max() <= 1e-5
    with pytest.raises(ValueError, match="stream belongs"):
        osx.softmax_rows(x, stream=torch.cuda.Stream(device=0))


def test_one_head_calls_take_a_2d_out(osx):
    """q, k, v given as 2-D [S, D] (one head): every attention call accepts a 2-D ``out`` like q and writes it,
    and returns 2-D results; the values match the oracle (fp32 bar)."""
    t, q, k, v = _qkv(Sq=64, Sk=100, d=48)
    q2, k2, v2 = q[0, 0].clone(), k[0, 0].clone(), v[0, 0].clone()  # head 0 as [S, D] (one KV head)
    ref = oracle.attention(t["q"][:, :1], t["k"], t["v"])[0, 0]
    for fn in (osx.attn_fwd, osx.attn_fwd_normalised):
        out = torch.full_like(q2, float("nan"))
        got = fn(q2, k2, v2, out=out)
        assert got.shape == q2.shape and got.data_ptr() == out.data_ptr()
        check(to_f64(out), ref, "f32", fn.__name__ + " 2-D out")
        check(to_f64(fn(q2, k2, v2)), ref, "f32", fn.__name__ + " 2-D")
    out = torch.full_like(q2, float("nan"))
    osx.attn_fwd_noalloc(q2, k2, v2, out)
    check(to_f64(out), ref, "f32", "noalloc 2-D out")
    tb, qb, kb, vb = _qkv("bf16", Sq=64, Sk=100, d=64)
    qb2, kb2, vb2 = qb[0, 0].clone(), kb[0, 0].clone(), vb[0, 0].clone()
    refb = oracle.attention(tb["q"][:, :1], tb["k"], tb["v"])[0, 0]
    out = torch.full_like(qb2, float("nan"))
    got = osx.attn_fwd_unfused(qb2, kb2, vb2, out=out)
    assert got.shape == qb2.shape and got.data_ptr() == out.data_ptr()
    check(to_f64(out), refb, "bf16", "unfused 2-D out")
    with pytest.raises(ValueError, match="contiguous"):
        osx.attn_fwd(q, k, v, workspace=torch.empty(64, 64, dtype=torch.uint8, device="cuda")[:, ::2])


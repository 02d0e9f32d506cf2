"""Attention calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The no-allocation entry point exists for code under graph capture, and
osx_attn_fwd with a caller's workspace and output allocates nothing either, so
both can be captured once the device's first call has run.  The library records
kernel launches only (no memset, copy or allocation).  Each graph is replayed
three times with new inputs written eagerly between the replays; every replay
must equal the eager call on the same inputs bit for bit (the same plan and
kernels run) and meet the oracle's bar.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, D, causal
    ("f32", 1, 1, 1, 2048, 2048, 128, False),   # key split: partial states in the workspace / static scratch
    ("bf16", 1, 8, 2, 700, 700, 128, True),     # persistent prefill, ragged tiles
    ("bf16", 2, 16, 4, 1, 20000, 128, False),   # decode with key splits and the combine kernel
]


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def _inputs(case, seed):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    return synth.random_attn(seed, dtype, B, Hq, Hkv, Sq, Sk, D)


def _same_bits(a, b, what):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    n = int((a.view(view) != b.view(view)).sum())
    assert n == 0, f"{what}: {n} values differ from the eager call"


@pytest.mark.parametrize("noalloc", [True, False], ids=["noalloc", "workspace"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_graph_replays_match_eager_calls(osx, case, noalloc):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"graph capture {case} noalloc={noalloc}", flush=True)
    t = _inputs(case, 11)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.empty_like(q)
    code = osx.OSX_F32 if dtype == "f32" else osx.OSX_BF16
    ws = torch.empty(max(osx.attn_fwd_workspace(code, B, Hq, Hkv, Sq, Sk, D, causal), 16), dtype=torch.uint8,
                     device="cuda")

    def call():
        if noalloc:
            osx.attn_fwd_noalloc(q, k, v, out, causal=causal)
        else:
            osx.attn_fwd(q, k, v, causal=causal, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # the device's first call (looks up the static scratch) runs outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(3):
        t = _inputs(case, 100 + rep)
        q.copy_(to_dev(t["q"]))
        k.copy_(to_dev(t["k"]))
        v.copy_(to_dev(t["v"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        eager = osx.attn_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        _same_bits(replayed, eager, f"{case} replay {rep}")
        check(to_f64(replayed), oracle.attention(t["q"], t["k"], t["v"], causal=causal), dtype,
              f"{case} replay {rep}")

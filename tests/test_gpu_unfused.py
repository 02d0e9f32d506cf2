"""GPU parity of the unfused attention comparator (osx_attn_fwd_unfused) against the fp64 oracle.

The comparator computes the same O as the single-pass kernels (bf16 bar
2e-2 + 1e-2|ref|).  Cases: ragged query and key counts (tails of the 128-row,
32-key and 64-key tiles), a key count that is not a multiple of 4 (scalar
score stores), GQA, both head dims, causal and not, one query row, and the
full-size causal GQA workload compared with the fused kernel in full and with
the oracle on sampled rows.
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


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (1, 2, 1, 200, 200, 64, True),
    (1, 4, 2, 100, 77, 128, False),     # Sk % 4 != 0: scalar score stores; ragged key block
    (2, 4, 1, 130, 130, 128, True),     # G = 4, two query tiles
    (1, 2, 2, 64, 300, 64, False),      # Sq < 128, keys over 5 blocks of 64
    (2, 8, 2, 1, 1000, 128, False),     # one query row (decode shape)
    (1, 4, 4, 257, 257, 128, True),     # MHA, 3 query tiles, one-row tail
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}h{}kv{}q{}k{}d{}{}".format(*c[:6], "c" if c[6] else ""))
def test_unfused_matches_oracle(osx, case):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case unfused {case}", flush=True)
    t = synth.random_attn(sum(case[:6]), "bf16", B, Hq, Hkv, Sq, Sk, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    osx.attn_fwd_unfused(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    check(to_f64(out), oracle.attention(t["q"], t["k"], t["v"], causal=causal), "bf16", str(case))


def test_unfused_explicit_scale(osx):
    t = synth.random_attn(4, "bf16", 1, 2, 1, 96, 96, 128)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    print("case unfused scale 0.3", flush=True)
    out = osx.attn_fwd_unfused(q, k, v, causal=True, scale=0.3)
    torch.cuda.synchronize()
    check(to_f64(out), oracle.attention(t["q"], t["k"], t["v"], causal=True, scale=0.3), "bf16", "scale 0.3")


def test_unfused_full_size_causal_gqa(osx):
    """B2 Hq32 Hkv8 S4096 d128 causal: the unfused O against the fused O everywhere, and against the
    oracle on sampled rows of several heads."""
    w = synth.WORKLOADS["gqa_prefill_bf16"]
    t = synth.attn_inputs(w)
    print(f"case unfused {w.name}", flush=True)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    fused = osx.attn_fwd(q, k, v, causal=True)
    unfused = torch.full_like(q, float("nan"))
    osx.attn_fwd_unfused(q, k, v, causal=True, out=unfused)
    torch.cuda.synchronize()
    got = to_f64(unfused)
    assert np.isfinite(got).all()
    both = np.abs(got - to_f64(fused))
    print(f"{w.name}: unfused vs fused max abs diff {both.max():.3e}")
    assert both.max() < 4e-2
    G = w.groups
    rows = [0, 1, 63, 64, 127, 128, 2047, 4000, 4095]
    for b, h in [(0, 0), (0, 5), (1, 31)]:
        ref = oracle.attention_rows(t["q"][b, h, rows], t["k"][b, h // G], t["v"][b, h // G], rows, causal=True,
                                    seq_q=w.seq_q)
        check(got[b, h, rows], ref, "bf16", f"unfused {w.name} b={b} h={h}")

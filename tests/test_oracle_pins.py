"""Pins of the fp64 oracle to facts fixed by the pages and by the mathematics.

Each test names what it pins.  A plausible slip anywhere in ``oracle/`` (a
dropped max shift, a wrong scale, softmax over the wrong axis, an off-by-one
causal mask, the wrong GQA head map, a transposed product, a zero-score tail)
fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import brute, recurrence
from tests.golden.load import load

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- worked example
def test_worked_rescale_example():
    """Page "softmax_attention", 实现思路: blocks [1,2,3] then [4,5,10]."""
    g = load("rescale_example.txt")
    row = np.array(g["block1"] + g["block2"], dtype=np.float64)
    y, hist = recurrence.softmax_online(row, block=len(g["block1"]), trace=True)
    (m1, l1, _), (m2, l2, alpha2) = hist
    assert m1 == g["max_after_block1"] and m2 == g["max_after_block2"]
    assert alpha2 == pytest.approx(math.exp(g["rescale_exponent"]), rel=1e-15)
    # denominator after block 1 is sum e^{x-3}; after block 2 it equals the direct sum e^{x-10}
    assert l1 == pytest.approx(math.exp(-2) + math.exp(-1) + 1.0, rel=1e-15)
    assert l2 == pytest.approx(math.fsum(math.exp(x - 10.0) for x in row), rel=1e-14)
    # the final row matches the oracle and an independent library softmax
    ref = scipy.special.softmax(row)
    np.testing.assert_allclose(y, ref, rtol=1e-13)
    np.testing.assert_allclose(oracle.softmax_rows(row[None])[0], ref, rtol=1e-13)


def test_block_invariant_holds_after_every_block():
    """Page "Softmax 算子的实现与优化", Online Softmax: l = sum_j e^{x_j - m} over what was seen."""
    x = RNG.normal(0, 3, 300)
    _, hist = recurrence.softmax_online(x, block=32, trace=True)
    for n, (m, l, _) in enumerate(hist):
        seen = x[: min((n + 1) * 32, x.shape[0])]
        assert m == seen.max()
        assert l == pytest.approx(math.fsum(np.exp(seen - m)), rel=1e-13)


# ---------------------------------------------------------------- softmax
def test_softmax_matches_library_and_sums_to_one():
    """Page "Puzzle 8: Long Softmax" spec shape [4,200]; rows sum to 1."""
    g = load("softmax_spec.txt")
    x = RNG.uniform(-10, 10, (g["rows"], g["cols"]))
    y = oracle.softmax_rows(x)
    np.testing.assert_allclose(y, scipy.special.softmax(x, axis=1), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, atol=1e-12)
    assert (y > 0).all()


@pytest.mark.parametrize("c", [-100.0, 37.5, 1e3])
def test_softmax_shift_invariance(c):
    """Page "Softmax 算子的实现与优化": a common shift leaves the softmax unchanged."""
    x = RNG.normal(0, 2, (3, 257))
    np.testing.assert_allclose(oracle.softmax_rows(x + c), oracle.softmax_rows(x), rtol=1e-10, atol=1e-300)


def test_softmax_large_inputs_do_not_overflow():
    """The max shift keeps e^x finite: equal huge logits give equal halves."""
    y = oracle.softmax_rows(np.array([[1000.0, 1000.0], [-1000.0, -1000.0]]))
    np.testing.assert_array_equal(y, 0.5)


def test_softmax_two_elements_is_logistic():
    """Closed form: softmax([a, b])[0] = 1 / (1 + e^{b-a})."""
    for a, b in [(0.0, 0.0), (3.0, -1.0), (-7.5, 2.25)]:
        y = oracle.softmax_rows(np.array([[a, b]]))[0]
        assert y[0] == pytest.approx(1.0 / (1.0 + math.exp(b - a)), rel=1e-15)
        assert y[1] == pytest.approx(1.0 / (1.0 + math.exp(a - b)), rel=1e-15)


def test_softmax_spike_closed_form():
    """A single spike s over N(0,4) noise: y[idx] = 1 / (1 + sum_{j != idx} e^{x_j - s})."""
    x = RNG.normal(0, 2, 1 << 16)
    idx = x.shape[0] - 1 - 123
    x[idx] = 50.0
    y = oracle.softmax_rows(x[None])[0]
    rest = np.delete(x, idx)
    assert y[idx] == pytest.approx(1.0 / (1.0 + math.fsum(np.exp(rest - 50.0))), rel=1e-14)
    np.testing.assert_allclose(y[:5], np.exp(x[:5] - 50.0) * y[idx], rtol=1e-12)


def test_softmax_brute_force():
    for n in (1, 2, 5, 33):
        x = RNG.normal(0, 4, n)
        np.testing.assert_allclose(oracle.softmax_rows(x[None])[0], brute.softmax(list(x)), rtol=1e-13)


# ---------------------------------------------------------------- attention
def _attn_single(q, k, v, **kw):
    return oracle.attention(q[None, None], k[None, None], v[None, None], **kw)[0, 0]


def test_attention_two_key_closed_form_pins_scale():
    """d=4, q=(2,0,0,0), k0=(1,0,0,0), k1=0: weight of key 0 is logistic(2*1/sqrt(4))."""
    q = np.array([[2.0, 0, 0, 0]])
    k = np.array([[1.0, 0, 0, 0], [0, 0, 0, 0]])
    v = np.array([[1.0, 2, 3, 4], [-1.0, 0, 5, 1]])
    w0 = 1.0 / (1.0 + math.exp(-1.0))
    o = _attn_single(q, k, v)
    np.testing.assert_allclose(o[0], w0 * v[0] + (1 - w0) * v[1], rtol=1e-15)
    # an explicit scale overrides 1/sqrt(d)
    o2 = _attn_single(q, k, v, scale=0.25)
    w0 = 1.0 / (1.0 + math.exp(-0.5))
    np.testing.assert_allclose(o2[0], w0 * v[0] + (1 - w0) * v[1], rtol=1e-15)
    # huge scores (1000 and 999 after scaling) must not overflow: the max shift is applied
    k3 = np.array([[1.0, 0, 0, 0], [0.999, 0, 0, 0]])
    o3 = _attn_single(np.array([[2000.0, 0, 0, 0]]), k3, v)
    w0 = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(o3[0], w0 * v[0] + (1 - w0) * v[1], rtol=1e-12)


def test_attention_weights_are_library_softmax():
    """With V = I (Sk = D) the output row is the weight row: library softmax of the scaled scores."""
    M, N = 7, 9
    q, k = RNG.normal(size=(M, N)), RNG.normal(size=(N, N))
    o = _attn_single(q, k, np.eye(N))
    ref = scipy.special.softmax(q @ k.T / math.sqrt(N), axis=1)
    np.testing.assert_allclose(o, ref, rtol=1e-13)
    np.testing.assert_allclose(o.sum(axis=1), 1.0, atol=1e-13)


def test_attention_constant_v_and_single_key():
    """Weights sum to 1: V = v0 everywhere gives O = v0; one key gives O = V[0]."""
    q, k = RNG.normal(size=(5, 8)), RNG.normal(size=(11, 8))
    v0 = RNG.normal(size=8)
    o = _attn_single(q, k, np.tile(v0, (11, 1)))
    np.testing.assert_allclose(o, np.tile(v0, (5, 1)), rtol=1e-14, atol=1e-15)
    v = RNG.normal(size=(1, 8))
    np.testing.assert_allclose(_attn_single(q, k[:1], v), np.tile(v[0], (5, 1)), rtol=1e-15)


def test_attention_shift_invariance_in_keys():
    """Adding one vector u to every key shifts each score row by a constant: O unchanged."""
    q, k, v = RNG.normal(size=(6, 16)), RNG.normal(size=(20, 16)), RNG.normal(size=(20, 16))
    u = RNG.normal(size=16) * 3
    np.testing.assert_allclose(_attn_single(q, k + u, v), _attn_single(q, k, v), rtol=1e-11, atol=1e-12)


def test_ragged_tail_rule():
    """Page "softmax_attention": N=100 in 32-row blocks; the tail must be -inf, not score 0."""
    g = load("ragged_tail.txt")
    N, blk = g["n_keys"], g["block"]
    last = (N - 1) // blk * blk
    assert last == g["last_block_first"] and last + blk - 1 == g["last_block_last"]
    assert N - 1 == g["last_valid"]
    q, k, v = RNG.normal(size=(8, 48)), RNG.normal(size=(N, 48)), RNG.normal(size=(N, 48))
    ref = _attn_single(q, k, v)
    good = recurrence.attention_blockwise(q, k, v, block=blk, tail="neg_inf")
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-13)
    bad = recurrence.attention_blockwise(q, k, v, block=blk, tail="zero_score")
    assert np.abs(bad - ref).max() > 1e-3


def test_recurrence_matches_definition_causal():
    q, k, v = RNG.normal(size=(40, 8)), RNG.normal(size=(40, 8)), RNG.normal(size=(40, 8))
    ref = _attn_single(q, k, v, causal=True)
    np.testing.assert_allclose(recurrence.attention_blockwise(q, k, v, block=16, causal=True), ref,
                               rtol=1e-12, atol=1e-13)


def test_closed_form_causal():
    """Page "从零开始写Qwen3…", softmax section: keep col <= row.  K = 0 makes the weights
    uniform over the visible keys; V[j, c] = bit c of j gives O[i,c] = #{j<=i: bit c}/(i+1)."""
    S, D = 70, 8
    j = np.arange(S)
    v = ((j[:, None] >> np.arange(D)[None, :]) & 1).astype(np.float64)
    o = _attn_single(RNG.normal(size=(S, D)), np.zeros((S, D)), v, causal=True)
    expect = np.cumsum(v, axis=0) / (j[:, None] + 1)
    np.testing.assert_allclose(o, expect, rtol=1e-14, atol=1e-15)


def test_causal_single_query_row_is_unmasked():
    """The eager reference applies the causal mask only when there is more than one query row."""
    q, k, v = RNG.normal(size=(1, 8)), RNG.normal(size=(9, 8)), RNG.normal(size=(9, 8))
    np.testing.assert_allclose(_attn_single(q, k, v, causal=True), _attn_single(q, k, v), rtol=1e-15)


def test_closed_form_gqa_head_map():
    """Page "从零开始写Qwen3…", section GQA: query head h reads KV head h // G.
    V[b, kv] = 8b + kv (constant) gives O[b, h] = 8b + h // G."""
    g = load("gqa_heads.txt")
    B, Hq, Hkv, S, D = 2, g["heads_q"], g["heads_kv"], 5, 4
    assert Hq // Hkv == g["groups"]
    q, k = RNG.normal(size=(B, Hq, S, D)), RNG.normal(size=(B, Hkv, S, D))
    v = np.empty((B, Hkv, S, D))
    for b in range(B):
        for kv in range(Hkv):
            v[b, kv] = 8 * b + kv
    o = oracle.attention(q, k, v, causal=True)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(o[b, h], 8 * b + g["kv_of_q"][h], rtol=1e-14)


def test_brute_force_small_shapes():
    """All small shapes B,Hkv<=2, G<=2, Sq,Sk<=4, d<=3, causal on/off (Sq==Sk when causal)."""
    n = 0
    for B, Hkv, G, Sq, Sk, D, causal in itertools.product((1, 2), (1, 2), (1, 2), (1, 2, 4), (1, 3, 4),
                                                           (1, 3), (False, True)):
        if causal and Sq > 1 and Sq != Sk:
            continue
        q = RNG.normal(size=(B, Hkv * G, Sq, D))
        k = RNG.normal(size=(B, Hkv, Sk, D))
        v = RNG.normal(size=(B, Hkv, Sk, D))
        got = oracle.attention(q, k, v, causal=causal)
        ref = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), causal=causal))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
        n += 1
    assert n > 100


def test_attention_rows_matches_brute_and_full():
    B, Hq, Hkv, S, D = 1, 4, 2, 6, 3
    q = RNG.normal(size=(B, Hq, S, D))
    k = RNG.normal(size=(B, Hkv, S, D))
    v = RNG.normal(size=(B, Hkv, S, D))
    ref = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), causal=True))
    rows = [0, 3, 5]
    for h in range(Hq):
        got = oracle.attention_rows(q[0, h, rows], k[0, h // 2], v[0, h // 2], rows, causal=True, seq_q=S)
        np.testing.assert_allclose(got, ref[0, h, rows], rtol=1e-12, atol=1e-13)


def test_bf16_bits_decoding():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits),
                                  [1.0, -1.0, 3.140625, 0.0, 3.3895313892515355e38])


# ---------------------------------------------------------------- log-sum-exp of the scores
def test_lse_closed_form_counts_visible_keys():
    """K = 0 makes every score 0: LSE is log(number of visible keys), log(i + 1) under the causal mask."""
    B, Hq, Hkv, S, D = 1, 2, 1, 9, 4
    q = RNG.standard_normal((B, Hq, S, D))
    k = np.zeros((B, Hkv, S, D))
    np.testing.assert_allclose(oracle.attention_lse(q, k), np.full((B, Hq, S), math.log(S)), rtol=1e-15)
    want = np.log(np.arange(1, S + 1, dtype=np.float64))
    np.testing.assert_allclose(oracle.attention_lse(q, k, causal=True)[0, 1], want, atol=1e-15)


def test_lse_two_keys_is_logaddexp():
    """d=4, q=(2,0,0,0), k0=(1,0,0,0), k1=0: scores 1 and 0, LSE = log(e + 1); the scale argument applies."""
    q = np.array([[[[2.0, 0, 0, 0]]]])
    k = np.array([[[[1.0, 0, 0, 0], [0, 0, 0, 0]]]])
    assert abs(oracle.attention_lse(q, k)[0, 0, 0] - math.log(math.e + 1.0)) < 1e-15
    assert abs(oracle.attention_lse(q, k, scale=0.25)[0, 0, 0] - math.log(math.exp(0.5) + 1.0)) < 1e-15
    # huge scores stay finite: max shift applied
    big = np.array([[[[2000.0, 0, 0, 0]]]])
    assert abs(oracle.attention_lse(big, k)[0, 0, 0] - (1000.0 + math.log1p(math.exp(-1000.0)))) < 1e-12


def test_lse_shifts_with_a_common_key_offset():
    """Adding u to every key adds scale * q_i . u to every score of row i, hence to its LSE."""
    q = RNG.standard_normal((1, 2, 6, 8))
    k = RNG.standard_normal((1, 1, 11, 8))
    u = RNG.standard_normal(8)
    base = oracle.attention_lse(q, k)
    shifted = oracle.attention_lse(q, k + u)
    np.testing.assert_allclose(shifted, base + (q @ u) / math.sqrt(8), rtol=1e-12, atol=1e-12)


def test_lse_matches_library_logsumexp_and_normalises_the_weights():
    """scipy's logsumexp of the masked scores; exp(S - LSE) are the attention weights (they sum to 1)."""
    q = RNG.standard_normal((2, 4, 7, 5))
    k = RNG.standard_normal((2, 2, 7, 5))
    lse = oracle.attention_lse(q, k, causal=True)
    for b, h in itertools.product(range(2), range(4)):
        s = q[b, h] @ k[b, h // 2].T / math.sqrt(5)
        s = np.where(np.tril(np.ones((7, 7), dtype=bool)), s, -np.inf)
        np.testing.assert_allclose(lse[b, h], scipy.special.logsumexp(s, axis=-1), rtol=1e-13)
        np.testing.assert_allclose(np.exp(s - lse[b, h][:, None]).sum(-1), 1.0, rtol=1e-13)


def test_lse_brute_force_small_shapes():
    for (B, Hkv, G, Sq, Sk, D, causal) in [(1, 1, 1, 3, 5, 2, False), (2, 2, 2, 4, 4, 3, True), (1, 2, 2, 1, 5, 4, True)]:
        q = RNG.standard_normal((B, Hkv * G, Sq, D))
        k = RNG.standard_normal((B, Hkv, Sk, D))
        want = np.array(brute.attention_lse(q.tolist(), k.tolist(), causal=causal))
        np.testing.assert_allclose(oracle.attention_lse(q, k, causal=causal), want, rtol=1e-12, atol=1e-12)


def test_lse_is_the_recurrence_final_state():
    """The blockwise recurrence's last (m, l) gives m + log l = LSE (the state page P4 carries block to block)."""
    q = RNG.standard_normal((5, 6))
    k = RNG.standard_normal((70, 6))
    v = RNG.standard_normal((70, 6))
    _, traces = recurrence.attention_blockwise(q, k, v, block=32, trace=True)
    lse = oracle.attention_lse(q[None, None], k[None, None])[0, 0]
    for i, hist in enumerate(traces):
        m, l, _ = hist[-1]
        assert abs(m + math.log(l) - lse[i]) < 1e-12


# ---------------------------------------------------------------- softmax options
def test_softmax_causal_constant_rows_are_uniform_over_visible_columns():
    """Constant logits: row r of each [P, cols] matrix is 1/(r mod P + 1) on columns <= r mod P, 0 after."""
    P, cols = 5, 7
    y = oracle.softmax_rows(np.full((2 * P, cols), 3.25), causal_period=P)
    for r in range(2 * P):
        lim = min(cols, r % P + 1)
        np.testing.assert_allclose(y[r, :lim], 1.0 / lim, rtol=1e-15)
        assert (y[r, lim:] == 0).all()


def test_softmax_scale_two_elements_is_logistic():
    """softmax(scale * [a, b])[0] = 1 / (1 + e^{scale (b - a)})."""
    for a, b, sc in [(3.0, -1.0, 0.125), (-7.5, 2.25, 2.0)]:
        y = oracle.softmax_rows(np.array([[a, b]]), scale=sc)[0]
        assert y[0] == pytest.approx(1.0 / (1.0 + math.exp(sc * (b - a))), rel=1e-15)


def test_softmax_masked_matches_library_on_the_visible_prefix():
    x = RNG.normal(0, 3, (12, 9))
    y = oracle.softmax_rows(x, causal_period=6, scale=0.5)
    for r in range(12):
        lim = r % 6 + 1
        np.testing.assert_allclose(y[r, :lim], scipy.special.softmax(0.5 * x[r, :lim]), rtol=1e-13)
        np.testing.assert_allclose(y[r].sum(), 1.0, rtol=1e-13)


def test_softmax_masked_brute_force_and_bf16_decoding():
    x = RNG.normal(0, 2, (7, 5))
    np.testing.assert_allclose(oracle.softmax_rows(x, causal_period=3, scale=1.5),
                               brute.softmax_masked(x.tolist(), 3, 1.5), rtol=1e-13, atol=1e-300)
    bits = np.array([[0x3F80, 0x4000, 0xC040]], dtype=np.uint16)  # 1, 2, -3 in bf16
    np.testing.assert_allclose(oracle.softmax_rows(bits), oracle.softmax_rows(np.array([[1.0, 2.0, -3.0]])),
                               rtol=1e-15)


# ---------------------------------------------------------------- normalised-output recurrence
def test_normalised_recurrence_matches_definition():
    """Page "Puzzle 9: Simple FlashAttention": the normalised recurrence ends at softmax(x) V, no final division."""
    for causal in (False, True):
        M, N, D = (9, 9, 5) if causal else (7, 40, 5)
        q = RNG.standard_normal((M, D)) * 2.0
        k = RNG.standard_normal((N, D))
        v = RNG.standard_normal((N, D))
        o, _, _ = recurrence.attention_normalised(q, k, v, causal=causal)
        ref = oracle.attention(q[None, None], k[None, None], v[None, None], causal=causal)[0, 0]
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
        want = np.array(brute.attention(q[None, None].tolist(), k[None, None].tolist(), v[None, None].tolist(),
                                        causal=causal))[0, 0]
        np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-13)


def test_normalised_output_is_the_prefix_softmax_after_every_key():
    """O'_i is the attention output over keys 1..i at every step (the invariant that makes O' normalised)."""
    D = 4
    q = RNG.standard_normal((3, D))
    k = RNG.standard_normal((25, D))
    k[11] *= 6.0  # a late key that moves the running max by a lot
    v = RNG.standard_normal((25, D))
    scale = 0.7
    _, _, _, hist = recurrence.attention_normalised(q, k, v, scale=scale, trace_row=1)
    x = (k @ q[1]) * scale
    assert len(hist) == 25
    for i, o_i in enumerate(hist):
        w = scipy.special.softmax(x[: i + 1])
        np.testing.assert_allclose(o_i, w @ v[: i + 1], rtol=1e-12, atol=1e-13)


def test_normalised_state_is_max_and_denominator():
    """The final (m, d') are max_j x_j and sum_j e^{x_j - m}: m + log d' is the row's log-sum-exp."""
    q = RNG.standard_normal((6, 3))
    k = RNG.standard_normal((30, 3))
    v = RNG.standard_normal((30, 3))
    for causal in (False, True):
        kk = k[:6] if causal else k
        vv = v[:6] if causal else v
        _, m, d = recurrence.attention_normalised(q, kk, vv, causal=causal)
        s = (q @ kk.T) / math.sqrt(3)
        if causal:
            s = np.where(np.tril(np.ones((6, 6), dtype=bool)), s, -np.inf)
        np.testing.assert_allclose(m, s.max(axis=1), rtol=1e-15)
        np.testing.assert_allclose(d, np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1), rtol=1e-13)
        lse = oracle.attention_lse(q[None, None], kk[None, None], causal=causal)[0, 0]
        np.testing.assert_allclose(m + np.log(d), lse, rtol=1e-13, atol=1e-13)


def test_normalised_two_keys_closed_form():
    """Two keys, d = 1: O = v1 sigma(x1 - x2) + v2 sigma(x2 - x1), also when the second key jumps the max by 50."""
    for x1, x2 in ((0.3, -1.2), (0.0, 50.0), (-7.0, -7.0)):
        q = np.array([[1.0]])
        k = np.array([[x1], [x2]])
        v = np.array([[2.0], [-3.0]])
        o, m, d = recurrence.attention_normalised(q, k, v, scale=1.0)
        s1 = scipy.special.expit(x1 - x2)
        assert o[0, 0] == pytest.approx(2.0 * s1 - 3.0 * (1.0 - s1), rel=1e-14, abs=1e-15)
        assert m[0] == max(x1, x2)
        assert d[0] == pytest.approx(1.0 + math.exp(min(x1, x2) - max(x1, x2)), rel=1e-15)
    # causal first row sees key 0 only: its output is V[0] exactly
    q = RNG.standard_normal((4, 3))
    k = RNG.standard_normal((4, 3))
    v = RNG.standard_normal((4, 3))
    o, _, _ = recurrence.attention_normalised(q, k, v, causal=True)
    assert np.array_equal(o[0], v[0])


def test_attention_heads_pool_matches_brute_force():
    """The pooled per-slice driver against pure-Python brute force (GQA groups of 1-3, causal on and off), O and
    LSE, with several threads: a wrong KV head or a mixed-up slice would miss by O(1)."""
    for B, Hkv, G, S, D, causal, scale in [(2, 2, 3, 5, 3, True, None), (1, 3, 2, 4, 2, False, 0.7),
                                           (2, 1, 1, 1, 4, True, 1.3)]:
        q = RNG.normal(size=(B, Hkv * G, S, D))
        k = RNG.normal(size=(B, Hkv, S, D))
        v = RNG.normal(size=(B, Hkv, S, D))
        o, lse = oracle.attention_heads(q, k, v, causal=causal, scale=scale, with_lse=True, workers=3)
        ref = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), causal=causal, scale=scale))
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
        ref_lse = np.array(brute.attention_lse(q.tolist(), k.tolist(), causal=causal, scale=scale))
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_attention_heads_pool_gqa_closed_form_and_subset():
    """V[b, kv] = 8b + kv gives O[b, h] = 8b + h // G for every head the pool computes; heads left out stay NaN."""
    B, Hq, Hkv, S, D = 2, 8, 2, 7, 4
    q, k = RNG.normal(size=(B, Hq, S, D)), RNG.normal(size=(B, Hkv, S, D))
    v = np.empty((B, Hkv, S, D))
    for b in range(B):
        for kv in range(Hkv):
            v[b, kv] = 8 * b + kv
    heads = [(0, 0), (0, 3), (0, 4), (1, 7)]
    o = oracle.attention_heads(q, k, v, causal=True, heads=heads, workers=2)
    for b in range(B):
        for h in range(Hq):
            if (b, h) in heads:
                np.testing.assert_allclose(o[b, h], 8 * b + h // (Hq // Hkv), rtol=1e-14)
            else:
                assert np.isnan(o[b, h]).all()

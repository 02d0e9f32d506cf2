"""The seeded input generators: determinism, shapes and planted structure."""
import numpy as np

import synth


def test_bf16_rounding_is_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7  # bf16 spacing at 1.0
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, -2.5, 1e-3], dtype=np.float32)
    bits = synth.round_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    # a tie rounds to the even neighbour: 1+ulp/2 -> 1.0, 1+3ulp/2 -> 1+2ulp
    np.testing.assert_array_equal(back[:5], np.array([1.0, 1.0, 1.0 + 2 * ulp, 1.0, -2.5], dtype=np.float32))
    assert abs(back[5] - 1e-3) <= 1e-3 * 2.0 ** -8


def test_attn_slices_are_deterministic_and_independent():
    w = synth.WORKLOADS["gqa_prefill_bf16"]
    a = synth.attn_slice(w, "k", 1, 3)
    b = synth.attn_slice(w, "k", 1, 3)
    c = synth.attn_slice(w, "k", 1, 4)
    assert a.dtype == np.uint16 and a.shape == (w.seq_k, w.head_dim)
    np.testing.assert_array_equal(a, b)
    assert (a != c).mean() > 0.9


def test_small_workloads_shapes():
    w = synth.WORKLOADS["attn_f32_m64_n100_d48"]
    t = synth.attn_inputs(w)
    assert t["q"].shape == (1, 1, 64, 48) and t["k"].shape == (1, 1, 100, 48) and t["v"].shape == (1, 1, 100, 48)
    assert t["q"].dtype == np.float32
    assert abs(t["k"].std() - 1.0) < 0.05
    x = synth.softmax_inputs(synth.WORKLOADS["softmax_4x200"])
    assert x.shape == (4, 200) and x.min() >= -10 and x.max() <= 10


def test_planted_key_row():
    w = synth.WORKLOADS["attn_f32_4k_d128"]
    k = synth.attn_slice(w, "k", 0, 0)
    raw = np.random.default_rng([w.seed, synth.TENSOR_ID["k"], 0, 0]).standard_normal(
        (w.seq_k, w.head_dim), dtype=np.float32)
    np.testing.assert_array_equal(k[3900], raw[3900] * np.float32(8.0))
    np.testing.assert_array_equal(k[3899], raw[3899])


def test_spike_in_final_percent():
    w = synth.WORKLOADS["softmax_1x16m"]
    x = synth.softmax_inputs(w)
    idx = int(np.argmax(x[0]))
    assert x[0, idx] == 50.0
    assert idx >= w.cols - w.cols // 100
    assert abs(np.delete(x[0], idx).std() - 2.0) < 0.01
    assert (x[0] == 50.0).sum() == 1


def test_flop_and_byte_counts():
    w = synth.WORKLOADS["gqa_prefill_bf16"]
    assert w.flops() == 0.5 * 4 * 2 * 32 * 4096 * 4096 * 128
    d = synth.WORKLOADS["gqa_decode_bf16"]
    assert d.bytes() == 2 * (2 * 64 * 32 * 128 + 2 * 64 * 8 * 8192 * 128)
    s = synth.WORKLOADS["softmax_1x16m"]
    assert s.bytes() == 3 * 4 * (1 << 24)


def test_causal_softmax_visible_count():
    """visible() against a direct count of the mask c <= r mod P, and the byte model on top of it."""
    for rows, cols, period in [(10, 7, 4), (6, 3, 6), (9, 20, 0), (5, 5, 1)]:
        w = synth.SoftmaxWorkload("t", rows, cols, seed=0, dist="normal", causal_period=period, dtype="bf16")
        count = sum(1 for r in range(rows) for c in range(cols) if period == 0 or c <= r % period)
        assert w.visible() == count
        assert w.bytes() == 2 * (2 * count + rows * cols) and w.bytes(1) == 2 * (count + rows * cols)
    w = synth.WORKLOADS["softmax_causal_bf16"]
    assert w.visible() == 16 * 2048 * 2049 // 2


def test_causal_softmax_inputs_are_bf16_patterns():
    w = synth.SoftmaxWorkload("t", 64, 48, seed=7, dist="normal", sigma=2.0, dtype="bf16", causal_period=64)
    x = synth.softmax_inputs(w)
    assert x.dtype == np.uint16 and x.shape == (64, 48)
    f = synth.bf16_bits_to_f32(x)
    assert np.isfinite(f).all() and 1.5 < f.std() < 2.5

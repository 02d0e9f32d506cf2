"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and mid sizes are compared element by element; the full-size workloads
either in full (when the oracle takes seconds) or on sampled rows that the
oracle computes one by one.  Bars: fp32 max abs 1e-5; bf16 2e-2 + 1e-2|ref|.
"""
import zlib

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import LSE_BF16_ATOL, LSE_F32_ATOL, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def _run_attn(osx, t, dtype, causal, poison=True):
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.empty_like(q)
    if poison:
        out.fill_(float("nan"))
    osx.attn_fwd(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    return to_f64(out)


# ------------------------------------------------------------------ workloads in full
def test_attn_f32_m64_n100_d48(osx):
    w = synth.WORKLOADS["attn_f32_m64_n100_d48"]
    t = synth.attn_inputs(w)
    print(f"case {w.name}", flush=True)
    got = _run_attn(osx, t, "f32", False)
    check(got, oracle.attention(t["q"], t["k"], t["v"]), "f32", w.name)


def test_attn_f32_4k_d128_planted_key(osx):
    w = synth.WORKLOADS["attn_f32_4k_d128"]
    t = synth.attn_inputs(w)
    print(f"case {w.name}", flush=True)
    got = _run_attn(osx, t, "f32", False)
    ref = oracle.attention(t["q"], t["k"], t["v"])
    err = check(got, ref, "f32", w.name)
    print(f"{w.name}: max abs err {err:.3e}")
    # rows where the planted key carries > 0.99 of the weight return ~V[3900]
    q, k = t["q"][0, 0].astype(np.float64), t["k"][0, 0].astype(np.float64)
    s = q @ k.T / np.sqrt(w.head_dim)
    wts = np.exp(s - s.max(axis=1, keepdims=True))
    wts /= wts.sum(axis=1, keepdims=True)
    rows = np.nonzero(wts[:, 3900] > 0.99)[0]
    assert rows.size > 10
    vmax = np.abs(t["v"][0, 0]).max()
    dev = np.abs(got[0, 0, rows] - t["v"][0, 0, 3900][None, :]).max(axis=1)
    assert (dev <= (1 - wts[rows, 3900]) * 2 * vmax + 1e-5).all()


def test_softmax_4x200(osx):
    w = synth.WORKLOADS["softmax_4x200"]
    x = synth.softmax_inputs(w)
    print(f"case {w.name}", flush=True)
    y = osx.softmax_rows(to_dev(x))
    torch.cuda.synchronize()
    check(to_f64(y), oracle.softmax_rows(x), "f32", w.name)


def test_softmax_1x16m_late_spike(osx):
    w = synth.WORKLOADS["softmax_1x16m"]
    x = synth.softmax_inputs(w)
    print(f"case {w.name}", flush=True)
    xd = to_dev(x)
    y = torch.full_like(xd, float("nan"))
    osx.softmax_rows(xd, out=y)
    torch.cuda.synchronize()
    got = to_f64(y)
    ref = oracle.softmax_rows(x)
    check(got, ref, "f32", w.name)
    idx = int(np.argmax(x[0]))
    assert got[0, idx] == pytest.approx(ref[0, idx], abs=1e-6)
    # diagnostic: relative error over all (normal, tiny) outputs
    rel = np.abs(got - ref) / ref
    print(f"{w.name}: max rel err {rel.max():.3e}")
    assert rel.max() < 1e-4


def test_gqa_prefill_bf16_full_size(osx):
    """The causal GQA prefill workload at full size: all 2 x 32 x 4096 output rows and their log-sum-exp against
    the oracle (computed over the host's cores); the call that writes the log-sum-exp must give the same O."""
    w = synth.WORKLOADS["gqa_prefill_bf16"]
    t = synth.attn_inputs(w)
    print(f"case {w.name}", flush=True)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    osx.attn_fwd(q, k, v, causal=True, out=out)
    out2 = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    osx.attn_fwd(q, k, v, causal=True, out=out2, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    got = to_f64(out)
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], causal=True, with_lse=True)
    err = check(got, ref, "bf16", w.name)
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(got_lse).all()
    lerr = float(np.abs(got_lse - ref_lse).max())
    print(f"{w.name}: {got.size} output elements, max abs err {err:.3e}; {got_lse.size} lse values, "
          f"max abs err {lerr:.3e}")
    assert lerr <= LSE_BF16_ATOL


def test_prefill_bf16_long_sequence_sampled_rows(osx):
    """A 2^20-token causal GQA prefill (bf16, d = 128, two query heads on one KV head): 8192 query tiles per head,
    byte offsets 256x those of the benchmark workload; sampled rows (the first, tile and block edges, the middle,
    the last) against the definition."""
    S, D = 1 << 20, 128
    print(f"case long prefill S={S}", flush=True)
    t = synth.random_attn(21, "bf16", 1, 2, 1, S, S, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    osx.attn_fwd(q, k, v, causal=True, out=out)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 63, 64, 127, 128, 4095, S // 2, S - 129, S - 128, S - 65, S - 64, S - 1]
                      + np.random.default_rng(21).integers(0, S, 6).tolist()))
    got = to_f64(out[:, :, rows])
    for h in (0, 1):
        ref = oracle.attention_rows(t["q"][0, h, rows], t["k"][0, 0], t["v"][0, 0], rows, causal=True, seq_q=S)
        check(got[0, h], ref, "bf16", f"long prefill h={h}")


def test_f32_long_sequence_sampled_rows(osx):
    """fp32, one head of 2^17 queries and keys, d = 128, non-causal (1024 row tiles, no key split): sampled rows of
    the plain and the normalised-output recurrence against the definition over all 131072 keys."""
    S, D = 1 << 17, 128
    print(f"case long fp32 S={S}", flush=True)
    t = synth.random_attn(22, "f32", 1, 1, 1, S, S, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    rows = sorted(set([0, 1, 31, 32, 127, 128, S // 2, S - 33, S - 32, S - 1]
                      + np.random.default_rng(22).integers(0, S, 6).tolist()))
    ref = oracle.attention_rows(t["q"][0, 0, rows], t["k"][0, 0], t["v"][0, 0], rows)
    for fn in (osx.attn_fwd, osx.attn_fwd_normalised):
        out = torch.full_like(q, float("nan"))
        fn(q, k, v, out=out)
        torch.cuda.synchronize()
        check(to_f64(out[0, 0, rows]), ref, "f32", f"long fp32 {fn.__name__}")


@pytest.mark.parametrize("Sq,Sk,D", [(63, 1000, 48), (1, 333, 128), (127, 1990, 100)])
def test_f32_split_with_an_odd_number_of_partial_states(osx, Sq, Sk, D):
    """fp32 key split where rows x slices is odd, so the (m, l) pairs end off a 16-byte boundary and the slice
    accumulators start at the next one: O and the log-sum-exp of the plain and the normalised-output forms
    against the oracle."""
    p = osx.attn_plan(osx.OSX_F32, 1, 1, 1, Sq, Sk, D)
    parts = Sq * p["splits"]
    assert p["splits"] > 1 and parts % 2 == 1, p
    assert p["workspace_bytes"] == ((2 * parts + 3) // 4 * 4 + parts * D) * 4
    print(f"case f32 odd partials Sq={Sq} Sk={Sk} d={D}", flush=True)
    t = synth.random_attn(41, "f32", 1, 1, 1, Sq, Sk, D)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    ref_o = oracle.attention(t["q"], t["k"], t["v"])
    ref_lse = oracle.attention_lse(t["q"], t["k"])
    for fn in (osx.attn_fwd, osx.attn_fwd_normalised):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        fn(q, k, v, out=out, lse=lse)
        torch.cuda.synchronize()
        check(to_f64(out), ref_o, "f32", f"{fn.__name__} Sq={Sq} Sk={Sk}")
        np.testing.assert_allclose(to_f64(lse), ref_lse, rtol=0, atol=LSE_F32_ATOL)


def test_gqa_decode_bf16_full_size(osx):
    """The GQA decode workload at full size: all 64 x 32 query heads and their log-sum-exp against the oracle.
    Non-gating diagnostic from the bar's derivation: max |err| / rms(O*) per head stays below 2e-2."""
    w = synth.WORKLOADS["gqa_decode_bf16"]
    t = synth.attn_inputs(w)
    print(f"case {w.name}", flush=True)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    osx.attn_fwd(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    del q, k, v
    got = to_f64(out)
    ref, ref_lse = oracle.attention_heads(t["q"], t["k"], t["v"], with_lse=True)
    err = check(got, ref, "bf16", w.name)
    rel = (np.abs(got - ref).max(axis=-1) / np.sqrt(np.mean(ref ** 2, axis=-1))).max()
    got_lse = lse.cpu().numpy().astype(np.float64)
    lerr = float(np.abs(got_lse - ref_lse).max())
    print(f"{w.name}: {got.size} output elements, max abs err {err:.3e}, max err / rms {rel:.3e}; "
          f"lse max abs err {lerr:.3e}")
    assert rel < 2e-2
    assert lerr <= LSE_BF16_ATOL


# ------------------------------------------------------------------ mid sizes, element by element
PREFILL_CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, D, causal
    ("bf16", 1, 4, 1, 200, 200, 128, True),     # G=4: 4 heads per workgroup, ragged tiles
    ("bf16", 1, 4, 2, 150, 333, 128, False),    # G=2, Sq != Sk, ragged key tail
    ("bf16", 2, 3, 3, 130, 130, 64, True),      # MHA, D=64, 128-row tiles
    ("bf16", 1, 8, 1, 97, 97, 128, True),       # G=8: two head groups
    ("bf16", 1, 2, 1, 1, 77, 128, False),       # Sq=1 through the decode path
    ("bf16", 1, 40, 2, 1, 300, 128, True),      # G=20 > 16: Sq=1 falls back to the prefill kernel
    # more row tiles than CUs: persistent workgroups walk several tiles, the
    # load stream and the scores run across tile boundaries
    ("bf16", 8, 32, 8, 257, 257, 128, True),    # 320 tiles of 64 rows (G=4)
    ("bf16", 16, 16, 8, 300, 300, 128, False),  # 384 tiles of 128 rows (G=2)
    ("bf16", 20, 32, 8, 100, 100, 64, True),    # 320 tiles of 1 and 2 key blocks, D=64
    ("bf16", 3, 96, 96, 130, 130, 64, True),    # 288 MHA tiles of 256 rows, one key block each
    ("f32", 1, 1, 1, 65, 257, 48, False),
    ("f32", 1, 2, 1, 100, 100, 128, True),
    ("f32", 2, 4, 2, 33, 90, 4, False),
    ("f32", 1, 3, 3, 64, 64, 96, True),
    ("f32", 1, 1, 1, 1, 5, 32, True),
    ("f32", 1, 2, 2, 40, 1, 64, False),         # a single key
    ("f32", 1, 1, 1, 600, 600, 64, True),       # key slices merged afterwards, some slices fully masked
    ("f32", 1, 1, 1, 130, 1000, 128, False),    # key slices, ragged last slice
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_attention_mid_sizes(osx, case):
    dtype, B, Hq, Hkv, Sq, Sk, D, causal = case
    print(f"case {case}", flush=True)
    t = synth.random_attn(zlib.crc32(str(case).encode()) % 1000, dtype, B, Hq, Hkv, Sq, Sk, D)
    got = _run_attn(osx, t, dtype, causal)
    check(got, oracle.attention(t["q"], t["k"], t["v"], causal=causal), dtype, str(case))


DECODE_CASES = [
    # B, Hq, Hkv, Sk, D
    (2, 8, 2, 1, 128), (1, 4, 4, 31, 128), (3, 16, 1, 33, 128), (2, 10, 2, 1000, 64), (1, 8, 8, 5000, 128),
    (4, 32, 8, 2049, 128), (1, 2, 1, 129, 64),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_mid_sizes(osx, case):
    B, Hq, Hkv, Sk, D = case
    print(f"case decode {case}", flush=True)
    assert osx.attn_plan(osx.OSX_BF16, B, Hq, Hkv, 1, Sk, D)["kernel_name"] == "decode_bf16"
    t = synth.random_attn(sum(case), "bf16", B, Hq, Hkv, 1, Sk, D)
    got = _run_attn(osx, t, "bf16", False)
    check(got, oracle.attention(t["q"], t["k"], t["v"]), "bf16", f"decode {case}")


SOFTMAX_CASES = [(1, 1), (3, 7), (5, 4), (2, 255), (1, 8192), (2, 8193), (3, 16384 * 2 + 5), (2, 32768 * 2 + 5), (2, 100000),
                 (64, 1000), (1, 1 << 20)]


@pytest.mark.parametrize("shape", SOFTMAX_CASES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_softmax_shapes(osx, shape):
    print(f"case softmax {shape}", flush=True)
    x = np.random.default_rng(shape[1]).normal(0, 3, shape).astype(np.float32)
    y = osx.softmax_rows(to_dev(x))
    torch.cuda.synchronize()
    check(to_f64(y), oracle.softmax_rows(x), "f32", f"softmax {shape}")


def test_softmax_in_place_and_shift(osx):
    x = np.random.default_rng(3).normal(0, 2, (4, 40000)).astype(np.float32)
    xd = to_dev(x)
    osx.softmax_rows(xd, out=xd)
    x_shift = x + np.float32(500.0)
    ys = osx.softmax_rows(to_dev(x_shift))
    torch.cuda.synchronize()
    check(to_f64(xd), oracle.softmax_rows(x), "f32", "in place")
    check(to_f64(ys), oracle.softmax_rows(x_shift), "f32", "shifted by 500")


# ------------------------------------------------------------------ exact index maps
@pytest.mark.parametrize("dtype,S,D", [("bf16", 300, 128), ("f32", 300, 64), ("bf16", 129, 64)])
def test_causal_index_map_exact(osx, dtype, S, D):
    """K = 0: visible weights are uniform; V[j, c] = bit c of j gives O[i, c] = #{j <= i: bit c} / (i+1)."""
    j = np.arange(S)
    bits = ((j[:, None] >> (np.arange(D)[None, :] % 9)) & 1).astype(np.float32)
    q = np.random.default_rng(1).normal(size=(1, 2, S, D)).astype(np.float32)
    k = np.zeros((1, 1, S, D), np.float32)
    v = np.broadcast_to(bits, (1, 1, S, D)).copy()
    if dtype == "bf16":
        q, k, v = (synth.round_to_bf16_bits(a) for a in (q, k, v))
    got = _run_attn(osx, {"q": q, "k": k, "v": v}, dtype, True)
    expect = np.cumsum(bits.astype(np.float64), axis=0) / (j[:, None] + 1)
    tol = 2.0 ** -8 * np.abs(expect) + 1e-7 if dtype == "bf16" else 1e-6
    for h in range(2):
        assert (np.abs(got[0, h] - expect) <= tol).all(), f"causal map wrong for head {h}"


@pytest.mark.parametrize("dtype,Sq", [("bf16", 70), ("bf16", 1), ("f32", 40)])
def test_gqa_index_map_exact(osx, dtype, Sq):
    """V[b, kv] = 8b + kv gives O[b, h] = 8b + h // G: exactly in bf16 (the kernel's weights are the
    rounded P and its denominator sums those same values); within 1e-5 in fp32, whose numerator and
    denominator round differently.  A wrong head map is off by at least 1."""
    B, Hq, Hkv, Sk, D = 2, 16, 4, 90, 64
    rng = np.random.default_rng(2)
    q = rng.normal(size=(B, Hq, Sq, D)).astype(np.float32)
    k = rng.normal(size=(B, Hkv, Sk, D)).astype(np.float32)
    v = np.empty((B, Hkv, Sk, D), np.float32)
    for b in range(B):
        for kv in range(Hkv):
            v[b, kv] = 8 * b + kv
    if dtype == "bf16":
        q, k, v = (synth.round_to_bf16_bits(a) for a in (q, k, v))
    got = _run_attn(osx, {"q": q, "k": k, "v": v}, dtype, False)
    for b in range(B):
        for h in range(Hq):
            if dtype == "bf16":
                np.testing.assert_array_equal(got[b, h], 8 * b + h // (Hq // Hkv))
            else:
                np.testing.assert_allclose(got[b, h], 8 * b + h // (Hq // Hkv), rtol=0, atol=1e-5)


# ------------------------------------------------------------------ properties
def test_deterministic_and_stream(osx):
    t = synth.random_attn(5, "bf16", 1, 8, 2, 256, 256, 128)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    a = osx.attn_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = osx.attn_fwd(q, k, v, causal=True)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_problems_launch_nothing(osx):
    q = torch.empty((0, 4, 16, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    assert osx.attn_fwd(q, k, k).shape == q.shape
    x = torch.empty((0, 5), dtype=torch.float32, device="cuda")
    assert osx.softmax_rows(x).shape == (0, 5)


def test_single_hip_runtime_in_process(osx):
    """The library must bind to the process's (torch's) HIP runtime, not load a second one."""
    with open("/proc/self/maps") as f:
        libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_decode_longest_supported_kv(osx):
    """Decode at the longest K/V the ABI accepts for d = 128 bf16: 2^23 - 1 keys, 2 GiB each for K and V.

    The oracle cannot hold 8M keys in fp64, so this checks a property that holds at any size: the last key
    is planted so that its scaled score is s* = 30 while every other score is ~0, so its weight is
    1 - O(Sk e^-30) ~ 1 - 1e-6 and O equals V[Sk - 1] within the bf16 bar, and the log-sum-exp is
    s* + O(1e-6).  The planted key sits at the very end of the 2 GiB ranges the kernel addresses.
    """
    Sk, D = (1 << 23) - 1, 128
    print(f"case decode longest kv Sk={Sk}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(23)
    q1 = torch.randn(D, device="cuda", generator=gen).to(torch.bfloat16)
    q = q1.expand(1, 4, 1, D).contiguous()
    k = (torch.randn(1, 1, Sk, D, device="cuda", generator=gen, dtype=torch.bfloat16) * 0.01).to(torch.bfloat16)
    v = torch.randn(1, 1, Sk, D, device="cuda", generator=gen, dtype=torch.bfloat16)
    qf = q1.double().cpu().numpy()
    k[0, 0, Sk - 1] = torch.from_numpy(30.0 * np.sqrt(D) * qf / (qf @ qf)).to("cuda").to(torch.bfloat16)
    o, lse = osx.attn_fwd(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    s_star = float(qf @ k[0, 0, Sk - 1].double().cpu().numpy()) / np.sqrt(D)
    assert abs(s_star - 30.0) < 0.5
    want = np.broadcast_to(to_f64(v[0, 0, Sk - 1]), (4, D))
    check(to_f64(o)[0, :, 0], want, "bf16", "planted last key")
    assert np.abs(lse.double().cpu().numpy()[0, :, 0] - s_star).max() < 1e-3
    del k, v


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Sk, d -> key splits of the plan
    (1, 16, 1, 131072, 64),   # 512 splits, the planner's largest: 8 batches of the combine
    (1, 4, 1, 40000, 128),    # 313 splits: a count that is not a multiple of the combine's batch
], ids=lambda c: "-".join(map(str, c)))
def test_decode_most_splits_against_the_oracle(osx, case):
    """Decode whose keys are split the most the planner does (one (batch, KV head) unit), compared in full with
    the oracle, output and log-sum-exp: every split's partial state enters the combine."""
    B, Hq, Hkv, Sk, d = case
    plan = osx.attn_plan(osx.OSX_BF16, B, Hq, Hkv, 1, Sk, d)
    print(f"case decode most splits {case}: {plan['splits']} splits", flush=True)
    assert plan["splits"] == min(512, -(-Sk // 128))
    t = synth.random_attn(zlib.crc32(str(case).encode()), "bf16", B, Hq, Hkv, 1, Sk, d)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    o, lse = osx.attn_fwd(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    check(to_f64(o), oracle.attention(t["q"], t["k"], t["v"]), "bf16", str(case))
    lerr = np.abs(lse.double().cpu().numpy() - oracle.attention_lse(t["q"], t["k"])).max()
    assert lerr <= LSE_BF16_ATOL, f"{case}: lse error {lerr:.3e}"


# ------------------------------------------------------------------ wide GQA groups
# Query heads per KV head beyond the common 1/2/4/8: G = 16 is the widest group
# the decode kernel packs into its MFMA columns; G = 32 decode therefore runs
# the prefill kernel with one query row; G = 6 and 5 give the prefill planner
# two and one heads per workgroup with several head groups per KV head.
@pytest.mark.parametrize("case", [
    # dtype, B, Hq, Hkv, Sq, Sk, d, causal
    ("bf16", 2, 16, 1, 1, 3000, 128, False),
    ("bf16", 1, 32, 1, 1, 700, 128, False),
    ("bf16", 1, 12, 2, 200, 200, 64, True),
    ("bf16", 2, 10, 2, 130, 130, 128, False),
    ("f32", 1, 12, 2, 200, 200, 48, True),
    ("f32", 1, 32, 1, 1, 500, 128, False),
], ids=lambda c: "-".join(map(str, c)))
def test_wide_gqa_groups(osx, case):
    dtype, B, Hq, Hkv, Sq, Sk, d, causal = case
    print(f"wide GQA {case}", flush=True)
    t = synth.random_attn(zlib.crc32(str(case).encode()), dtype, B, Hq, Hkv, Sq, Sk, d)
    plan = osx.attn_plan(osx.OSX_BF16 if dtype == "bf16" else osx.OSX_F32, B, Hq, Hkv, Sq, Sk, d, causal)
    print(f"  plan {plan['kernel_name']} grid {plan['grid']} heads_per_wg {plan['heads_per_wg']}", flush=True)
    got = _run_attn(osx, t, dtype, causal)
    check(got, oracle.attention(t["q"], t["k"], t["v"], causal=causal), dtype, str(case))

"""GPU parity of osx_softmax_rows_ex (scale, causal mask, bf16 in/out) against the fp64 oracle.

Covers the row-in-registers kernels (one wavefront or one workgroup per row)
and the split (chunked) kernels, at the boundaries between them,
16-byte and scalar paths (column counts that are and are not multiples of the
vector width), chunks that are wholly, partly or not masked, and in place.
Masked outputs must be exactly 0.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import F32_ATOL, SOFTMAX_BF16_ATOL, SOFTMAX_BF16_RTOL, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [  # dtype, rows, cols, causal_period, scale
    ("f32", 64, 100, 64, 0.125),       # one causal [64, 100] score matrix
    ("f32", 4096, 4096, 4096, 0.0883883),  # a full causal 4096 x 4096 head, row kernel
    ("bf16", 150, 77, 50, 1.0),        # three heads of [50, 77], scalar path (77 % 8 != 0)
    ("f32", 140, 101, 70, 0.3),        # two heads of [70, 101], scalar path (101 % 4 != 0)
    ("bf16", 96, 4096, 48, 0.5),       # vector path, period < cols
    ("bf16", 33, 2048, 0, 1.0),        # longest wavefront row; 33 rows = 8 full workgroups + 1 row
    ("f32", 5, 8192, 3, 1.0),          # longest workgroup row, 16-byte path
    ("f32", 10, 5001, 7, 0.5),         # workgroup row, scalar path
    ("bf16", 6, 2049, 4, 1.0),         # shortest workgroup row, scalar path
    ("bf16", 2, 65536, 0, 2.0),        # split, 16-byte path, full chunks
    ("bf16", 2, 100003, 0, 1.0),       # split, scalar path, ragged last chunk
    ("f32", 3, 40000, 3, 1.0),         # split: all but the first chunk wholly masked
    ("f32", 2, 20000, 0, 0.75),        # split, scale only
]


@pytest.fixture(scope="module")
def osx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import online_softmax_02_amd
    return online_softmax_02_amd


def _inputs(dtype, rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 3.0, (rows, cols)).astype(np.float32)
    return synth.round_to_bf16_bits(x) if dtype == "bf16" else x


def _check(got, ref, dtype, period, what):
    rows, cols = ref.shape
    assert np.isfinite(got).all(), what
    if period:
        lim = np.minimum(np.arange(rows) % period + 1, cols)
        masked = np.arange(cols)[None, :] >= lim[:, None]
        assert (got[masked] == 0).all(), f"{what}: masked outputs are not 0"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= F32_ATOL, f"{what}: max abs error {err.max():.3e}"
    else:
        bad = err > SOFTMAX_BF16_ATOL + SOFTMAX_BF16_RTOL * np.abs(ref)
        assert not bad.any(), f"{what}: {int(bad.sum())} outputs off, worst {err.max():.3e}"


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_softmax_options_match_oracle(osx, case):
    dtype, rows, cols, period, scale = case
    if rows * cols > (1 << 26):  # keep the fp64 oracle within a few seconds: check a band of rows
        pytest.skip("too large for the element-wise check")
    print(f"case softmax_ex {case}", flush=True)
    x = _inputs(dtype, rows, cols, rows + cols)
    y = osx.softmax_rows(to_dev(x), causal_period=period, scale=scale)
    torch.cuda.synchronize()
    _check(to_f64(y), oracle.softmax_rows(x, causal_period=period, scale=scale), dtype, period, str(case))


def test_softmax_options_large_masked_rows_sampled(osx):
    """One causal fp32 head of [chunk + 40, chunk + 136] rows (chunk = the split kernels' chunk length, from the
    plan): every row is split into 2 chunks, and the visible part of the sampled rows ends inside chunk 0,
    exactly at its last column, at the first column of chunk 1, or inside chunk 1.  The 4.3 GB input is drawn
    on the GPU (seeded torch generator); the sampled rows are copied back for the oracle."""
    chunk = osx.softmax_rows_plan(1, 1 << 24)["block_m"]
    rows, cols = chunk + 40, chunk + 136
    assert osx.softmax_rows_plan(rows, cols)["kernel_name"] == "softmax_split"
    gen = torch.Generator(device="cuda").manual_seed(11)
    xd = torch.randn(rows, cols, device="cuda", generator=gen).mul_(3.0)
    y = osx.softmax_rows(xd, causal_period=rows)
    torch.cuda.synchronize()
    pick = np.array([0, 1, 5000, chunk - 2, chunk - 1, chunk, chunk + 1, rows - 1])
    idx = torch.from_numpy(pick).cuda()
    x = xd[idx].cpu().numpy()
    got = y[idx].cpu().numpy().astype(np.float64)
    del xd, y
    ref = np.zeros((len(pick), cols))
    for i, r in enumerate(pick):  # row r keeps columns <= r: the oracle on that row's visible prefix
        ref[i, :r + 1] = oracle.softmax_rows(x[i:i + 1, :r + 1])[0]
    _check(got, ref, "f32", 0, "sampled rows")
    for i, r in enumerate(pick):
        assert (got[i, r + 1:] == 0).all()


def test_softmax_causal_bf16_workload_sampled(osx):
    """The timed causal score-row workload at full size (16 heads of [2048, 2048] bf16, scale 1/sqrt(128)),
    same call as the benchmark: rows sampled from every head, first/last rows of a head included."""
    w = synth.WORKLOADS["softmax_causal_bf16"]
    x = synth.softmax_inputs(w)
    y = osx.softmax_rows(to_dev(x), causal_period=w.causal_period, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    pick = np.unique(np.concatenate([[0, 1, 2047, 2048, w.rows - 1], rng.integers(0, w.rows, 59)]))
    got = to_f64(y[torch.from_numpy(pick).cuda()])
    # row r of a head keeps columns <= r mod 2048: the oracle on that visible prefix
    ref = np.stack([_masked_row(x[r], r % w.causal_period, w.scale) for r in pick])
    _check(got, ref, "bf16", 0, "causal bf16 workload rows")
    for i, r in enumerate(pick):
        assert (got[i, r % w.causal_period + 1:] == 0).all()


def _masked_row(xr, last, scale):
    """Oracle softmax of one row whose visible columns are [0, last]; zeros after."""
    out = np.zeros(xr.shape[0])
    out[:last + 1] = oracle.softmax_rows(xr[None, :last + 1], scale=scale)[0]
    return out


def test_softmax_options_in_place_bf16(osx):
    x = _inputs("bf16", 40, 4096, 5)
    xd = to_dev(x)
    y = osx.softmax_rows(xd, out=xd, causal_period=40, scale=0.25)
    torch.cuda.synchronize()
    assert y.data_ptr() == xd.data_ptr()
    _check(to_f64(y), oracle.softmax_rows(x, causal_period=40, scale=0.25), "bf16", 40, "in place")


def test_softmax_options_defaults_equal_plain_softmax(osx):
    """scale 1 and no mask through osx_softmax_rows_ex give the same bits as osx_softmax_rows."""
    x = to_dev(_inputs("f32", 3, 30000, 9))
    plain = osx.softmax_rows(x)
    ex = torch.empty_like(x)
    st = osx.lib.osx_softmax_rows_ex(x.data_ptr(), ex.data_ptr(), osx.OSX_F32, 3, 30000, 0, 1.0,
                                     torch.empty(osx.softmax_rows_workspace(3, 30000), dtype=torch.uint8,
                                                 device="cuda").data_ptr(), osx.softmax_rows_workspace(3, 30000),
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(plain, ex)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [2048, 8192, 40000])
def test_softmax_base_not_16_byte_aligned(osx, dtype, cols):
    """x and y one element past a 16-byte boundary (column counts that would take the vector path): the scalar path
    runs and matches the oracle, for each kernel (wavefront, workgroup, split)."""
    rows = 3
    print(f"case softmax offset base {dtype} {cols}", flush=True)
    x = np.random.default_rng(cols).normal(0.0, 3.0, (rows, cols)).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_to_bf16_bits(x)
    xd = to_dev(x)
    buf_x = torch.empty(rows * cols + 1, dtype=xd.dtype, device="cuda")
    buf_y = torch.full_like(buf_x, float("nan"))
    xs = buf_x[1:].view(rows, cols)
    ys = buf_y[1:].view(rows, cols)
    xs.copy_(xd)
    assert xs.data_ptr() % 16 != 0
    osx.softmax_rows(xs, out=ys, causal_period=rows, scale=0.5)
    torch.cuda.synchronize()
    got, ref = to_f64(ys), oracle.softmax_rows(x, causal_period=rows, scale=0.5)
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= F32_ATOL, err.max()
    else:
        assert (err <= SOFTMAX_BF16_ATOL + SOFTMAX_BF16_RTOL * np.abs(ref)).all(), err.max()

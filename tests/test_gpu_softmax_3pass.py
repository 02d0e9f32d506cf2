"""GPU parity of the three-pass softmax comparators (osx_softmax_rows_3pass) against the fp64 oracle.

Both designs compute the plain row softmax, so the oracle is the same
definition as for osx_softmax_rows.  Cases: short rows (one chunk), ragged
rows on the scalar path, rows split into several chunks with a ragged last
one, the full-size long-row workload (the one the benchmark times) with its
late spike, rows far below zero (the max must be the row's own, not 0), and
in place.
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


METHODS = {"atomic": 1, "stash": 2}
SHAPES = [(4, 200), (3, 1001), (5, 40000), (2, 16384), (2, 32768), (2, 32769), (2, 70001), (7, 3)]


@pytest.mark.parametrize("method", list(METHODS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_3pass_matches_oracle(osx, method, shape):
    rows, cols = shape
    print(f"case 3pass {method} {shape}", flush=True)
    x = np.random.default_rng(rows * 7 + cols).normal(0.0, 3.0, shape).astype(np.float32)
    y = osx.softmax_rows_3pass(to_dev(x), METHODS[method])
    torch.cuda.synchronize()
    check(to_f64(y), oracle.softmax_rows(x), "f32", f"{method} {shape}")


@pytest.mark.parametrize("method", list(METHODS))
def test_3pass_long_row_workload(osx, method):
    """x[1, 2^24] with a +50 spike in the last 1%: all the row's chunks merge one (max, sum)."""
    w = synth.WORKLOADS["softmax_1x16m"]
    x = synth.softmax_inputs(w)
    print(f"case 3pass {method} {w.name}", flush=True)
    xd = to_dev(x)
    y = torch.full_like(xd, float("nan"))
    osx.softmax_rows_3pass(xd, METHODS[method], out=y)
    torch.cuda.synchronize()
    got, ref = to_f64(y), oracle.softmax_rows(x)
    check(got, ref, "f32", f"{method} {w.name}")
    rel = np.abs(got - ref) / ref
    assert rel.max() < 1e-4, f"max rel err {rel.max():.3e}"


@pytest.mark.parametrize("method", list(METHODS))
def test_3pass_rows_far_below_zero(osx, method):
    """All values near -1000: e^{x - 0} would underflow to 0 everywhere; the row max must be used."""
    x = (np.random.default_rng(3).normal(0.0, 1.0, (3, 50000)) - 1000.0).astype(np.float32)
    print(f"case 3pass {method} negative rows", flush=True)
    y = osx.softmax_rows_3pass(to_dev(x), METHODS[method])
    torch.cuda.synchronize()
    check(to_f64(y), oracle.softmax_rows(x), "f32", f"{method} negative")


@pytest.mark.parametrize("method", list(METHODS))
def test_3pass_in_place(osx, method):
    x = np.random.default_rng(5).uniform(-10, 10, (6, 20000)).astype(np.float32)
    print(f"case 3pass {method} in place", flush=True)
    xd = to_dev(x)
    y = osx.softmax_rows_3pass(xd, METHODS[method], out=xd)
    torch.cuda.synchronize()
    assert y.data_ptr() == xd.data_ptr()
    check(to_f64(xd), oracle.softmax_rows(x), "f32", f"{method} in place")


def test_3pass_repeated_calls_reset_the_atomic_state(osx):
    """The atomic design resets its per-row (max, sum) each call: a second call on other data is not polluted."""
    a = np.random.default_rng(8).normal(0, 1, (4, 30000)).astype(np.float32) + 20.0
    b = np.random.default_rng(9).normal(0, 1, (4, 30000)).astype(np.float32)
    ws = torch.empty(osx.softmax_rows_3pass_workspace(4, 30000, 1), dtype=torch.uint8, device="cuda")
    osx.softmax_rows_3pass(to_dev(a), 1, workspace=ws)
    y = osx.softmax_rows_3pass(to_dev(b), 1, workspace=ws)
    torch.cuda.synchronize()
    check(to_f64(y), oracle.softmax_rows(b), "f32", "second call")

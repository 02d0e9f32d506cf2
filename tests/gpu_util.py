"""Helpers for the GPU tests: host<->device transfer and the parity bars."""
import numpy as np

import oracle

# Parity bars: fp32 max abs error 1e-5; bf16 |err| <= 2e-2 + 1e-2 |ref| per element.
F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
# Log-sum-exp of the scores.  fp32: the row max and the fp32 sum of up to a few
# thousand terms, each scaled score accurate to ~1e-6 -> 5e-5 absolute.  bf16:
# the sum is taken over P rounded to bf16 (relative error <= 2^-9 each, so the
# sum's relative error is below 2^-9 and ln of it below 2e-3) -> 4e-3 absolute.
LSE_F32_ATOL, LSE_BF16_ATOL = 5e-5, 4e-3
# Row softmax with bf16 output: y is rounded to bf16 (relative error <= 2^-9)
# after fp32 arithmetic (relative ~1e-6): |err| <= 2^-8 |y*| + 1e-6.
SOFTMAX_BF16_RTOL, SOFTMAX_BF16_ATOL = 2.0 ** -8, 1e-6


def to_dev(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """Assert the parity bar; returns the max abs error."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    if dtype == "f32":
        worst = float(err.max()) if err.size else 0.0
        assert worst <= F32_ATOL, f"{what}: max abs error {worst:.3e} > {F32_ATOL}"
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
        bad = err > bound
        assert not bad.any(), f"{what}: {int(bad.sum())} elements outside 2e-2 + 1e-2|ref|, worst {err.max():.3e}"
    return float(err.max()) if err.size else 0.0

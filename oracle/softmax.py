"""fp64 row softmax, the plain definition (test infrastructure only).

Page "Softmax 算子的实现与优化" defines y_i = e^{x_i} / sum_j e^{x_j} and uses
its invariance to a common shift to subtract the row maximum first; page
"Puzzle 8: Long Softmax" gives the same computation as its row-wise spec over
an [N0, T] batch.  The options follow page "从零开始写Qwen3（五-其一）使用Triton
实现自注意力", section softmax的triton实现: a scale on the logits and the causal
mask that loads columns beyond the row index as -inf.
"""
import numpy as np


def softmax_rows(x, *, causal_period: int = 0, scale: float = 1.0) -> np.ndarray:
    """y[r, :] = exp(t[r, :] - max t[r, :]) / sum exp(t[r, :] - max t[r, :]), fp64, t = scale * x.

    With ``causal_period`` P > 0, t[r, c] = -inf for c > r mod P (row r of a
    stack of [P, cols] matrices keeps the columns up to its own index), so
    those y are 0.  bf16 bit patterns (uint16) are decoded exactly.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    x = np.asarray(x, dtype=np.float64) * scale
    if causal_period:
        assert x.ndim == 2
        r = np.arange(x.shape[0])[:, None] % causal_period
        x = np.where(np.arange(x.shape[1])[None, :] <= r, x, -np.inf)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)

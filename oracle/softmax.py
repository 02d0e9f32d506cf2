"""fp64 row softmax, the plain definition (test infrastructure only).

Page "Softmax 算子的实现与优化" defines y_i = e^{x_i} / sum_j e^{x_j} and uses
its invariance to a common shift to subtract the row maximum first; page
"Puzzle 8: Long Softmax" gives the same computation as its row-wise spec over
an [N0, T] batch.
"""
import numpy as np


def softmax_rows(x) -> np.ndarray:
    """y[r, :] = exp(x[r, :] - max x[r, :]) / sum exp(x[r, :] - max x[r, :]), fp64."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)

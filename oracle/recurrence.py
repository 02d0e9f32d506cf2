"""Blockwise model of the online-softmax recurrence, in fp64 (test infrastructure).

Not the oracle: it exists to check page-fixed facts (the worked rescale
example, the block invariant, the ragged-tail rule) against the plain
definition in ``oracle.attention`` / ``oracle.softmax``.

Follows page "softmax_attention", section 实现思路 (one query at a time, keys in
blocks, state = running max m, denominator l, accumulator acc; each block
rescales the history by exp(m_old - m_new)) and page "Softmax 算子的实现与优化",
section Online Softmax (the boxed update m' = max(m, m_b),
l' = l e^{m - m'} + sum_{x in B} e^{x - m'}, started from m = -inf, l = 0).

``attention_normalised`` is the other recurrence of page "Puzzle 9: Simple
FlashAttention", which keeps the output normalised at every key; it is the
oracle for the library's normalised-output attention variant, pinned to the
plain definition and to prefix softmaxes.
"""
import math

import numpy as np


def _block_update(m, l, acc, scores, vals):
    """One block of the recurrence; returns new (m, l, acc, alpha)."""
    m_new = max(m, float(np.max(scores)))
    if m_new == -math.inf:  # nothing visible yet: keep the empty state
        return m, l, acc, 1.0
    alpha = math.exp(m - m_new) if m != -math.inf else 0.0
    p = np.exp(scores - m_new)
    l_new = l * alpha + float(np.sum(p))
    acc_new = None
    if acc is not None:
        acc_new = acc * alpha + p @ vals
    return m_new, l_new, acc_new, alpha


def softmax_online(x, block: int = 32, trace: bool = False):
    """Two-pass softmax of one row: online (m, l) over blocks, then normalise.

    Out-of-range positions of the last block are -inf (they add nothing to
    the max and e^{-inf} = 0 to the sum).  With ``trace`` also returns the
    list of (m, l, alpha) after every block.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    m, l = -math.inf, 0.0
    hist = []
    for start in range(0, n, block):
        blk = np.full(block, -np.inf)
        seg = x[start:start + block]
        blk[:seg.shape[0]] = seg
        m, l, _, alpha = _block_update(m, l, None, blk, None)
        hist.append((m, l, alpha))
    y = np.exp(x - m) / l
    return (y, hist) if trace else y


def attention_blockwise(q, k, v, *, scale=None, block: int = 32, tail: str = "neg_inf",
                        causal: bool = False, trace: bool = False):
    """Single-head attention via the online recurrence, one query row at a time.

    q: [M, D], k, v: [N, D].  K/V are visited in ``block``-row blocks; rows of
    the last block past N are zero-filled.  ``tail="neg_inf"`` sets their
    scores to -inf (the rule the page states); ``tail="zero_score"`` leaves
    the zero-filled scores in place, the mistake the page warns about.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, D = q.shape
    N = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((M, D))
    traces = []
    for i in range(M):
        m, l, acc = -math.inf, 0.0, np.zeros(D)
        hist = []
        for start in range(0, N, block):
            kb = np.zeros((block, D))
            vb = np.zeros((block, D))
            seg = slice(start, min(start + block, N))
            kb[: seg.stop - start] = k[seg]
            vb[: seg.stop - start] = v[seg]
            s = (kb @ q[i]) * scale
            idx = start + np.arange(block)
            if tail == "neg_inf":
                s = np.where(idx < N, s, -np.inf)
            if causal and M > 1:
                s = np.where(idx <= i, s, -np.inf)
            m, l, acc, alpha = _block_update(m, l, acc, s, vb)
            hist.append((m, l, alpha))
        out[i] = acc / l
        traces.append(hist)
    return (out, traces) if trace else out


def attention_normalised(q, k, v, *, scale=None, causal: bool = False, trace_row: int | None = None):
    """Single-head attention via the normalised-output recurrence, one key at a time.

    Page "Puzzle 9: Simple FlashAttention" (fadingcoder.top), the recurrence
    under its scalar FlashAttention spec: for each query row and each key i in
    order, with x_i the scaled score,
        m_i  = max(m_{i-1}, x_i)
        d'_i = d'_{i-1} e^{m_{i-1} - m_i} + e^{x_i - m_i}
        O'_i = O'_{i-1} (d'_{i-1} / d'_i) e^{m_{i-1} - m_i} + (e^{x_i - m_i} / d'_i) V_i
    started from m_0 = -inf, d'_0 = 0, O'_0 = 0.  O' stays normalised at every
    step, so the last O' is the output with no final division.  Keys a row
    may not see (causal, query index < key index, with more than one query
    row) are skipped: a score of -inf would leave m, d' and O' unchanged.

    q: [M, D], k, v: [N, D].  Returns (O [M, D], m [M], d' [M]) with m the
    natural-log-domain running max.  With ``trace_row`` also returns the list
    of O'_i of that row after every visible key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, D = q.shape
    N = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((M, D))
    m_out = np.full(M, -math.inf)
    d_out = np.zeros(M)
    hist = []
    for r in range(M):
        m, d, o = -math.inf, 0.0, np.zeros(D)
        last = r if (causal and M > 1) else N - 1
        for i in range(min(last, N - 1) + 1):
            x = float(q[r] @ k[i]) * scale
            m_new = max(m, x)
            shrink = math.exp(m - m_new)  # e^{m_{i-1} - m_i}; 0 on the first key
            e = math.exp(x - m_new)
            d_new = d * shrink + e
            o = o * (d / d_new) * shrink + (e / d_new) * v[i]
            m, d = m_new, d_new
            if r == trace_row:
                hist.append(o.copy())
        out[r], m_out[r], d_out[r] = o, m, d
    if trace_row is not None:
        return out, m_out, d_out, hist
    return out, m_out, d_out

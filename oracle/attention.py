"""fp64 attention, the plain definition (test infrastructure only).

Follows page "从零开始写Qwen3（五-其一）使用Triton实现自注意力", section 自注意力原理:
the eager reference groups the query heads by KV head (query head h reads KV
head h // G, with G = Hq / Hkv), scales Q K^T by head_dim^-1/2, applies a
lower-triangular causal mask only when there is more than one query row, takes
a softmax over the keys and multiplies by V.  Page "softmax_attention",
section 实现思路 gives the single-head form with the same scale.

The score matrix is materialised one (batch, query head) at a time; no
blocking, no online rescaling.
"""
import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


def _softmax_last(s: np.ndarray) -> np.ndarray:
    # max-shifted exponentials over the key axis, then divide by their sum
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, *, causal: bool = False, scale: float | None = None) -> np.ndarray:
    """O[b, h] = softmax(mask(Q[b,h] K[b,h//G]^T * scale)) V[b,h//G], in fp64.

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D]; fp32/fp64 arrays or bf16 bit
    patterns (uint16).  ``scale`` defaults to D**-0.5.  With ``causal`` and
    Sq > 1, key j is visible to query i only when j <= i (top-left aligned);
    with Sq == 1 no mask is applied.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    assert Bk == B and Dk == D and v.shape == k.shape
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, Sq, D), dtype=np.float64)
    keep = None
    if causal and Sq > 1:
        keep = np.tril(np.ones((Sq, Sk), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            s = (q[b, h] @ k[b, kv].T) * scale
            if keep is not None:
                s = np.where(keep, s, -np.inf)
            out[b, h] = _softmax_last(s) @ v[b, kv]
    return out


def attention_rows(q_rows, k, v, rows, *, causal: bool = False, seq_q: int | None = None,
                   scale: float | None = None) -> np.ndarray:
    """The definition for selected query rows of one (batch, query head).

    q_rows: [n, D] query vectors whose row indices are ``rows``; k, v: [Sk, D]
    of the KV head this query head reads.  ``seq_q`` is the query length of
    the full problem (the causal mask applies only when it exceeds 1).
    """
    q_rows, k, v = _as_f64(q_rows), _as_f64(k), _as_f64(v)
    D = q_rows.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s = (q_rows @ k.T) * scale
    if causal and (seq_q is None or seq_q > 1):
        j = np.arange(k.shape[0])[None, :]
        i = np.asarray(rows)[:, None]
        s = np.where(j <= i, s, -np.inf)
    return _softmax_last(s) @ v


def attention_lse(q, k, v=None, *, causal: bool = False, scale: float | None = None) -> np.ndarray:
    """Log-sum-exp of each query row's scaled, masked scores, in fp64: [B, Hq, Sq].

    LSE[b, h, i] = log sum_j exp(S[i, j]) over the visible keys j, with S the
    same scaled (and causally masked) score matrix as in ``attention``.  It is
    the final online state of page "Softmax 算子的实现与优化", section Online
    Softmax, folded into one number: m + log l with m the row max and
    l = sum_j e^{S[i, j] - m}.  (``v`` is accepted for symmetry and unused.)
    """
    q, k = _as_f64(q), _as_f64(k)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    assert Bk == B and Dk == D and Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    keep = np.tril(np.ones((Sq, Sk), dtype=bool)) if causal and Sq > 1 else None
    out = np.empty((B, Hq, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            s = (q[b, h] @ k[b, h // G].T) * scale
            if keep is not None:
                s = np.where(keep, s, -np.inf)
            m = np.max(s, axis=-1)
            out[b, h] = m + np.log(np.sum(np.exp(s - m[:, None]), axis=-1))
    return out

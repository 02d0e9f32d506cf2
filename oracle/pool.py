"""The fp64 attention definition over many heads at once (test infrastructure only).

Large problems (tens of 4096 x 4096 heads) would take minutes one head after
another.  This module maps ``oracle.attention`` / ``oracle.attention_lse`` --
the plain definition of page "从零开始写Qwen3（五-其一）使用Triton实现自注意力",
section 自注意力原理, with its GQA head map -- over independent
(batch, query head) slices on a pool of host threads.  Each slice is handed
to the unchanged single-head definition with the KV head that query head
reads (h // G, section GQA); no arithmetic of the method lives here.  numpy's
products and element-wise loops release the interpreter lock, so the threads
run in parallel; BLAS is held to one thread per call while the pool runs, so
the pool's threads do not oversubscribe the cores.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import attention, attention_lse


def default_workers() -> int:
    """Host threads to use: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def attention_heads(q, k, v, *, causal: bool = False, scale: float | None = None, with_lse: bool = False,
                    workers: int | None = None, heads=None):
    """``oracle.attention`` (and, with ``with_lse``, ``oracle.attention_lse``) slice by slice on a thread pool.

    q: [B, Hq, Sq, D], k, v: [B, Hkv, Sk, D] as for ``oracle.attention``.
    ``heads``: an iterable of (b, h) pairs to compute (default: all); other
    slices of the result are left NaN.  Returns O [B, Hq, Sq, D] in fp64, or
    (O, LSE [B, Hq, Sq]) with ``with_lse``.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    assert k.shape[0] == B and Hq % Hkv == 0
    G = Hq // Hkv
    out = np.full((B, Hq, Sq, D), np.nan)
    lse = np.full((B, Hq, Sq), np.nan) if with_lse else None
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)

    def one(bh):
        b, h = bh
        kv = h // G
        qs, ks, vs = q[b:b + 1, h:h + 1], k[b:b + 1, kv:kv + 1], v[b:b + 1, kv:kv + 1]
        out[b, h] = attention(qs, ks, vs, causal=causal, scale=scale)[0, 0]
        if with_lse:
            lse[b, h] = attention_lse(qs, ks, causal=causal, scale=scale)[0, 0]

    n = workers or default_workers()
    limiter = None
    if n > 1:
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(limits=1, user_api="blas")
        except ImportError:
            limiter = None
    try:
        if n == 1:
            for bh in todo:
                one(bh)
        else:
            with ThreadPoolExecutor(max_workers=n) as ex:
                list(ex.map(one, todo))
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    return (out, lse) if with_lse else out

"""Seeded synthetic inputs for the attention and row-softmax workloads.

This module only draws and rounds numbers.  It holds none of the method's
arithmetic (no scores, no exponentials, no reductions), so both the fp64
oracle and the GPU path can take their inputs from it without sharing any
computation.

Recipe (every draw is ``numpy.random.default_rng`` / PCG64):

* Large tensors are drawn slice by slice.  The slice ``[b, h, :, :]`` of
  tensor ``name`` comes from ``default_rng([seed, TENSOR_ID[name], b, h])``
  as fp32 ``standard_normal``.  A slice can therefore be regenerated alone,
  which lets a test compute sampled oracle rows at full size.
* bf16 tensors are the fp32 draws rounded to bfloat16 with
  round-to-nearest-even; they are returned as ``uint16`` bit patterns, and
  the rounded values are the inputs on both sides.
* The five workloads and their structure (ragged tails, planted key, late
  spike) are in :data:`WORKLOADS`.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TENSOR_ID = {"q": 1, "k": 2, "v": 3, "x": 4}


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    dtype: str  # "f32" or "bf16"
    batch: int
    heads_q: int
    heads_kv: int
    seq_q: int
    seq_k: int
    head_dim: int
    causal: bool
    seed: int
    planted_key: int | None = None  # key row scaled by planted_scale (all b, kv)
    planted_scale: float = 1.0
    kind: str = "attn"

    @property
    def groups(self) -> int:
        return self.heads_q // self.heads_kv

    def q_shape(self):
        return (self.batch, self.heads_q, self.seq_q, self.head_dim)

    def kv_shape(self):
        return (self.batch, self.heads_kv, self.seq_k, self.head_dim)

    def flops(self) -> float:
        """Algorithmic flop count, 4*B*Hq*Sq*Sk*d, halved when causal."""
        f = 4.0 * self.batch * self.heads_q * self.seq_q * self.seq_k * self.head_dim
        return f * 0.5 if self.causal else f

    def bytes(self) -> float:
        """Algorithmic bytes: Q, K, V read once, O written once."""
        es = 4 if self.dtype == "f32" else 2
        nq = self.batch * self.heads_q * self.seq_q * self.head_dim
        nkv = self.batch * self.heads_kv * self.seq_k * self.head_dim
        return float(es * (2 * nq + 2 * nkv))


@dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    rows: int
    cols: int
    seed: int
    dist: str  # "uniform" or "normal"
    low: float = 0.0
    high: float = 0.0
    sigma: float = 1.0
    spike: float | None = None  # value set at one index in the final 1% of each row
    kind: str = "softmax"
    dtype: str = "f32"      # "f32" or "bf16" (input and output)
    causal_period: int = 0  # > 0: row r keeps columns c <= r mod period
    scale: float = 1.0      # logits are scale * x

    def visible(self) -> int:
        """Number of unmasked elements over all rows."""
        if self.causal_period <= 0:
            return self.rows * self.cols
        r = np.arange(self.rows, dtype=np.int64) % self.causal_period
        return int(np.minimum(r + 1, self.cols).sum())

    def bytes(self, reads: int = 2) -> float:
        """Algorithmic bytes: the visible x read ``reads`` times (2 when the two passes each read it from memory,
        1 when the row stays on chip between them), all of y written once."""
        es = 2 if self.dtype == "bf16" else 4
        return float(es * (reads * self.visible() + self.rows * self.cols))


WORKLOADS = {
    # Single-head fp32, ragged last key block (100 = 3*32 + 4), d=48 not a power of two.
    "attn_f32_m64_n100_d48": AttnWorkload("attn_f32_m64_n100_d48", "f32", 1, 1, 1, 64, 100, 48, False, seed=1),
    # Row softmax, short rows: x[4,200] ~ U(-10,10).
    "softmax_4x200": SoftmaxWorkload("softmax_4x200", 4, 200, seed=2, dist="uniform", low=-10.0, high=10.0),
    # Row softmax, one row of 2^24 ~ N(0, variance 4) with a +50 spike in the last 1%.
    "softmax_1x16m": SoftmaxWorkload("softmax_1x16m", 1, 1 << 24, seed=3, dist="normal", sigma=2.0, spike=50.0),
    # Causal score rows in bf16: 16 heads of [2048, 2048] logits ~ N(0, 4), scale 1/sqrt(128).
    "softmax_causal_bf16": SoftmaxWorkload("softmax_causal_bf16", 16 * 2048, 2048, seed=7, dist="normal", sigma=2.0,
                                           dtype="bf16", causal_period=2048, scale=0.08838834764831845),
    # Single-head fp32 4096x4096, d=128; key row 3900 scaled by 8.
    "attn_f32_4k_d128": AttnWorkload("attn_f32_4k_d128", "f32", 1, 1, 1, 4096, 4096, 128, False, seed=4,
                                     planted_key=3900, planted_scale=8.0),
    # GQA causal prefill bf16: B2, Hq 32, Hkv 8, S 4096, d 128.
    "gqa_prefill_bf16": AttnWorkload("gqa_prefill_bf16", "bf16", 2, 32, 8, 4096, 4096, 128, True, seed=5),
    # GQA decode bf16: B64, Hq 32, Hkv 8, one query token, KV 8192, d 128.
    "gqa_decode_bf16": AttnWorkload("gqa_decode_bf16", "bf16", 64, 32, 8, 1, 8192, 128, False, seed=6),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = (u >> 16) & np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= 16
    return t.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _slice_f32(seed: int, name: str, b: int, h: int, rows: int, cols: int) -> np.ndarray:
    rng = np.random.default_rng([seed, TENSOR_ID[name], b, h])
    return rng.standard_normal((rows, cols), dtype=np.float32)


def attn_slice(w: AttnWorkload, name: str, b: int, h: int) -> np.ndarray:
    """One [S, D] slice of q, k or v, in the workload's dtype (bf16 as uint16 bits).

    ``h`` is a query head for ``q`` and a KV head for ``k``/``v``.
    """
    rows = w.seq_q if name == "q" else w.seq_k
    x = _slice_f32(w.seed, name, b, h, rows, w.head_dim)
    if name == "k" and w.planted_key is not None and w.planted_key < rows:
        x[w.planted_key, :] *= np.float32(w.planted_scale)
    if w.dtype == "bf16":
        return round_to_bf16_bits(x)
    return x


def _fill(args):
    w, name, b, h = args
    return attn_slice(w, name, b, h)


def attn_inputs(w: AttnWorkload, workers: int | None = None) -> dict:
    """Full q, k, v for a workload as numpy arrays ([B,H,S,D]; bf16 as uint16 bits)."""
    out = {}
    big = w.batch * (w.heads_q * w.seq_q + 2 * w.heads_kv * w.seq_k) * w.head_dim > (1 << 24)
    for name in ("q", "k", "v"):
        heads = w.heads_q if name == "q" else w.heads_kv
        shape = w.q_shape() if name == "q" else w.kv_shape()
        dt = np.uint16 if w.dtype == "bf16" else np.float32
        arr = np.empty(shape, dtype=dt)
        jobs = [(w, name, b, h) for b in range(w.batch) for h in range(heads)]
        if big:
            # Host threads, not processes: numpy's generators and element-wise
            # loops release the interpreter lock, and no process is forked
            # from one that may already hold a GPU context.
            n = workers or min(16, len(os.sched_getaffinity(0)))
            with ThreadPoolExecutor(max_workers=n) as ex:
                for (_, _, b, h), s in zip(jobs, ex.map(_fill, jobs)):
                    arr[b, h] = s
        else:
            for (_, _, b, h) in jobs:
                arr[b, h] = attn_slice(w, name, b, h)
        out[name] = arr
    return out


def softmax_inputs(w: SoftmaxWorkload) -> np.ndarray:
    """x[rows, cols] for a softmax workload: fp32, or bf16 bit patterns (uint16).

    ``normal``: N(0, sigma^2) rows; with ``spike``, element ``cols-1-r`` of each
    row is set to the spike value, ``r`` uniform in [0, cols/100) (a late max).
    """
    rng = np.random.default_rng([w.seed, TENSOR_ID["x"]])
    if w.dist == "uniform":
        x = rng.uniform(w.low, w.high, size=(w.rows, w.cols)).astype(np.float32)
    else:
        x = rng.standard_normal((w.rows, w.cols), dtype=np.float32)
        x *= np.float32(w.sigma)
    if w.spike is not None:
        tail = max(1, w.cols // 100)
        for r in range(w.rows):
            idx = w.cols - 1 - int(rng.integers(0, tail))
            x[r, idx] = np.float32(w.spike)
    if w.dtype == "bf16":
        return round_to_bf16_bits(x)
    return x


def spike_index(w: SoftmaxWorkload) -> list[int]:
    """Column of the planted spike in each row (recomputed from the seed)."""
    x = softmax_inputs(w)
    return [int(np.argmax(x[r])) for r in range(w.rows)]


def random_attn(seed: int, dtype: str, batch: int, heads_q: int, heads_kv: int, seq_q: int, seq_k: int,
                head_dim: int, causal: bool = False, scale_std: float = 1.0) -> dict:
    """Small ad-hoc attention inputs (tests): N(0, scale_std^2) in the given dtype."""
    rng = np.random.default_rng([seed, 99])
    out = {}
    for name, shape in (("q", (batch, heads_q, seq_q, head_dim)),
                        ("k", (batch, heads_kv, seq_k, head_dim)),
                        ("v", (batch, heads_kv, seq_k, head_dim))):
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale_std)
        out[name] = round_to_bf16_bits(x) if dtype == "bf16" else x
    return out

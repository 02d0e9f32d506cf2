"""fp64 CPU oracle for single-pass attention and the two-pass row softmax.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library.

Contents
--------
attention        the plain definition O = softmax(mask(Q K^T * scale)) V with
                 GQA and a top-left causal mask, materialising the score matrix
                 (page "从零开始写Qwen3（五-其一）使用Triton实现自注意力",
                 section 自注意力原理; page "softmax_attention", section 实现思路).
attention_rows   the same definition for a chosen set of query rows of one head.
attention_lse    log sum_j exp(score) per query row: the final (max, sum) state of
                 the online recurrence as one number (page "Softmax 算子的实现与优化",
                 section Online Softmax).
softmax_rows     the stable row softmax (page "Softmax 算子的实现与优化", the
                 max-shifted definition; page "Puzzle 8: Long Softmax", its spec).
recurrence       a blockwise model of the online recurrence (running max, running
                 denominator, unnormalised accumulator) used to check page-fixed
                 facts against the definition; and ``attention_normalised``, the
                 per-key normalised-output recurrence of page "Puzzle 9: Simple
                 FlashAttention" (oracle of the normalised-output variant).
brute            pure-Python loops over tiny inputs.
pool             ``attention`` / ``attention_lse`` mapped over (batch, query head)
                 slices on host threads, for full-size problems.

Every function is pinned by ``tests/test_oracle_pins.py`` to values, closed
forms and invariants the pages and the mathematics fix.  No function here is
"parity unpinned".
"""
from .attention import attention, attention_lse, attention_rows, bf16_bits_to_f64
from .softmax import softmax_rows
from . import recurrence, brute, pool
from .pool import attention_heads

__all__ = ["attention", "attention_lse", "attention_rows", "attention_heads", "softmax_rows", "bf16_bits_to_f64",
           "recurrence", "brute", "pool"]

"""fp64 causal attention of a chunk of new tokens over contiguous per-sequence K/V (oracle).

TEST INFRASTRUCTURE ONLY: imported by tests and the bench's CPU baseline; never by the
library.

What is computed.  In the prefill phase a sequence's tokens are written into its blocks
("Stop Wasting GPU Memory" page, Technical Details, "Single Sequence Generation"), and the
zhichai.net page ("PagedAttention: How Virtual Memory Paging Solved LLM KV Cache Waste",
Key points, "Engineering insight") says paging leaves the transformer's math unchanged.
The pages do not write the mask out; the plain reading of autoregressive generation is
that a token attends to itself and to the tokens before it.  For a sequence of n cached
tokens whose last c are the chunk being prefilled (their K/V already written), chunk row
i sits at position p = n - c + i and, per query head j with KV head h = j // (H_q / H_kv):

    x_t   = scale * sum_d q[i, j, d] * K[t, h, d]        t = 0 .. p
    out   = sum_t exp(x_t - max x) V[t, h, :] / sum_t exp(x_t - max x)

All arithmetic is float64; ``scale`` enters as float64(float32(scale)).
"""
from __future__ import annotations

import numpy as np

from .attention import attend_one_head


def prefill_attention_seq(q_chunk: np.ndarray, k_s: np.ndarray, v_s: np.ndarray, scale: float,
                          rows=None, heads=None) -> np.ndarray:
    """q_chunk [c, H_q, D] (the chunk's queries), k_s/v_s [n, H_kv, D] with n >= c (float64).

    Returns [len(rows), len(heads), D] for the requested chunk rows and query heads.
    """
    c, hq, d = q_chunk.shape
    n, hkv = k_s.shape[0], k_s.shape[1]
    if c > n:
        raise ValueError("the chunk is longer than the context")
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = hq // hkv
    rows = range(c) if rows is None else rows
    heads = range(hq) if heads is None else heads
    scale = float(np.float32(scale))
    out = np.empty((len(rows), len(heads), d), dtype=np.float64)
    for a, i in enumerate(rows):
        p = n - c + i
        for b, j in enumerate(heads):
            h = j // g
            out[a, b] = attend_one_head(q_chunk[i, j], k_s[:p + 1, h, :], v_s[:p + 1, h, :], scale)
    return out

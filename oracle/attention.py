"""fp64 single-query attention over contiguous per-sequence K/V (oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU baseline; never by the library.

What is computed.  The zhichai.net page ("PagedAttention: How Virtual Memory
Paging Solved LLM KV Cache Waste", Key points, "Engineering insight", and its
Summary) states that paging leaves the transformer's math unchanged, and its
"Why it matters" section says the attention kernel only gathers the scattered
blocks.  So the oracle is plain attention of one decode query per head over
the sequence's cached tokens held contiguously: no block table enters it.
For sequence s with n = context length, query head j and its KV head
h = j // (H_q / H_kv) (grouped query heads share one KV head, contiguous
grouping):

    x_t   = scale * sum_d q[s, j, d] * K_s[t, h, d]      t = 0 .. n-1
    m     = max_t x_t
    w_t   = exp(x_t - m)
    out   = sum_t w_t V_s[t, h, :] / sum_t w_t

All arithmetic is float64 on inputs decoded exactly from their stored type;
``scale`` enters as float64(float32(scale)), the value the library receives.
A sequence with n = 0 has out = 0 (a reading: the pages never attend over an
empty context).  Subtracting m changes nothing mathematically; it only keeps
exp() finite.
"""
from __future__ import annotations

import numpy as np


def attend_one_head(q_vec: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                    scale: float) -> np.ndarray:
    """Attention of one query vector [D] over n keys/values [n, D] (float64)."""
    n = k_rows.shape[0]
    if n == 0:
        return np.zeros(v_rows.shape[1], dtype=np.float64)
    x = scale * (k_rows @ q_vec)            # scores, step 1
    m = x.max()                             # step 2
    w = np.exp(x - m)                       # step 3
    return (w @ v_rows) / w.sum()           # step 4


def decode_attention_seq(q_s: np.ndarray, k_s: np.ndarray, v_s: np.ndarray, scale: float,
                         heads=None) -> np.ndarray:
    """One sequence: q_s [H_q, D], k_s/v_s [n, H_kv, D] (float64).

    Returns [len(heads), D] for the requested query heads (all by default).
    """
    hq = q_s.shape[0]
    hkv = k_s.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = hq // hkv
    heads = range(hq) if heads is None else heads
    scale = float(np.float32(scale))
    out = np.empty((len(heads), q_s.shape[1]), dtype=np.float64)
    for i, j in enumerate(heads):
        h = j // g
        out[i] = attend_one_head(q_s[j], k_s[:, h, :], v_s[:, h, :], scale)
    return out


def decode_attention(q: np.ndarray, keys, values, scale: float) -> np.ndarray:
    """All sequences: q [S, H_q, D]; keys[s], values[s] are [n_s, H_kv, D].

    Inputs are float64 arrays (use ``synth.decode_f64`` on stored values).
    Returns out [S, H_q, D] float64.
    """
    S, hq, d = q.shape
    out = np.empty((S, hq, d), dtype=np.float64)
    for s in range(S):
        out[s] = decode_attention_seq(q[s], keys[s], values[s], scale)
    return out

"""Where K/V elements live in the paged cache, element by element (oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU baseline; never by the library.

The pages fix the block structure — B tokens of keys and values per block,
blocks anywhere in GPU memory, a block table per sequence ("Stop Wasting GPU
Memory" page, Technical Details, "Core Architecture") — but no byte layout.
The library documents its layout in its public header; this module restates it
with plain scalar index formulas so a cache copied to the host can be checked
against the contiguous truth:

    K: element (block b, kv head h, token slot t, dim d) at
       (((b * H + h) * (D / X) + d / X) * B + t) * X + d % X,   X = 16 bytes / elem size
    V: element (b, h, t, d) at ((b * H + h) * D + d) * B + t

A token at logical position p of a sequence with table T sits in block
T[p // B], slot p % B (the ml-canon page's block-table sketch maps logical
positions onto physical blocks).  ``kv_append`` writes each new token to the
slot its slot mapping names (slot = block * B + offset; -1 = skip), and
``block_copy`` copies every element of a source block (all slots, all heads,
K and V) to a destination block, reading the pre-copy contents (copy-on-write
copies only the diverging block: same page, "Copy-on-Write for Parallel
Sampling").
"""
from __future__ import annotations

import numpy as np


def x_of(elem_bytes: int) -> int:
    return 16 // elem_bytes


def k_index(b, h, t, d, H, D, B, X):
    return (((b * H + h) * (D // X) + d // X) * B + t) * X + d % X


def v_index(b, h, t, d, H, D, B):
    return ((b * H + h) * D + d) * B + t


def _token_index_grids(H, D, B, X):
    """Flat offsets (within one block) of every (h, t, d) element, by the
    scalar formulas above, as [B, H, D] integer arrays."""
    h = np.arange(H).reshape(1, H, 1)
    t = np.arange(B).reshape(B, 1, 1)
    d = np.arange(D).reshape(1, 1, D)
    kidx = k_index(0, h, t, d, H, D, B, X)
    vidx = v_index(0, h, t, d, H, D, B)
    return np.broadcast_to(kidx, (B, H, D)), np.broadcast_to(vidx, (B, H, D))


def gather_sequence(k_flat, v_flat, table, ctx, H, D, B, elem_bytes):
    """Read tokens [0, ctx) of a sequence out of flat K/V caches.

    Returns (k, v) arrays [ctx, H, D] in the caches' storage dtype.
    """
    X = x_of(elem_bytes)
    kg, vg = _token_index_grids(H, D, B, X)
    per_block = H * D * B
    k = np.empty((ctx, H, D), dtype=k_flat.dtype)
    v = np.empty((ctx, H, D), dtype=v_flat.dtype)
    for p in range(ctx):
        b = int(table[p // B])
        t = p % B
        k[p] = k_flat[b * per_block + kg[t]]
        v[p] = v_flat[b * per_block + vg[t]]
    return k, v


def apply_kv_append(k_flat, v_flat, slots, k_new, v_new, H, D, B, elem_bytes):
    """Expected caches after ``kv_append``: token i goes to slots[i]
    (block slots[i] // B, offset slots[i] % B); slot -1 is skipped."""
    X = x_of(elem_bytes)
    kg, vg = _token_index_grids(H, D, B, X)
    per_block = H * D * B
    k_out = k_flat.copy()
    v_out = v_flat.copy()
    for i, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        b, t = divmod(int(s), B)
        k_out[b * per_block + kg[t]] = k_new[i]
        v_out[b * per_block + vg[t]] = v_new[i]
    return k_out, v_out


def apply_block_copy(k_flat, v_flat, pairs, H, D, B):
    """Expected caches after ``block_copy``: dst block := pre-copy src block,
    K and V, every element; nothing else changes."""
    per_block = H * D * B
    k_out = k_flat.copy()
    v_out = v_flat.copy()
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        k_out[dst * per_block:(dst + 1) * per_block] = k_flat[src * per_block:(src + 1) * per_block]
        v_out[dst * per_block:(dst + 1) * per_block] = v_flat[src * per_block:(src + 1) * per_block]
    return k_out, v_out

"""Pins for the oracle's paged-cache layout reader.

The scalar index formulas are checked against a second formulation (numpy
reshape/transpose of the whole cache), for being a bijection onto the pool,
and for append-then-gather round trips; block copies against the copy-on-write
rule that only the diverging block is duplicated.
"""
import numpy as np
import pytest

from oracle import paged_layout as pl
from oracle.allocator_model import BlockAllocatorModel


@pytest.mark.parametrize("elem_bytes,H,D", [(4, 4, 64), (2, 8, 128), (2, 3, 64)])
def test_offsets_are_a_bijection_per_block(elem_bytes, H, D):
    B = 16
    X = pl.x_of(elem_bytes)
    N = 3
    b, h, t, d = np.meshgrid(np.arange(N), np.arange(H), np.arange(B), np.arange(D), indexing="ij")
    for idx in (pl.k_index(b, h, t, d, H, D, B, X), pl.v_index(b, h, t, d, H, D, B)):
        flat = np.sort(idx.ravel())
        assert np.array_equal(flat, np.arange(N * H * B * D))
        # every element of block b lies inside block b's contiguous range
        per = H * B * D
        assert np.all(idx // per == b)


@pytest.mark.parametrize("elem_bytes,H,D", [(4, 4, 64), (2, 8, 128)])
def test_gather_matches_transpose_formulation(elem_bytes, H, D):
    B, N = 16, 6
    X = pl.x_of(elem_bytes)
    rng = np.random.default_rng(1)
    kc = rng.standard_normal(N * H * D * B)
    vc = rng.standard_normal(N * H * D * B)
    # K as [N, H, D/X, B, X] -> [N, B, H, D]; V as [N, H, D, B] -> [N, B, H, D]
    k_tok = kc.reshape(N, H, D // X, B, X).transpose(0, 3, 1, 2, 4).reshape(N, B, H, D)
    v_tok = vc.reshape(N, H, D, B).transpose(0, 3, 1, 2)
    table = [4, 0, 5]
    ctx = 37
    k, v = pl.gather_sequence(kc, vc, table, ctx, H, D, B, elem_bytes)
    for p in range(ctx):
        assert np.array_equal(k[p], k_tok[table[p // B], p % B])
        assert np.array_equal(v[p], v_tok[table[p // B], p % B])


def test_append_then_gather_round_trip():
    H, D, B, eb = 2, 64, 16, 2
    a = BlockAllocatorModel(10, B, [9, 3, 7, 1, 0, 2, 4, 5, 6, 8])
    a.add(0)
    a.add(1)
    rng = np.random.default_rng(2)
    kc = np.full(10 * H * D * B, np.nan)
    vc = np.full(10 * H * D * B, np.nan)
    truth = {0: ([], []), 1: ([], [])}
    for step in range(40):
        s = step % 2
        n = 1 + (step % 3)
        slots, pairs = a.append(s, n)
        assert pairs == []
        kn = rng.standard_normal((n, H, D))
        vn = rng.standard_normal((n, H, D))
        kc, vc = pl.apply_kv_append(kc, vc, slots, kn, vn, H, D, B, eb)
        truth[s][0].extend(kn)
        truth[s][1].extend(vn)
    for s in (0, 1):
        k, v = pl.gather_sequence(kc, vc, a.table(s), a.seq_len(s), H, D, B, eb)
        assert np.array_equal(k, np.array(truth[s][0]))
        assert np.array_equal(v, np.array(truth[s][1]))


def test_append_skips_minus_one_slots():
    H, D, B = 1, 8, 16
    kc = np.zeros(2 * H * D * B)
    vc = np.zeros(2 * H * D * B)
    k2, v2 = pl.apply_kv_append(kc, vc, [-1, 17], np.ones((2, H, D)), np.ones((2, H, D)), H, D, B, 4)
    assert k2.sum() == D and v2.sum() == D
    k, _ = pl.gather_sequence(k2, v2, [1], 2, H, D, B, 4)
    assert np.all(k[1] == 1) and np.all(k[0] == 0)


def test_block_copy_copies_whole_block_from_pre_copy_state():
    H, D, B = 2, 8, 16
    per = H * D * B
    rng = np.random.default_rng(3)
    kc = rng.standard_normal(5 * per)
    vc = rng.standard_normal(5 * per)
    k2, v2 = pl.apply_block_copy(kc, vc, [(1, 3), (3, 4)], H, D, B)
    assert np.array_equal(k2[3 * per:4 * per], kc[1 * per:2 * per])
    assert np.array_equal(k2[4 * per:5 * per], kc[3 * per:4 * per])     # pre-copy src
    assert np.array_equal(v2[3 * per:4 * per], vc[1 * per:2 * per])
    untouched = np.r_[0:3 * per]
    assert np.array_equal(k2[untouched], kc[untouched])
    assert np.array_equal(v2[untouched], vc[untouched])

"""Pins for the shared-prefix grouping (oracle/shared_prefix.py).

What fixes it, beyond restating the rule:
* a hand-worked batch whose groups are written out below;
* the facts the pages give about forking: branches of one prompt keep the
  prompt's blocks ("Stop Wasting GPU Memory" page, Technical Details,
  "Copy-on-Write for Parallel Sampling"), so on real allocator traces every
  group's members hold the same physical ids in their prefix, hence the same
  K/V;
* the parallel-sampling workload's closed form: P prompts of L tokens, each
  forked into M samples, group into P * ceil(M / max_members) groups covering
  floor(L / B) blocks;
* the invariants every grouping must satisfy, on random fork trees;
* the attention identity that reading shared blocks once relies on: attention over a prefix and
  over the rest, merged by the log-sum-exp rule, equals attention over the
  whole context (fp64, against the oracle's plain attention).
"""
import math

import numpy as np
import pytest

from oracle.allocator_model import BlockAllocatorModel
from oracle.attention import decode_attention_seq
from oracle.shared_prefix import shared_prefix_groups

B = 16


def test_hand_worked_batch():
    # rows 0-2 share 3 leading blocks (row 2 fills only 2 of them), row 3 shares 1 block with row 2,
    # rows 4-5 are identical but short, row 6 is alone.
    tables = [
        [7, 8, 9, 10, -1],
        [7, 8, 9, 11, -1],
        [7, 8, 9, 12, -1],
        [7, 20, 21, -1, -1],
        [30, 31, -1, -1, -1],
        [30, 31, -1, -1, -1],
        [40, -1, -1, -1, -1],
    ]
    lens = [64, 60, 40, 40, 31, 32, 16]
    # full blocks: 4, 3, 2, 2, 1, 2, 1
    prefix, groups = shared_prefix_groups(tables, lens, B, max_members=8, min_blocks=1)
    # run 0: k = 4 -> row 1: min(4, 3, common 3) = 3 -> row 2: min(3, 2, 3) = 2 -> row 3: min(2, 2, common 1) = 1
    #        -> row 4: common 0 < 1, stop.  group (0, 4, 1)
    # run 4: k = 1 -> row 5: min(1, 2, common 2) = 1 -> row 6: common 0, stop.  group (4, 2, 1)
    # run 6: alone.
    assert groups == [(0, 4, 1), (4, 2, 1)]
    assert prefix == [1, 1, 1, 1, 1, 1, 0]
    # min_blocks = 2 stops run 0 before row 3 (common 1): group (0, 3, 2); rows 3.. share fewer than 2 blocks
    prefix, groups = shared_prefix_groups(tables, lens, B, max_members=8, min_blocks=2)
    assert groups == [(0, 3, 2)]
    assert prefix == [2, 2, 2, 0, 0, 0, 0]
    # max_members = 2: (0, 1) share 3, then (2, 3) share 1, then (4, 5) share 1
    prefix, groups = shared_prefix_groups(tables, lens, B, max_members=2, min_blocks=1)
    assert groups == [(0, 2, 3), (2, 2, 1), (4, 2, 1)]
    assert shared_prefix_groups(tables, lens, B, max_members=1, min_blocks=1) == ([0] * 7, [])


def test_empty_and_degenerate_batches():
    assert shared_prefix_groups([], [], B, 4, 1) == ([], [])
    # zero-length and sub-block sequences fill no block: nothing to share
    tables = [[3, -1], [3, -1], [3, -1]]
    assert shared_prefix_groups(tables, [0, 15, 15], B, 4, 1) == ([0, 0, 0], [])
    # identical full rows share everything they fill, capped by the row width
    tables = [[1, 2], [1, 2]]
    assert shared_prefix_groups(tables, [100, 40], B, 4, 1) == ([2, 2], [(0, 2, 2)])
    with pytest.raises(ValueError):
        shared_prefix_groups(tables, [1, 1], B, 0, 1)
    with pytest.raises(ValueError):
        shared_prefix_groups(tables, [1, 1], B, 4, 0)


def check_grouping(tables, lens, prefix, groups, max_members, min_blocks):
    S = len(lens)
    seen = set()
    for first, members, k in groups:
        assert 2 <= members <= max_members
        assert k >= min_blocks
        rng_ = range(first, first + members)
        assert not seen.intersection(rng_)
        seen.update(rng_)
        for s in rng_:
            assert prefix[s] == k
            assert k <= lens[s] // B  # full blocks of every member
            assert list(tables[s][:k]) == list(tables[first][:k])
    for s in range(S):
        if s not in seen:
            assert prefix[s] == 0
    # groups are in batch order
    assert [g[0] for g in groups] == sorted(g[0] for g in groups)


def sampling_tables(prompts, samples, prefix_len, steps, seed):
    order = np.random.default_rng(seed).permutation(prompts * (prefix_len // B + 2 + samples * (steps // B + 2)))
    a = BlockAllocatorModel(len(order), B, order.tolist())
    for i in range(prompts):
        a.add(i * samples)
        a.append(i * samples, prefix_len)
        for c in range(1, samples):
            a.fork(i * samples, i * samples + c)
    seqs = list(range(prompts * samples))
    for _ in range(steps):
        for s in seqs:
            a.append(s, 1)
    width = -(-(prefix_len + steps) // B)
    tables, lens = a.build_batch(seqs, width)
    return tables, lens


@pytest.mark.parametrize("samples,max_members", [(8, 4), (8, 8), (5, 4), (3, 16)])
@pytest.mark.parametrize("steps", [1, 17, 200])
def test_parallel_sampling_closed_form(samples, max_members, steps):
    prompts, L = 6, 1000
    tables, lens = sampling_tables(prompts, samples, L, steps, seed=samples * 100 + steps)
    prefix, groups = shared_prefix_groups(tables, lens, B, max_members, min_blocks=1)
    check_grouping(tables, lens, prefix, groups, max_members, 1)
    per_prompt = math.ceil(samples / max_members)
    # a trailing run of one sample shares with nobody
    last = samples - (per_prompt - 1) * max_members
    expect_groups = prompts * (per_prompt - (1 if last == 1 else 0))
    assert len(groups) == expect_groups
    assert {k for _, _, k in groups} == {L // B}
    assert sum(m for _, m, _ in groups) == prompts * (samples - (1 if last == 1 else 0))


def test_random_fork_trees_hold_the_invariants():
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(40, 120))
        a = BlockAllocatorModel(n, B, rng.permutation(n).tolist())
        live = [0]
        a.add(0)
        a.append(0, int(rng.integers(1, 80)))
        nxt = 1
        for _ in range(int(rng.integers(5, 30))):
            op = rng.random()
            try:
                if op < 0.3 and len(live) < 12:
                    p = live[int(rng.integers(len(live)))]
                    a.fork(p, nxt)
                    live.append(nxt)
                    nxt += 1
                elif op < 0.4 and len(live) > 1:
                    s = live.pop(int(rng.integers(len(live))))
                    a.free_seq(s)
                else:
                    s = live[int(rng.integers(len(live)))]
                    a.append(s, int(rng.integers(1, 40)))
            except Exception:
                continue  # out of blocks: the model's state is unchanged
        order = sorted(live)
        width = max(1, max(-(-a.seq_len(s) // B) for s in order))
        tables, lens = a.build_batch(order, width)
        for mm in (2, 3, 16):
            for mb in (1, 2):
                prefix, groups = shared_prefix_groups(tables, lens, B, mm, mb)
                check_grouping(tables, lens, prefix, groups, mm, mb)


def test_prefix_and_rest_merge_to_the_whole_attention():
    """Attention over tokens [0, P) and over [P, n), merged by the log-sum-exp rule with each
    part's (max, sum, normalised output), equals attention over [0, n)."""
    rng = np.random.default_rng(3)
    D = 32
    for n, P in [(40, 16), (33, 32), (100, 96), (17, 16)]:
        q = rng.standard_normal(D)
        K = rng.standard_normal((n, D))
        V = rng.standard_normal((n, D))
        scale = float(np.float32(1 / math.sqrt(D)))  # the oracle takes the scale as float32

        def part(lo, hi):
            x = scale * K[lo:hi] @ q
            m = x.max()
            w = np.exp(x - m)
            return m, w.sum(), (w @ V[lo:hi]) / w.sum()

        m1, l1, o1 = part(0, P)
        m2, l2, o2 = part(P, n)
        M = max(m1, m2)
        a1, a2 = math.exp(m1 - M) * l1, math.exp(m2 - M) * l2
        merged = (a1 * o1 + a2 * o2) / (a1 + a2)
        ref = decode_attention_seq(q[None, :], K[:, None, :], V[:, None, :], scale)[0]
        assert np.max(np.abs(merged - ref)) < 1e-13


def test_cover_cuts_the_batch_into_runs_in_order():
    from oracle.shared_prefix import shared_prefix_cover
    tables = [[7, 8, 9, 10, -1], [7, 8, 9, 11, -1], [7, 8, 9, 12, -1], [7, 20, 21, -1, -1],
              [30, 31, -1, -1, -1], [30, 31, -1, -1, -1], [40, -1, -1, -1, -1]]
    lens = [64, 60, 40, 40, 31, 32, 16]
    assert shared_prefix_cover(tables, lens, B, 8, 2) == [(0, 3, 2), (3, 1, 0), (4, 1, 0), (5, 1, 0), (6, 1, 0)]
    assert shared_prefix_cover(tables, lens, B, 2, 1) == [(0, 2, 3), (2, 2, 1), (4, 2, 1), (6, 1, 0)]
    assert shared_prefix_cover([], [], B, 4, 1) == []
    rng = np.random.default_rng(2)
    for _ in range(30):
        S = int(rng.integers(1, 12))
        tables = rng.integers(0, 3, (S, 4)).tolist()
        lens = rng.integers(0, 70, S).tolist()
        runs = shared_prefix_cover(tables, lens, B, int(rng.integers(1, 5)), 1)
        assert [r[0] for r in runs] == list(np.cumsum([0] + [r[1] for r in runs[:-1]]))
        assert sum(r[1] for r in runs) == S
        assert all(r[2] == 0 for r in runs if r[1] == 1)

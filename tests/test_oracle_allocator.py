"""Pins for the allocator model: the rules the pages state, as checks.

* waste only in the last block, a new block exactly when the last one is full
  ("Stop Wasting GPU Memory" page, Technical Details, "Single Sequence
  Generation"; the ml-canon page's block-table sketch);
* shared blocks carry reference counts, copy-on-write copies only the diverging
  block and lowers the old count by one (same page, "Copy-on-Write for Parallel
  Sampling"; Chinese section 技术解析);
* one copy per branching event, and blocks at count zero go back to the free
  pool at once (same page, "Beam Search Optimization").

Plus exhaustive enumeration of every short operation sequence on a tiny pool
with the invariants checked after each step.
"""
import itertools

import pytest

from oracle.allocator_model import AllocError, BlockAllocatorModel

B = 16


def check_invariants(a: BlockAllocatorModel):
    used = [b for b in range(a.num_blocks) if a.refcount[b] > 0]
    # free pool + blocks in use == pool
    assert len(a.free) + len(used) == a.num_blocks
    assert len(set(a.free)) == len(a.free)
    # refcount 0 <=> in the free pool
    assert set(a.free) == {b for b in range(a.num_blocks) if a.refcount[b] == 0}
    # refcount conservation: every table entry is one reference
    assert sum(a.refcount) == sum(len(t) for t in a.block_table.values())
    for s, t in a.block_table.items():
        n = a.length[s]
        # table covers exactly ceil(len / B) blocks: waste < B, all in the last block
        assert len(t) == -(-n // a.block_size)
        assert len(t) * a.block_size - n < a.block_size or n == 0
        for b in t:
            assert a.refcount[b] >= 1


def test_new_block_exactly_when_last_is_full():
    a = BlockAllocatorModel(8, B)
    a.add(0)
    for pos in range(70):
        before = len(a.table(0))
        slots, pairs = a.append(0, 1)
        assert pairs == []
        assert (len(a.table(0)) == before + 1) == (pos % B == 0)
        # the token sits in block table[pos // B] at offset pos % B
        assert slots == [a.table(0)[pos // B] * B + pos % B]
        check_invariants(a)
    assert a.seq_len(0) == 70 and len(a.table(0)) == 5


def test_fresh_pool_hands_out_in_free_order():
    order = [5, 2, 7, 0, 1, 3, 6, 4]
    a = BlockAllocatorModel(8, B, order)
    a.add(0)
    a.append(0, 8 * B)
    assert a.table(0) == order
    with pytest.raises(AllocError) as e:
        a.append(0, 1)
    assert e.value.status == "PA_ERR_OUT_OF_BLOCKS"


def test_bulk_append_equals_token_by_token():
    a1 = BlockAllocatorModel(16, B, list(range(15, -1, -1)))
    a2 = BlockAllocatorModel(16, B, list(range(15, -1, -1)))
    a1.add(3)
    a2.add(3)
    s1, _ = a1.append(3, 50)
    s2 = []
    for _ in range(50):
        s2 += a2.append(3, 1)[0]
    assert s1 == s2 and a1.table(3) == a2.table(3)


def test_fork_shares_blocks_by_refcount():
    a = BlockAllocatorModel(10, B)
    a.add(0)
    a.append(0, 40)                      # 3 blocks, last holds 8 tokens
    for c in range(1, 4):
        a.fork(0, c)
    t = a.table(0)
    for c in range(1, 4):
        assert a.table(c) == t and a.seq_len(c) == 40
    assert [a.refcount[b] for b in t] == [4, 4, 4]
    check_invariants(a)


def test_copy_on_write_copies_only_the_diverging_block():
    # k branches share a partial last block: the first k-1 writers each copy it once,
    # the last writer holds it alone and writes in place.
    k = 8
    a = BlockAllocatorModel(80, B)
    a.add(0)
    a.append(0, 1000)                    # 62 full blocks + 8 tokens in block 63
    for c in range(1, k):
        a.fork(0, c)
    shared = a.table(0)
    last = shared[-1]
    assert a.refcount[last] == k
    copies = []
    for c in range(k):
        slots, pairs = a.append(c, 1)
        copies += pairs
        t = a.table(c)
        assert t[:-1] == shared[:-1]                    # history stays shared
        assert slots == [t[-1] * B + 1000 % B]
        check_invariants(a)
    assert len(copies) == k - 1                         # one copy per divergence
    assert all(src == last for src, _ in copies)
    assert len({dst for _, dst in copies}) == k - 1
    assert a.table(k - 1)[-1] == last and a.refcount[last] == 1
    for _, dst in copies:
        assert a.refcount[dst] == 1
    # the full shared blocks are still referenced by all k branches
    assert all(a.refcount[b] == k for b in shared[:-1])
    # physical blocks: 62 shared + 8 private last blocks, against 8 * 63 unshared
    assert a.num_blocks - a.num_free() == 62 + k


def test_no_copy_when_shared_block_is_full():
    a = BlockAllocatorModel(10, B)
    a.add(0)
    a.append(0, 32)                      # exactly 2 full blocks
    a.fork(0, 1)
    _, p0 = a.append(0, 1)
    _, p1 = a.append(1, 1)
    assert p0 == [] and p1 == []
    assert a.table(0)[:2] == a.table(1)[:2] and a.table(0)[2] != a.table(1)[2]
    check_invariants(a)


def test_free_returns_blocks_at_zero_immediately_lifo():
    a = BlockAllocatorModel(10, B)
    a.add(0)
    a.append(0, 20)                      # blocks 0, 1
    a.fork(0, 1)
    a.append(1, 20)                      # CoW of block 1 -> 2, then block 3
    assert a.table(1) == [0, 2, 3]
    n_free = a.num_free()
    a.free_seq(1)                        # block 0 still held by seq 0; 2 and 3 freed
    assert a.num_free() == n_free + 2
    assert a.refcount[0] == 1 and a.refcount[2] == 0 and a.refcount[3] == 0
    check_invariants(a)
    a.add(5)
    a.append(5, 1)
    assert a.table(5) == [3]             # last freed, first handed out
    a.free_seq(0)
    assert a.refcount[0] == 0 and a.refcount[1] == 0
    check_invariants(a)


def test_beam_prune_tree():
    # A beam tree: a root prompt, two beams, each beam splits again, two leaves pruned.
    a = BlockAllocatorModel(64, B)
    a.add(0)
    a.append(0, 24)
    a.fork(0, 1)
    a.append(0, 10)
    a.append(1, 10)
    a.fork(1, 2)
    a.fork(0, 3)
    for s in (0, 1, 2, 3):
        a.append(s, 5)
        check_invariants(a)
    a.free_seq(3)
    a.free_seq(2)
    check_invariants(a)
    a.free_seq(0)
    a.free_seq(1)
    check_invariants(a)
    assert a.num_free() == 64


def test_out_of_blocks_changes_nothing():
    a = BlockAllocatorModel(3, B)
    a.add(0)
    a.append(0, 20)
    a.fork(0, 1)                         # block 1 shared, partial
    snapshot = (list(a.free), list(a.refcount), a.table(0), a.table(1), a.seq_len(1))
    with pytest.raises(AllocError) as e:
        a.append(1, 30)                  # needs 1 CoW + 1 fresh = 2 > 1 free
    assert e.value.status == "PA_ERR_OUT_OF_BLOCKS"
    assert snapshot == (list(a.free), list(a.refcount), a.table(0), a.table(1), a.seq_len(1))


def test_errors():
    a = BlockAllocatorModel(4, B)
    a.add(0)
    for fn in (lambda: a.add(0), lambda: a.fork(7, 1), lambda: a.fork(0, 0),
               lambda: a.append(9, 1), lambda: a.free_seq(9), lambda: a.append(0, -1)):
        with pytest.raises(AllocError) as e:
            fn()
        assert e.value.status == "PA_ERR_INVALID_ARG"
    with pytest.raises(AllocError):
        BlockAllocatorModel(4, B, [0, 1, 1, 2])


def test_build_batch_pads_with_minus_one():
    a = BlockAllocatorModel(8, B, [7, 6, 5, 4, 3, 2, 1, 0])
    a.add(10)
    a.add(11)
    a.append(10, 17)
    a.append(11, 3)
    tables, lens = a.build_batch([11, 10], 3)
    assert tables == [[5, -1, -1], [7, 6, -1]] and lens == [3, 17]


OPS = ("add", "fork", "app1", "app16", "app5", "free")


def _apply(a, op, ids):
    live = sorted(a.block_table)
    if op == "add":
        a.add(ids[0])
        ids[0] += 1
    elif not live:
        return
    elif op == "fork":
        a.fork(live[-1], ids[0])
        ids[0] += 1
    elif op == "free":
        a.free_seq(live[0])
    else:
        n = {"app1": 1, "app16": 16, "app5": 5}[op]
        need = a.blocks_needed(live[-1], n)
        try:
            slots, pairs = a.append(live[-1], n)
        except AllocError as e:
            assert e.status == "PA_ERR_OUT_OF_BLOCKS" and need > a.num_free()
            return
        assert len(slots) == n and len(set(slots)) == n
        for s in slots:
            assert a.refcount[s // a.block_size] == 1        # every write hits a private block
        assert len(pairs) <= 1


def test_exhaustive_short_sequences_on_tiny_pool():
    count = 0
    for seq in itertools.product(OPS, repeat=6):
        a = BlockAllocatorModel(4, 4)
        ids = [0]
        for op in seq:
            _apply(a, op, ids)
            check_invariants(a)
        count += 1
    assert count == len(OPS) ** 6

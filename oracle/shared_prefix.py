"""Which sequences of a decode batch read the same leading blocks (oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, never by the library.

Forked sequences (parallel samples of one prompt, beams of one search) keep
pointing at the same physical blocks for everything they have in common, and a
block is copied only when a branch writes into one it shares ("Stop Wasting GPU
Memory" page, Technical Details, "Copy-on-Write for Parallel Sampling" and
"Beam Search Optimization"; the zhichai.net page, Key points: new blocks only
when sequences diverge).  So the block tables of such a batch hold the same
physical ids in their leading entries.  Those blocks hold the same K/V for every
sharer, and attention over them can be computed once for all sharers' queries,
then merged with each sharer's own blocks by the log-sum-exp rule.  The softmax
is unchanged (the zhichai.net page, Key points: the attention math is not
altered by paging).

The grouping rule (index work, compared bit for bit with the library's):

* full(s) = min(floor(len_s / B), row width): the blocks sequence s fills
  completely.  Only full blocks are shared through the prefix pass, so every
  member reads all B tokens of each prefix block.
* Groups are runs of consecutive sequences in batch order.  A run starts at the
  first sequence i not yet grouped with candidate prefix k = full(i).  The next
  sequence j joins while the run has fewer than ``max_members`` members and
      k' = min(k, full(j), common leading entries of row i and row j)
  is at least ``min_blocks``; then k = k'.  Row i is compared with row j
  because every member already equals row i on [0, k).
* A run of at least two members is a group (first sequence, members, k), and
  prefix[s] = k for its members; everything else has prefix 0.  The next run
  starts right after the last member (or at i + 1 for a run of one).
"""
from __future__ import annotations


def shared_prefix_groups(tables, lens, block_size: int, max_members: int, min_blocks: int):
    """Returns (prefix: list[int] per sequence, groups: list[(first, members, prefix_blocks)])."""
    if block_size <= 0 or max_members < 1 or min_blocks < 1:
        raise ValueError("block_size and max_members must be positive, min_blocks at least 1")
    S = len(lens)
    width = len(tables[0]) if S else 0
    full = [min(int(lens[s]) // block_size, width) if int(lens[s]) > 0 else 0 for s in range(S)]
    prefix = [0] * S
    groups = []
    i = 0
    while i < S:
        k = full[i]
        members = 1
        j = i + 1
        while j < S and members < max_members:
            common = 0
            lim = min(k, full[j])
            while common < lim and int(tables[i][common]) == int(tables[j][common]):
                common += 1
            if common < min_blocks:
                break
            k = common
            members += 1
            j += 1
        if members >= 2:
            groups.append((i, members, k))
            for s in range(i, i + members):
                prefix[s] = k
            i += members
        else:
            i += 1
    return prefix, groups


def shared_prefix_cover(tables, lens, block_size: int, max_members: int, min_blocks: int):
    """The batch cut into runs, in order: the groups above and every other sequence as a run of one
    with no shared blocks.  Returns [(first, members, prefix_blocks)]."""
    _, groups = shared_prefix_groups(tables, lens, block_size, max_members, min_blocks)
    runs = []
    s = 0
    for first, members, k in groups + [(len(lens), 0, 0)]:
        while s < first:
            runs.append((s, 1, 0))
            s += 1
        if members:
            runs.append((first, members, k))
            s = first + members
    return runs

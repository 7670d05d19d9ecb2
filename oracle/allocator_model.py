"""Pure-Python model of the paged KV block allocator (oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU baseline; never by the library.

Policy, in the order the pages describe it:

* Blocks.  The cache is cut into fixed-size blocks of B tokens (default 16) and
  each sequence owns a block table mapping its logical blocks to physical ones
  ("Stop Wasting GPU Memory" page, Technical Details, "Core Architecture"; the
  ml-canon page's box "Paging for the KV cache" and its block-table sketch).
* Appending.  A token is written into the current last block; a new physical
  block is taken from the free pool only when the last one is full, so waste is
  confined to the unfilled slots of the last block (same page, "Single Sequence
  Generation"; the sketch's test for whether the table needs one more block, read with len = tokens
  before this append, so a block is taken exactly when len % B == 0).  The
  token's slot is  table[-1] * B + len % B  (the sketch writes into the last
  block without naming the offset; len % B is the offset its test implies), and
  len grows by one.
* Sharing.  Forked branches reference the same physical blocks; each physical
  block carries a reference count (same page, "Copy-on-Write for Parallel
  Sampling"; the Chinese section 技术解析 on Copy-on-Write).
* Copy-on-write.  A write into a block whose reference count is above one copies
  only that block to a fresh physical block, decrements the old block's count
  and points the writer's table at the copy (count 1).  A write into a block
  the writer holds alone (count 1) happens in place — so of k branches sharing
  a partial block, k-1 copy and the last writer keeps the original.  The copy
  happens at the first write, not at the fork, and only for a partial block:
  when len % B == 0 the token opens a fresh block and nothing is copied.
* Release.  Freeing a sequence (a finished or pruned beam) decrements the
  count of each block in its table, in logical order; a block reaching zero is
  returned to the free pool at once (same page, "Beam Search Optimization").

Readings where the pages are silent:

* Which free block ``alloc()`` returns: the pool is a LIFO stack.  A fresh pool
  hands blocks out in the caller's ``free_order`` (first element first, default
  0, 1, 2, ...); freed blocks are pushed on top and handed out first.
* Out of blocks: an append first counts the blocks it needs (new blocks plus
  one copy-on-write target) and fails with no state change if the pool is short.
* Errors: unknown or duplicate sequence ids, negative counts, forks onto an
  existing id raise ``AllocError`` with the status name the C library uses.
"""
from __future__ import annotations


class AllocError(Exception):
    def __init__(self, status: str, msg: str = ""):
        super().__init__(f"{status}: {msg}")
        self.status = status


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError("PA_ERR_INVALID_ARG", "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError("PA_ERR_INVALID_ARG", "free_order must be a permutation")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(reversed(order))        # top of the stack = end of the list
        self.refcount = [0] * num_blocks
        self.block_table: dict[int, list[int]] = {}  # sequence id -> [phys_block, ...]
        self.length: dict[int, int] = {}

    # -- the pool
    def _alloc(self) -> int:
        b = self.free.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        assert self.refcount[b] >= 0
        if self.refcount[b] == 0:
            self.free.append(b)

    # -- sequences
    def add(self, seq: int) -> None:
        if seq in self.block_table:
            raise AllocError("PA_ERR_INVALID_ARG", f"sequence {seq} exists")
        self.block_table[seq] = []
        self.length[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.block_table:
            raise AllocError("PA_ERR_INVALID_ARG", f"unknown sequence {parent}")
        if child in self.block_table:
            raise AllocError("PA_ERR_INVALID_ARG", f"sequence {child} exists")
        table = list(self.block_table[parent])
        for b in table:
            self.refcount[b] += 1
        self.block_table[child] = table
        self.length[child] = self.length[parent]

    def blocks_needed(self, seq: int, n: int) -> int:
        blocks = self.block_table[seq]
        length = self.length[seq]
        B = self.block_size
        fresh = -(-(length + n) // B) - (-(-length // B))
        cow = 1 if (n > 0 and length % B != 0 and self.refcount[blocks[-1]] > 1) else 0
        return fresh + cow

    def append(self, seq: int, n: int = 1):
        """Append n tokens.  Returns (slots, copy_pairs): the cache slot of each
        token, and the (src, dst) block copies the device must do first."""
        if seq not in self.block_table:
            raise AllocError("PA_ERR_INVALID_ARG", f"unknown sequence {seq}")
        if n < 0:
            raise AllocError("PA_ERR_INVALID_ARG", "negative token count")
        if self.blocks_needed(seq, n) > len(self.free):
            raise AllocError("PA_ERR_OUT_OF_BLOCKS", f"sequence {seq} needs more blocks")
        blocks = self.block_table[seq]
        B = self.block_size
        slots, pairs = [], []
        for _ in range(n):
            length = self.length[seq]
            if len(blocks) * B <= length:            # last block full (or none): open a new one
                blocks.append(self._alloc())
            elif self.refcount[blocks[-1]] > 1:      # shared partial block: copy on write
                old = blocks[-1]
                new = self._alloc()
                self.refcount[old] -= 1              # still >= 1: another branch holds it
                blocks[-1] = new
                pairs.append((old, new))
            slots.append(blocks[-1] * B + length % B)
            self.length[seq] = length + 1
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        if seq not in self.block_table:
            raise AllocError("PA_ERR_INVALID_ARG", f"unknown sequence {seq}")
        for b in self.block_table.pop(seq):
            self._release(b)
        del self.length[seq]

    # -- views
    def table(self, seq: int) -> list[int]:
        return list(self.block_table[seq])

    def seq_len(self, seq: int) -> int:
        return self.length[seq]

    def num_free(self) -> int:
        return len(self.free)

    def build_batch(self, seqs, max_blocks: int):
        """Block tables padded with -1 to ``max_blocks`` columns, and lengths."""
        tables, lens = [], []
        for s in seqs:
            t = self.block_table[s]
            if len(t) > max_blocks:
                raise AllocError("PA_ERR_INVALID_ARG", "table longer than max_blocks")
            tables.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.length[s])
        return tables, lens

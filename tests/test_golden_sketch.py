"""Pin the allocator model to a trace derived by hand from the pages' block-table sketch
(tests/golden/sketch_append_trace.txt; ml-canon page "49 vLLM / PagedAttention", the block-table
box; "Stop Wasting GPU Memory" page, Technical Details, "Single Sequence Generation")."""
import os

from oracle.allocator_model import BlockAllocatorModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sketch_append_trace.txt")


def _rows():
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            n, blocks, new, waste = line.split()
            yield int(n), int(blocks), new == "yes", int(waste)


def test_model_follows_the_sketch_trace():
    rows = {n: (b, new, w) for n, b, new, w in _rows()}
    m = BlockAllocatorModel(16, 16)
    m.add(0)
    held = 0
    for n in range(1, max(rows) + 1):
        m.append(0, 1)
        table = m.table(0)
        took = len(table) > held
        held = len(table)
        if n in rows:
            blocks, new, waste = rows[n]
            assert len(table) == blocks, n
            assert took == new, n
            assert len(table) * 16 - n == waste, n

"""pa_prefill_order (host): sequences by descending prefill work, ties in batch order.

The work of a sequence with n cached tokens whose last c are the chunk is the number of (row, token)
pairs the causal attention visits: row i sits at position n - c + i and sees that many tokens plus
one, rows at negative positions see none.  Checked against that count taken row by row.
"""
import numpy as np
import pytest

import paged_kv_cache_358_amd as pa


def _work_by_rows(n, c):
    return sum(max(0, n - c + i + 1) for i in range(c))


@pytest.mark.parametrize("seed", range(6))
def test_order_is_descending_work_stable_on_ties(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 60))
    lens = rng.integers(0, 3000, size=S).astype(np.int32)
    lens[rng.random(S) < 0.3] = 64                       # ties
    chunks = np.minimum(rng.integers(0, 700, size=S), lens + rng.integers(0, 3, size=S))  # a few c > n
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    order = pa.prefill_order(lens, qs)
    work = [_work_by_rows(int(lens[s]), int(chunks[s])) for s in range(S)]
    assert sorted(order.tolist()) == list(range(S))
    assert order.tolist() == sorted(range(S), key=lambda s: (-work[s], s))


def test_closed_cases():
    # one row at the end of a 100-token context sees 100 tokens; a whole-sequence chunk of 4 sees
    # 1 + 2 + 3 + 4; a chunk longer than its context has rows without a position
    lens = np.array([100, 4, 2, 0], np.int32)
    qs = np.array([0, 1, 5, 8, 8], np.int32)
    assert [_work_by_rows(100, 1), _work_by_rows(4, 4), _work_by_rows(2, 3), 0] == [100, 10, 3, 0]
    assert pa.prefill_order(lens, qs).tolist() == [0, 1, 2, 3]
    assert pa.prefill_order(np.zeros(0, np.int32), np.zeros(1, np.int32)).size == 0
    with pytest.raises(ValueError):
        pa.prefill_order(lens, qs[:-1])

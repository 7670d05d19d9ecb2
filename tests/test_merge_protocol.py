"""CPU models of the split decode kernel's cross-workgroup merge (no GPU).

The split kernel cuts the weighted partitions of all (sequence, KV head) contexts into one
contiguous run per workgroup.  A context that spans several runs is merged by the run that
publishes its last partial; the partials live in the workspace per run (two slots each) and an
arrival counter per context counts published partitions.  Two things must hold:

* the schedule: every partial a run writes for a context is read by that context's merger, from
  the same (run, slot), and no two partials share a slot;
* the arrival counter: whatever interleaving of the runs' atomic operations, and whatever the
  counter held before the launch, exactly one run sees its add complete the count, and the count
  ends exact.

Both are restated here from the kernel's rules (weights, chunk bounds, slot choice, and the
load / compare-and-swap / fetch-add sequence of ``arrive``) and checked on many shapes and, for
the counter, on every interleaving of up to four runs.
"""
import bisect
import random

import pytest

MASK32 = (1 << 32) - 1
MASK64 = (1 << 64) - 1


# ----------------------------------------------------------------------------- the schedule
def chunk_lo(j, W, R, NR):
    r, t = divmod(j, R)
    if r >= NR:
        return W
    T0 = W - (W >> r)
    T1 = W if r + 1 >= NR else W - (W >> (r + 1))
    return T0 + (T1 - T0) * t // R


def chunk_owner(off, W, R, NR):
    r = 0
    while r + 1 < NR and W - (W >> (r + 1)) <= off:
        r += 1
    T0 = W - (W >> r)
    T1 = W if r + 1 >= NR else W - (W >> (r + 1))
    return r * R + ((off - T0 + 1) * R - 1) // (T1 - T0)


def simulate(nbs, hkv, PB, C, CE, J, NR):
    """Run the schedule of one launch: returns (writes, reads) as {context: set of (run, slot,
    first partition, partitions)} for the runs' partials and the mergers' reads."""
    def wnb(nb):
        return 0 if nb == 0 else nb + C * (-(-nb // PB)) + CE
    PW = PB + C
    starts = []  # (weighted start, context, partition, partitions of the context)
    A = {}
    off = 0
    for s, nb in enumerate(nbs):
        for h in range(hkv):
            A[(s, h)] = off
            np_ = -(-nb // PB)
            for p in range(np_):
                starts.append((off + p * PW, (s, h), p, np_))
            off += wnb(nb)
    W = off
    R = J // NR
    keys = [x[0] for x in starts]  # increasing
    writes, counts = {}, {}
    merged = set()
    for k in range(J):
        lo, hi = chunk_lo(k, W, R, NR), chunk_lo(k + 1, W, R, NR)
        mine = starts[bisect.bisect_left(keys, lo):bisect.bisect_left(keys, hi)]
        segs = []
        for st, ctx, p, np_ in mine:
            if segs and segs[-1][0] == ctx:
                segs[-1][2] = p
            else:
                segs.append([ctx, p, p, np_])
        for i, (ctx, p0, p1, np_) in enumerate(segs):
            if p0 == 0 and p1 == np_ - 1:
                continue  # the whole context in one run: written as output, no partial
            slot = 0 if i == len(segs) - 1 else 1
            assert i in (0, len(segs) - 1), "only a run's first and last segments can be partial"
            writes.setdefault(ctx, set()).add((k, slot, p0, p1 - p0 + 1))
            counts[ctx] = counts.get(ctx, 0) + (p1 - p0 + 1)
    reads = {}
    for ctx, total in counts.items():
        s, h = ctx
        np_ = -(-nbs[s] // PB)
        assert total == np_, "the runs' partials cover every partition once"
        a = A[ctx]
        k0 = chunk_owner(a, W, R, NR)
        k1 = chunk_owner(a + (np_ - 1) * PW, W, R, NR)
        nr = k1 - k0 + 1
        run_p0 = [0] + [-(-(chunk_lo(k0 + i, W, R, NR) - a) // PW) for i in range(1, nr)] + [np_]
        last_slot = 1 if a + wnb(nbs[s]) < chunk_lo(k1 + 1, W, R, NR) else 0
        for r in range(nr):
            if run_p0[r] < run_p0[r + 1]:
                reads.setdefault(ctx, set()).add(
                    (k0 + r, last_slot if r == nr - 1 else 0, run_p0[r], run_p0[r + 1] - run_p0[r]))
        merged.add(ctx)
    return writes, reads, W


def test_chunk_owner_inverts_chunk_lo():
    rng = random.Random(1)
    for _ in range(300):
        NR = rng.choice([1, 1, 2, 3])
        R = rng.choice([1, 2, 8, 64, 512])
        W = rng.randint(1, 200000)
        J = R * NR
        for off in sorted({0, W - 1, *(rng.randrange(W) for _ in range(50))}):
            k = chunk_owner(off, W, R, NR)
            assert 0 <= k < J
            assert chunk_lo(k, W, R, NR) <= off < chunk_lo(k + 1, W, R, NR)


@pytest.mark.parametrize("seed", range(40))
def test_every_partial_is_read_from_the_slot_it_was_written_to(seed):
    rng = random.Random(seed)
    S = rng.choice([1, 2, 4, 7, 64, 256])
    hkv = rng.choice([1, 2, 8, 32])
    PB = rng.choice([1, 2, 4, 32, 64])
    kind = rng.choice(["uniform", "long", "mixed"])
    if kind == "uniform":
        nbs = [rng.randint(1, 128) for _ in range(S)]
    elif kind == "long":
        nbs = [rng.randint(1000, 9000) for _ in range(S)]
    else:
        nbs = [rng.choice([0, 1, 2, rng.randint(1, 600)]) for _ in range(S)]
    while sum(-(-nb // PB) for nb in nbs) * hkv > 200000:  # keep the model's partition count small
        PB *= 2
    J = rng.choice([1, 3, 8, 256, 512, 1024])
    NR = rng.choice([1, 1, 2]) if J % 2 == 0 else 1
    C, CE = rng.choice([(5, 5), (0, 0), (3, 12)])
    writes, reads, W = simulate(nbs, hkv, PB, C, CE, J, NR)
    assert writes.keys() == reads.keys()
    for ctx in writes:
        assert writes[ctx] == reads[ctx], ctx
    slots = [(k, slot) for w in writes.values() for (k, slot, _, _) in w]
    assert len(slots) == len(set(slots)), "two partials in one slot"


def test_context_ending_exactly_at_a_run_boundary():
    # One context per run, cut at run edges: the merger must read slot 0 of the last run.
    for J in (2, 3, 4, 5):
        writes, reads, W = simulate([40], 1, 4, 0, 0, J, 1)
        assert writes == reads


# ----------------------------------------------------------------------------- the arrival counter
def arrive_steps(tag, add, load_first=True):
    """``arrive`` as a sequence of atomic steps on one 64-bit word.  A generator: it yields a
    function applied atomically to the counter (returning the value it reads, and the new value
    or None), receives what that step read, and finally returns the count before this run's add."""
    mine = tag << 32
    if load_first:
        old = yield ("load", None)
        while (old >> 32) != tag:
            ok, old = yield ("cas", (old, mine | add))
            if ok:
                return 0
        old = yield ("add", add)
        return old & MASK32
    # the fetch-add-first protocol: the add may land on a stale counter first
    old = yield ("add", add)
    if (old >> 32) == tag:
        return old & MASK32
    old = yield ("load", None)
    while (old >> 32) != tag:
        ok, old = yield ("cas", (old, mine | add))
        if ok:
            return 0
    old = yield ("add", add)
    return old & MASK32


def apply(op, arg, ctr):
    if op == "load":
        return ctr, ctr
    if op == "add":
        return ctr, (ctr + arg) & MASK64
    expect, new = arg
    if ctr == expect:
        return (True, ctr), new
    return (False, ctr), ctr


def all_schedules(adds, tag, init, load_first):
    """Every interleaving of the runs' atomic steps: yields (final counter, [count before each
    run's add]).  A run is replayed from the values its steps read so far (generators cannot be
    copied), so each branch of the search holds only those histories."""
    def state(i, history):
        g = arrive_steps(tag, adds[i], load_first)
        req = g.send(None)
        for got in history:
            try:
                req = g.send(got)
            except StopIteration as e:
                return ("done", e.value)
        return ("next", req)

    def rec(hist, ctr, results):
        live = [i for i in range(len(adds)) if results[i] is None]
        if not live:
            yield ctr, list(results)
            return
        for i in live:
            op, arg = state(i, hist[i])[1]
            got, new = apply(op, arg, ctr)
            h2 = list(hist)
            h2[i] = hist[i] + (got,)
            r2 = list(results)
            after = state(i, h2[i])
            if after[0] == "done":
                r2[i] = after[1]
            yield from rec(h2, new, r2)

    yield from rec([() for _ in adds], init, [None] * len(adds))


TAG = 0x1234ABCD
INITIAL = {
    "previous launch": ((TAG - 1) << 32) | 7,
    "other process": (0x0BADF00D << 32) | 123456,
    "this launch's tag, count 0": TAG << 32,
    "zeroed": 0,
    "all ones": MASK64,
    "stale tag, low word near 2^32": ((TAG - 1) << 32) | (MASK32 - 1),
    "stale tag, low word 2^32 - 1": ((TAG - 1) << 32) | MASK32,
}


@pytest.mark.parametrize("name", sorted(INITIAL))
@pytest.mark.parametrize("adds", [(1, 1, 1), (2, 1, 3), (1, 2, 1, 1)])
def test_arrive_counts_exactly_under_every_interleaving(name, adds):
    init = INITIAL[name]
    if init >> 32 == TAG and init & MASK32:
        pytest.skip("a counter with this launch's tag and a nonzero count is not a stale state")
    total = sum(adds)
    n = 0
    for final, before in all_schedules(adds, TAG, init, load_first=True):
        n += 1
        assert final == (TAG << 32) | total
        # exactly one run completes the count, and the counts before each add are distinct prefixes
        assert sum(b + a == total for b, a in zip(before, adds)) == 1
        assert sorted(before) == sorted(set(before))
        assert all(0 <= b < total for b in before)
    assert n > len(adds)


def test_fetch_add_first_can_forge_the_tag():
    # The earlier protocol added before looking: on a stale counter whose low word is near 2^32 the
    # add carries into the tag and forges this launch's tag with a bogus count.  No run then sees its
    # add complete the count (the context would never be merged) in some interleaving.
    init = INITIAL["stale tag, low word near 2^32"]
    adds = (2, 1, 1)
    bad = [b for _, b in all_schedules(adds, TAG, init, load_first=False)
           if sum(x + a == sum(adds) for x, a in zip(b, adds)) != 1]
    assert bad

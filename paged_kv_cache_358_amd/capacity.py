"""KV-cache capacity of paged blocks against contiguous per-request reservation (host only).

The pages' comparison:
* A contiguous system reserves, per request, a buffer for the maximum length; the slots a
  shorter request never fills sit idle.  They put the waste at 60-80% ("Stop Wasting GPU
  Memory" page, TL;DR; "PagedAttention: How Virtual Memory Paging Solved LLM KV Cache
  Waste" page, "The KV cache problem"; ml-canon page, "Paging for the KV cache", internal
  fragmentation).
* Paged blocks bound the waste to the unfilled slots of each sequence's last block
  ("Stop Wasting GPU Memory" page, Technical Details, "Single Sequence Generation"), under 4%;
  forks share blocks until they diverge ("Copy-on-Write for Parallel Sampling").
* Less waste means more requests in the same memory, the source of the pages' 2-4x
  throughput (ml-canon page, "where the x2-4 comes from").
* Beam search and shared system prompts: beams and requests with a common prefix hold its
  blocks once ("Stop Wasting GPU Memory" page, "Beam Search Optimization"; ml-canon page,
  prefix sharing).  Beside the blocks held, the study counts the K/V tokens one decode step
  reads: per sequence, or with the batch cut into groups that read their shared blocks once
  (``shared_prefixes``, as the decode kernel does).

The paged side is counted by running the library's own block allocator over the lengths
(``BlockAllocator``), so forks and copy-on-write are the real ones; the contiguous side is
the plain arithmetic of a max-length reservation.

    python -m paged_kv_cache_358_amd.capacity        # one JSON line per workload
"""
from __future__ import annotations

import hashlib
import json

import numpy as np

from . import BlockAllocator, shared_prefixes


def paged_footprint(lens, block_size: int = 16) -> dict:
    """Blocks the allocator hands out for sequences of `lens` tokens (no sharing)."""
    lens = [int(x) for x in lens]
    need = sum(-(-n // block_size) for n in lens)
    alloc = BlockAllocator(max(need, 1), block_size)
    for i, n in enumerate(lens):
        alloc.add(i)
        if n:
            alloc.append(i, n)
    blocks = alloc.num_blocks - alloc.num_free()
    return _summary(blocks * block_size, sum(lens), blocks=blocks)


def contiguous_footprint(lens, reserve: int) -> dict:
    """Each request reserves `reserve` token slots up front."""
    lens = [int(x) for x in lens]
    if any(n > reserve for n in lens):
        raise ValueError("a request is longer than the reservation")
    return _summary(len(lens) * reserve, sum(lens))


def sampling_footprint(prompts: int, samples: int, prefix_len: int, new_tokens: int, block_size: int = 16) -> dict:
    """Parallel sampling: each prompt is forked into `samples` sequences that share its
    blocks; every sample then appends `new_tokens`, copying a shared partial block on its
    first write.  Returns the allocator's block count with sharing and without."""
    full = prefix_len // block_size
    per_seq = -(-(prefix_len + new_tokens) // block_size)
    cap = prompts * (full + samples * (per_seq - full + 1)) + 1
    alloc = BlockAllocator(cap, block_size)
    seqs = []
    for p in range(prompts):
        root = p * samples
        alloc.add(root)
        alloc.append(root, prefix_len)
        seqs.append(root)
        for c in range(1, samples):
            alloc.fork(root, root + c)
            seqs.append(root + c)
    ones = np.ones(len(seqs), np.int32)
    for _ in range(new_tokens):
        alloc.append_batch(seqs, ones)
    shared = alloc.num_blocks - alloc.num_free()
    unshared = len(seqs) * per_seq
    return {"tokens": len(seqs) * (prefix_len + new_tokens), "blocks": shared, "blocks_without_sharing": unshared,
            "saved_frac": round(1.0 - shared / unshared, 4)}


def beam_search_footprint(width: int, prompt_len: int, steps: int, block_size: int = 16, seed: int = 0,
                          skew: float = 1.5, alloc_factory=None) -> dict:
    """Beam search as a process tree ("Stop Wasting GPU Memory" page, Technical Details, "Beam
    Search Optimization"): each step every new beam forks the beam it extends, the old beams
    are freed (a pruned beam's blocks go back to the pool when no beam holds them), and every
    beam appends its token (copying a shared partial block on the first write).  Parents are
    drawn from a seeded generator, beam r with weight r^-skew (skew 0: uniform; larger: a few
    beams take most of the children, as a search that keeps extending its best paths).
    Returns peak and mean blocks with sharing and without (every beam holding its whole
    history).  `alloc_factory(num_blocks, block_size)` builds the allocator (the library's by
    default)."""
    rng = np.random.default_rng(seed)
    worst = width * -(-(prompt_len + steps) // block_size)
    alloc = (alloc_factory or BlockAllocator)(worst + width + 1, block_size)
    next_id = 0
    alloc.add(next_id)
    alloc.append(next_id, prompt_len)
    beams = [next_id] * width
    live = {next_id}
    shared, unshared = [], []
    reads, reads_grouped = [], []
    weights = 1.0 / np.arange(1, width + 1) ** skew
    weights /= weights.sum()
    for t in range(steps):
        parents = rng.choice(np.arange(width), size=width, p=weights) if t else np.zeros(width, int)
        children = []
        for par in parents:
            next_id += 1
            alloc.fork(beams[par], next_id)
            children.append(next_id)
        for old in sorted(live):
            alloc.free(old)
        live = set(children)
        beams = children
        alloc.append_batch(children, np.ones(len(children), np.int32))
        shared.append(alloc.num_blocks - alloc.num_free())
        unshared.append(width * -(-(prompt_len + t + 1) // block_size))
        # the decode batch with children of one parent next to each other
        batch = [children[i] for i in np.argsort(parents, kind="stable")]
        total, grouped = step_read_tokens(alloc, batch, block_size)
        reads.append(total)
        reads_grouped.append(grouped)
    return {"width": width, "prompt_len": prompt_len, "steps": steps, "skew": skew,
            "peak_blocks": int(max(shared)), "peak_blocks_without_sharing": int(max(unshared)),
            "mean_saved_frac": round(1.0 - float(np.mean(shared)) / float(np.mean(unshared)), 4),
            "peak_saved_frac": round(1.0 - max(shared) / max(unshared), 4),
            "mean_read_tokens": round(float(np.mean(reads)), 1),
            "mean_read_tokens_grouped": round(float(np.mean(reads_grouped)), 1),
            "read_saved_frac": round(1.0 - float(np.sum(reads_grouped)) / float(np.sum(reads)), 4)}


class PrefixIndex:
    """Shared prompts held once: the index maps a prompt's tokens to a sequence that holds its
    blocks, and a request with that prompt forks from it (ml-canon page, "prefix sharing":
    a long system prompt stored once and referenced from every request, copy-on-write)."""

    def __init__(self, alloc, first_id: int):
        self.alloc = alloc
        self._holders = {}
        self._next = first_id

    def holder(self, prompt) -> int:
        """The sequence holding `prompt` (tokens), allocated on first use."""
        key = hashlib.sha256(np.asarray(prompt, dtype=np.int64).tobytes()).hexdigest()
        if key not in self._holders:
            h = self._next
            self._next += 1
            self.alloc.add(h)
            self.alloc.append(h, len(prompt))
            self._holders[key] = h
        return self._holders[key]


def step_read_tokens(alloc, batch, block_size: int = 16, max_members: int = 8) -> tuple[int, int]:
    """K/V tokens one decode step over `batch` reads: every sequence its whole context, and with
    the batch cut into groups of consecutive sequences that read their shared full blocks once
    (at most `max_members` per group: 32 query columns over the query heads of one KV head)."""
    lens = [alloc.seq_len(s) for s in batch]
    width = max(1, max(-(-n // block_size) for n in lens))
    tables, lens = alloc.build_batch(batch, width)
    groups = shared_prefixes(np.asarray(tables, np.int32), np.asarray(lens, np.int32), max_members,
                             block_size=block_size)
    total = int(np.sum(lens))
    repeated = sum((m - 1) * block_size * k for _, m, k in groups.tolist())
    return total, total - repeated


def shared_prompt_footprint(prompt_len: int, suffix_lens, block_size: int = 16, seed: int = 0,
                            alloc_factory=None) -> dict:
    """Requests that share one system prompt of `prompt_len` tokens, each followed by its own
    suffix: through a PrefixIndex (one holder, every request forks from it) and without."""
    suffix_lens = [int(x) for x in suffix_lens]
    prompt = np.random.default_rng(seed).integers(0, 32000, size=prompt_len)
    need = -(-prompt_len // block_size) + sum(-(-(prompt_len + s) // block_size) for s in suffix_lens)
    alloc = (alloc_factory or BlockAllocator)(need + 1, block_size)
    index = PrefixIndex(alloc, first_id=len(suffix_lens))
    for r, s in enumerate(suffix_lens):
        alloc.fork(index.holder(prompt), r)
        if s:
            alloc.append(r, s)
    shared = alloc.num_blocks - alloc.num_free()
    unshared = sum(-(-(prompt_len + s) // block_size) for s in suffix_lens)
    total, grouped = step_read_tokens(alloc, list(range(len(suffix_lens))), block_size)
    return {"requests": len(suffix_lens), "prompt_len": prompt_len, "blocks": shared,
            "blocks_without_sharing": unshared, "saved_frac": round(1.0 - shared / unshared, 4),
            "read_tokens": total, "read_tokens_grouped": grouped, "read_saved_frac": round(1.0 - grouped / total, 4)}


def max_batch(budget_slots: int, lens, block_size: int, reserve: int) -> dict:
    """Requests (taken in order) that fit in `budget_slots` token slots, paged and contiguous."""
    used, paged = 0, 0
    for n in lens:
        b = -(-int(n) // block_size) * block_size
        if used + b > budget_slots:
            break
        used += b
        paged += 1
    contiguous = min(len(lens), budget_slots // reserve)
    return {"budget_slots": budget_slots, "paged": paged, "contiguous": contiguous,
            "ratio": round(paged / contiguous, 3) if contiguous else None}


def _summary(slots: int, tokens: int, **extra) -> dict:
    out = {"slots": slots, "tokens": tokens, "waste_frac": round(1.0 - tokens / slots, 4) if slots else 0.0}
    out.update(extra)
    return out


def study() -> list[dict]:
    """The decode workloads' length distributions (seeded, as in the tests and the bench)."""
    import synth

    rows = []
    for cfg, reserve in ((synth.C2, 2048), (synth.C3, 8192), (synth.C5, 131072)):
        lens = synth.context_lens(cfg).tolist()
        paged = paged_footprint(lens)
        contiguous = contiguous_footprint(lens, reserve)
        # a budget that holds the whole batch under max-length reservation, and a tenth of it
        batch = [max_batch(len(lens) * reserve // k, _repeat(lens, 64), 16, reserve) for k in (1, 10)]
        rows.append({"workload": cfg.name, "sequences": len(lens), "reserve_tokens": reserve,
                     "mean_tokens": round(float(np.mean(lens)), 1), "paged": paged, "contiguous": contiguous,
                     "max_batch": batch})
    c4 = synth.C4
    rows.append({"workload": c4.name, "prompts": c4.num_prompts, "samples": c4.samples,
                 "paged_after_all_steps": sampling_footprint(c4.num_prompts, c4.samples, c4.prefix_len, c4.steps)})
    for width, prompt, steps in ((4, 512, 256), (8, 1000, 200)):
        for skew in (0.0, 1.5):
            rows.append({"workload": "beam_search", **beam_search_footprint(width, prompt, steps, skew=skew)})
    suffixes = np.random.default_rng(7).integers(16, 512, size=256).tolist()
    rows.append({"workload": "shared_system_prompt", **shared_prompt_footprint(2000, suffixes)})
    return rows


def _repeat(lens, times):
    """The length distribution drawn again and again: a queue of requests to admit."""
    return [n for _ in range(times) for n in lens]


if __name__ == "__main__":
    for row in study():
        print(json.dumps(row))

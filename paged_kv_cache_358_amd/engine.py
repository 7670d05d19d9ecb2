"""One decode layer driven end to end: allocator step -> copies -> appends -> attention.

Host orchestration only; all device work is the library's kernels.  Per decode
step the C++ allocator appends one token to each sequence (opening blocks as
they fill, copy-on-write for shared partial blocks: "Stop Wasting GPU Memory"
page, Technical Details, "Single Sequence Generation" and "Copy-on-Write for
Parallel Sampling"), its slot mapping, copy pairs and block tables are staged in
pinned host memory and copied to the device on the compute stream, then
``block_copy`` -> ``kv_append`` -> ``paged_attention_decode`` run on that stream
in that order.  (The kernels could read the pinned buffer in place, but the
attention kernel then fetches its lengths and tables over the bus: measured on
MI355X the step time was the same and the attention kernel 1-3% slower, so the
metadata is copied, in the same launch as the append.)  Nothing in a step waits for the device, except when a pinned
staging buffer is about to be reused while its previous copy is still pending.

Forked sequences keep the blocks they inherited until they write into one, so
consecutive samples or beams of one prompt share their leading blocks; each step
groups them (``shared_prefixes``) and the attention call reads a group's shared
blocks once for all members.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import (PA_MAX_GROUPED_SEQS, PA_OK, BlockAllocator, DecodeParams, PagedAttnError, SharedPrefix, _P32, _P64,
               alloc_kv_cache, block_copy, cache_desc, kv_append, lib, paged_attention_workspace_bytes, stage_copy,
               torch_dtype_code)


def group_batches(groups: np.ndarray, num_seqs: int, limit: int = PA_MAX_GROUPED_SEQS):
    """Cut a batch whose groups (rows [first, members, shared blocks], consecutive and covering
    sequences 0 .. num_seqs - 1 in order) are read through one description into runs of whole
    groups of at most ``limit`` sequences: [(s0, s1, g0, g1)], sequences s0 .. s1 - 1 and groups
    g0 .. g1 - 1 of each run.  Every group holds at most ``limit`` members."""
    ng = len(groups)
    if ng == 0 or num_seqs <= limit:
        return [(0, num_seqs, 0, ng)]
    ends = groups[:, 0].astype(np.int64) + groups[:, 1]
    runs = []
    s0 = g0 = 0
    while g0 < ng:
        # the last group that ends within limit sequences of s0 (at least the first: members <= limit)
        g1 = max(g0 + 1, int(np.searchsorted(ends, s0 + limit, side="right")))
        s1 = int(groups[g1, 0]) if g1 < ng else num_seqs
        runs.append((s0, s1, g0, g1))
        s0, g0 = s1, g1
    return runs


class _Staging:
    """One pinned host buffer and one device buffer holding a step's metadata, int32:
    context lengths [max_seqs] | slots [max_tokens] | copy pairs [max_seqs, 2] | groups of
    sequences sharing leading blocks [max_seqs, 3] | block tables [max_seqs, max_blocks].
    A step moves the used prefix in one host->device copy."""

    def __init__(self, max_seqs: int, max_blocks: int, max_tokens: int, device):
        self.o_lens = 0
        self.o_slots = max_seqs
        self.o_pairs = self.o_slots + max_tokens
        self.o_groups = self.o_pairs + 2 * max_seqs
        self.o_tables = self.o_groups + 3 * max_seqs
        total = (self.o_tables + max_seqs * max_blocks + 3) // 4 * 4
        self.max_blocks = max_blocks
        self.host = torch.empty(total, dtype=torch.int32, pin_memory=True)
        self.dev = torch.empty(total, dtype=torch.int32, device=device)
        h = self.host.numpy()
        self.h_lens = h[self.o_lens:self.o_slots]
        self.h_slots = h[self.o_slots:self.o_pairs]
        self.h_pairs = h[self.o_pairs:self.o_groups].reshape(max_seqs, 2)
        self.h_groups = h[self.o_groups:self.o_tables].reshape(max_seqs, 3)
        self.h_tables = h[self.o_tables:].reshape(max_seqs, max_blocks)
        self.host_ptr = self.host.data_ptr()
        self.dev_ptr = self.dev.data_ptr()
        # ctypes views of the host regions for the allocator calls
        self.c_slots = self.h_slots.ctypes.data_as(_P32)
        self.c_pairs = self.h_pairs.ctypes.data_as(_P32)
        self.c_groups = self.h_groups.ctypes.data_as(_P32)
        self.c_tables = self.h_tables.ctypes.data_as(_P32)
        self.c_lens = self.h_lens.ctypes.data_as(_P32)
        self.done = None  # event that ends the step that last read this buffer
        self.own_done = torch.cuda.Event()
        self.own_done.record()  # create it now: kernel launches can only mark existing events

    def d_slots(self, n):
        return self.dev[self.o_slots:self.o_slots + n]

    def d_pairs(self, n):
        return self.dev[self.o_pairs:self.o_pairs + 2 * n].view(n, 2)



class PagedDecodeLayer:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, num_q_heads: int, dtype,
                 max_seqs: int, max_blocks_per_seq: int, free_order=None, partition_size: int = 512,
                 device="cuda", stream=None, share_prefixes: bool = True, share_min_blocks: int = 4,
                 block_size: int = 16):
        self.block_size = block_size
        self.alloc = BlockAllocator(num_blocks, block_size, free_order)
        self.k_cache, self.v_cache = alloc_kv_cache(num_blocks, num_kv_heads, head_dim, dtype, device,
                                                    block_size=block_size)
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.dtype = dtype
        self.max_seqs = max_seqs
        self.max_blocks = max_blocks_per_seq
        self.partition_size = partition_size
        # Shared leading blocks are read once per group when at least share_min_blocks are shared.
        self.share_prefixes = share_prefixes
        self.share_min_blocks = share_min_blocks
        self.share_max_members = 32 // (num_q_heads // num_kv_heads)  # two 16-column tiles of query heads
        self.device = device
        self.stream = torch.cuda.current_stream() if stream is None else stream
        # Three staging buffers: the host fills one while the stream may still read the two
        # before it, so host work on a step overlaps the GPU's previous steps.
        self._stage = [_Staging(max_seqs, max_blocks_per_seq, max_seqs, device) for _ in range(3)]
        self._turn = 0
        self._ones = np.ones(max_seqs, np.int32)
        self._c_ones = self._ones.ctypes.data_as(_P32)
        self._npairs = ctypes.c_int32(0)
        self._ngroups = ctypes.c_int32(0)
        # Sized for a whole batch and, with sharing, for a run of PA_MAX_GROUPED_SEQS grouped sequences
        # (a larger grouped batch is read in such runs).
        ws = 16
        for n in {max_seqs, min(max_seqs, PA_MAX_GROUPED_SEQS)}:
            probe_q = torch.empty(n, num_q_heads, head_dim, dtype=dtype, device=device)
            probe_t = torch.empty(n, max_blocks_per_seq, dtype=torch.int32, device=device)
            ws = max(ws, paged_attention_workspace_bytes(probe_q, self.k_cache, self.v_cache, probe_t,
                                                         torch.empty_like(probe_q, dtype=torch.float32),
                                                         max_blocks_per_seq * block_size, partition_size,
                                                         shared=share_prefixes))
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        # The per-step library calls go straight to the C ABI with argument blocks built here once:
        # the layer owns the caches, staging buffers and workspace, so only the step's tensors,
        # sizes and events change between calls.
        self._cdesc = cache_desc(self.k_cache, self.v_cache)
        self._k_ptr = self.k_cache.data_ptr()
        self._v_ptr = self.v_cache.data_ptr()
        self._stream_ptr = self.stream.cuda_stream
        self._shared = SharedPrefix(None, 0)
        self._params = DecodeParams(0, num_q_heads, max_blocks_per_seq, 0, partition_size, 0, self._cdesc,
                                    self.workspace.data_ptr(), self.workspace.numel(), self._stream_ptr, None, None,
                                    None)

    # ------------------------------------------------------------------ sequence management
    def add(self, seq: int):
        self.alloc.add(seq)

    def fork(self, parent: int, child: int):
        self.alloc.fork(parent, child)

    def free(self, seq: int):
        self.alloc.free(seq)

    def prefill(self, seq: int, k, v):
        """Place a prompt's K/V [n, H_kv, D] (device tensors) into the cache."""
        n = k.shape[0]
        slots, pairs = self.alloc.append(seq, n)
        with torch.cuda.stream(self.stream):
            if len(pairs):
                block_copy(self.k_cache, self.v_cache, torch.from_numpy(pairs).to(self.device), stream=self.stream)
            kv_append(k, v, torch.from_numpy(slots).to(self.device), self.k_cache, self.v_cache, stream=self.stream)

    # ------------------------------------------------------------------ one decode step
    def decode_step(self, seqs, q, k_new, v_new, out, scale: float, timing=None):
        """Each of ``seqs`` (sequence ids: a list, or an int64 array, which is used without a copy)
        appends one token (k_new/v_new [S, H_kv, D]) and attends
        with q [S, H_q, D] over its whole context; writes out [S, H_q, D].

        ``timing`` = (start, end) timing-enabled torch.cuda.Events (already recorded once)
        mark the start and end of the attention call's kernels.  No event is recorded
        between kernels (a marker packet delays the stream by microseconds): the events
        travel with the attention launch, and the end event also tells the host when the
        staging buffer may be rewritten.  Returns the number of copy-on-write block copies."""
        S = len(seqs)
        hq, hkv, D = self.num_q_heads, self.num_kv_heads, self.head_dim
        for t, shape in ((q, (S, hq, D)), (out, (S, hq, D)), (k_new, (S, hkv, D)), (v_new, (S, hkv, D))):
            if tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"decode_step: expected a contiguous device tensor of shape {shape}")
        if q.dtype != self.dtype or k_new.dtype != self.dtype or v_new.dtype != self.dtype:
            raise ValueError("decode_step: q, k_new and v_new must have the cache dtype")
        st = self._stage[self._turn]
        self._turn = (self._turn + 1) % len(self._stage)
        if st.done is not None:
            st.done.synchronize()  # previous copies out of this pinned buffer have finished
        if S > self.max_seqs:
            raise ValueError("decode_step: more sequences than the layer was sized for")
        ids = np.ascontiguousarray(seqs, dtype=np.int64)  # no copy for a contiguous int64 array
        c_ids = ids.ctypes.data_as(_P64)
        # The allocator's step, straight through the C ABI into the staging buffer: one token per
        # sequence (slots, copy-on-write pairs), the block tables and lengths, and the groups of
        # sequences that share leading blocks.
        rc = lib.pa_seq_append_batch(self.alloc._h, c_ids, S, self._c_ones, st.c_slots, st.c_pairs, self.max_seqs,
                                     ctypes.byref(self._npairs))
        if rc != PA_OK:
            raise PagedAttnError(rc, "pa_seq_append_batch")
        rc = lib.pa_build_batch(self.alloc._h, c_ids, S, self.max_blocks, st.c_tables, st.c_lens)
        if rc != PA_OK:
            raise PagedAttnError(rc, "pa_build_batch")
        np_tables, np_lens = st.h_tables[:S], st.h_lens[:S]
        max_ctx = int(np_lens.max()) if S else 0
        npairs = self._npairs.value
        ngroups = 0  # groups covering the batch; 0 when no two sequences share a block
        if self.share_prefixes and S >= 2 and self.share_max_members >= 2:
            rc = lib.pa_shared_prefixes(st.c_tables, st.c_lens, S, self.max_blocks, self.block_size, self.share_max_members,
                                        self.share_min_blocks, st.c_groups, self.max_seqs, ctypes.byref(self._ngroups))
            if rc != PA_OK:
                raise PagedAttnError(rc, "pa_shared_prefixes")
            ngroups = self._ngroups.value if self._ngroups.value < S else 0
        group_rows = st.h_groups[:ngroups].copy() if ngroups else None
        # A grouped batch of more than PA_MAX_GROUPED_SEQS sequences goes to the library in runs of whole
        # groups, each description counting its first sequences from the run's first.
        runs = group_batches(st.h_groups[:ngroups], S) if ngroups else [(0, S, 0, 0)]
        for s0, _, g0, g1 in runs[1:]:
            st.h_groups[g0:g1, 0] -= s0
        used = st.o_tables + S * self.max_blocks  # lengths, slots, pairs, sharing and the first S table rows
        if npairs:
            # copy-on-write blocks are copied before the append writes into them
            stage_copy(st.dev, st.host, used * 4, stream=self.stream)
            block_copy(self.k_cache, self.v_cache, st.d_pairs(npairs), stream=self.stream)
            kv_append(k_new, v_new, st.d_slots(S), self.k_cache, self.v_cache, stream=self.stream)
        else:
            # one launch: the metadata copy, and the append reading its slots from the staging buffer
            rc = lib.pa_stage_append(st.dev_ptr, st.host_ptr, used * 4, k_new.data_ptr(), v_new.data_ptr(),
                                     st.host_ptr + 4 * st.o_slots, S, self._k_ptr, self._v_ptr,
                                     ctypes.byref(self._cdesc), self._stream_ptr)
            if rc != PA_OK:
                raise PagedAttnError(rc, "pa_stage_append")
        # the staging copies (earlier in the stream) are done when the attention kernels are
        st.done = st.own_done if timing is None else timing[1]
        p = self._params
        p.max_context_len = max_ctx
        p.out_dtype = torch_dtype_code(out.dtype)
        q_row = hq * D * q.element_size()
        out_row = hq * D * out.element_size()
        for i, (s0, s1, g0, g1) in enumerate(runs):
            p.num_seqs = s1 - s0
            # the start event on the first call, the end event on the last
            p.start_event = None if timing is None or i > 0 else timing[0].cuda_event
            p.stop_event = st.done.cuda_event if i == len(runs) - 1 else None
            if g1 > g0:
                self._shared.groups = st.dev_ptr + 4 * (st.o_groups + 3 * g0)
                self._shared.num_groups = g1 - g0
                p.shared = ctypes.pointer(self._shared)
            else:
                p.shared = None
            rc = lib.paged_attention_decode(q.data_ptr() + s0 * q_row, self._k_ptr, self._v_ptr,
                                            st.dev_ptr + 4 * (st.o_tables + s0 * self.max_blocks),
                                            st.dev_ptr + 4 * (st.o_lens + s0), float(scale),
                                            out.data_ptr() + s0 * out_row, ctypes.byref(p))
            if rc != PA_OK:
                raise PagedAttnError(rc, "paged_attention_decode")
        self.last_runs = runs
        self.last_groups = ngroups
        self.last_group_rows = group_rows
        self.last_lens = np_lens.copy()
        self.last_tables = np_tables  # view into the pinned staging buffer: valid until three steps later
        return npairs

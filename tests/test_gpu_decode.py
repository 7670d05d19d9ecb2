"""Paged decode attention on the GPU against the fp64 oracle.

Tolerance (max abs error, fp32 output): 1e-5 for fp32 inputs, 5e-3 for bf16/fp16
inputs with fp32 accumulation.  Pool memory the kernels must not read (free
blocks, a foreign sequence's blocks, slots past each context) holds NaN.
"""
import math

import numpy as np
import pytest
import torch

import synth
from paged_setup import PagedDecode, bound_16bit, check_16bit_output, tol_for

pytestmark = pytest.mark.gpu


def max_err(out: torch.Tensor, pd: PagedDecode, seqs=None, heads=None):
    o = out.float().cpu().numpy()
    worst = 0.0
    for s in (range(pd.cfg.num_seqs) if seqs is None else seqs):
        hs = list(range(pd.cfg.num_q_heads)) if heads is None else heads
        ref = pd.oracle(s, hs)
        assert np.all(np.isfinite(o[s, hs]))
        worst = max(worst, float(np.max(np.abs(o[s, hs] - ref))))
    return worst


def test_c1_tiny_fp32_all_outputs():
    pd = PagedDecode(synth.C1)
    out = pd.run()
    assert max_err(out, pd) <= 1e-5
    # context of one token: the output is that token's V, bit for bit
    k, v = pd.truth[0]
    assert np.array_equal(out[0].cpu().numpy(), v[0])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_single_token_context_is_exact(dtype):
    cfg = synth.scaled(synth.C3, lens=[1, 1, 17, 1], dtype=dtype)
    pd = PagedDecode(cfg)
    out = pd.run().cpu().numpy()
    for s in (0, 1, 3):
        _, v = pd.truth[s]
        expect = synth.decode_f64(v[0], dtype).astype(np.float32)     # [H_kv, D]
        assert np.array_equal(out[s], np.repeat(expect, cfg.group, axis=0))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mha_ragged(dtype):
    # MHA head layout of the 64-sequence workload; lengths span partial blocks,
    # partition edges and several partitions.
    lens = [1, 2, 15, 16, 17, 31, 33, 128, 500, 511, 512, 513, 1024, 1500, 2048, 2047]
    cfg = synth.scaled(synth.C2, lens=lens, dtype=dtype)
    pd = PagedDecode(cfg)
    out = pd.run()
    assert max_err(out, pd) <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gqa_fragmented_pool(dtype):
    cfg = synth.scaled(synth.C3, num_seqs=24, dtype=dtype, lens_args=(300.0, 1.0, 16, 3000))
    pd = PagedDecode(cfg)
    assert pd.alloc.num_free() < pd.num_blocks * 0.75          # foreign sequence holds ~30%
    out = pd.run()
    assert max_err(out, pd) <= tol_for(dtype)


def test_head_dim_64_and_group_4():
    cfg = synth.DecodeConfig("d64_g4", 31, 6, 16, 4, 64, "bf16", "fixed", (1, 40, 700, 16, 1025, 64))
    pd = PagedDecode(cfg)
    out = pd.run()
    assert max_err(out, pd) <= 5e-3


def test_generic_path_shapes():
    # group 48 (> 32 query heads per KV head), fp32 head_dim 256 and head_dim 256 on 48-token blocks
    # take the VALU kernel
    for cfg in (synth.DecodeConfig("g48", 32, 3, 48, 1, 128, "bf16", "fixed", (5, 600, 1100)),
                synth.DecodeConfig("d256_f32", 33, 3, 4, 2, 256, "f32", "fixed", (7, 530, 40)),
                synth.DecodeConfig("d256_b48", 33, 3, 4, 2, 256, "bf16", "fixed", (7, 530, 40), block_size=48,
                                   partition_size=480),
                synth.DecodeConfig("f32_gqa", 34, 3, 8, 2, 64, "f32", "fixed", (3, 1030, 48))):
        pd = PagedDecode(cfg)
        out = pd.run()
        assert max_err(out, pd) <= tol_for(cfg.dtype), cfg.name


@pytest.mark.parametrize("hq,hkv,D,dtype,B", [(32, 1, 128, "bf16", 16), (24, 1, 64, "f16", 16), (17, 1, 128, "bf16", 8),
                                                (64, 2, 128, "f16", 32), (32, 1, 64, "bf16", 64)])
def test_more_than_16_query_heads_per_kv_head(hq, hkv, D, dtype, B):
    # 17 to 32 query heads per KV head run on the split kernel's two 16-column tiles, each sequence a group
    # of its own: ragged, block-edge and multi-partition contexts against the oracle, and a 16-bit output
    # that is the fp32 result rounded once.
    lens = (1, B - 1, B + 1, 511, 1030, 2100)
    cfg = synth.DecodeConfig(f"g{hq // hkv}", 50 + hq, len(lens), hq, hkv, D, dtype, "fixed", lens, block_size=B)
    pd = PagedDecode(cfg)
    import paged_kv_cache_358_amd as pa
    kernel = pa.paged_attention_decode_kernel(pd.q, pd.k_cache, pd.v_cache, pd.block_tables,
                                              torch.empty(pd.q.shape, dtype=torch.float32, device="cuda"),
                                              pd.max_context_len, pd.cfg.partition_size)
    assert kernel == "decode_split_kernel"
    out = pd.run()
    assert max_err(out, pd) <= tol_for(dtype)
    o16 = pd.run(out_dtype=pd.q.dtype).float().cpu().numpy()
    check_16bit_output(o16, out.cpu().numpy(), dtype)


@pytest.mark.parametrize("part", [16, 64, 256, 512, 1024])
def test_partition_size_does_not_change_the_result(part):
    cfg = synth.scaled(synth.C3, lens=[16, 100, 1024, 3000, 4097], num_seqs=None)
    pd = PagedDecode(cfg)
    out = pd.run(partition_size=part)
    assert max_err(out, pd) <= 5e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_physical_block_permutation_is_bitwise_invisible(dtype):
    base = synth.scaled(synth.C3, lens=[5, 77, 600, 1500], dtype=dtype)
    a = PagedDecode(base)
    n = a.num_blocks
    b = PagedDecode(base, free_order=np.random.default_rng(99).permutation(n))
    assert not np.array_equal(a.tables_np, b.tables_np)
    oa, ob = a.run(), b.run()
    assert torch.equal(oa, ob)


def test_empty_context_gives_zero():
    cfg = synth.scaled(synth.C3, lens=[0, 20, 0])
    pd = PagedDecode(cfg)
    out = pd.run().cpu().numpy()
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.max(np.abs(out[1] - pd.oracle(1))) <= 5e-3


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_16bit_output(dtype):
    cfg = synth.scaled(synth.C3, lens=[3, 333, 2222], dtype=dtype)
    pd = PagedDecode(cfg)
    out = pd.run(out_dtype=torch.bfloat16 if dtype == "bf16" else torch.float16).float().cpu().numpy()
    check_16bit_output(out, pd.run().cpu().numpy(), dtype)   # the fp32 result rounded once
    for s in range(3):
        ref = pd.oracle(s)
        assert np.all(np.abs(out[s] - ref) <= bound_16bit(ref, dtype))


def test_tables_past_context_are_never_read():
    # Garbage (out-of-range ids) in table entries past each context must not matter.
    cfg = synth.scaled(synth.C3, lens=[20, 300, 1])
    pd = PagedDecode(cfg)
    ref = pd.run()
    t = pd.tables_np.copy()
    for s, n in enumerate(pd.lens):
        t[s, -(-int(n) // 16):] = 2 ** 30
    out = pd.run(block_tables=torch.from_numpy(t).cuda())
    assert torch.equal(ref, out)


# ----------------------------------------------------------------- full-size workloads
# The workloads at the sizes the bench times.  Every sequence is checked against the fp64 oracle
# (each drawn alone, one KV head at a time), on two query heads of different KV heads for the MHA
# and GQA workloads and on every query head of every sequence for the long-context workload; every
# output of the batch must be finite.
def _full_check(cfg, heads_of):
    pd = PagedDecode(cfg, keep_truth=False)
    out = pd.run().cpu().numpy()
    assert np.all(np.isfinite(out))
    worst = 0.0
    for s in range(cfg.num_seqs):
        heads = heads_of(s)
        ref = pd.oracle_rows(s, heads)
        worst = max(worst, float(np.max(np.abs(out[s, heads] - ref))))
    assert worst <= tol_for(cfg.dtype), worst
    return pd


def test_full_c2_mha_every_sequence():
    _full_check(synth.C2, lambda s: [s % 32, (s + 16) % 32])


def test_full_c3_gqa_every_sequence():
    pd = _full_check(synth.C3, lambda s: [s % 64, (s + 36) % 64])
    assert pd.lens.max() > 4096


def test_full_c5_long_context_every_row():
    _full_check(synth.C5, lambda s: list(range(64)))


# ----------------------------------------------------------------- scheduling paths of the MFMA kernels
def test_more_sequences_than_the_persistent_index_covers():
    # 2100 sequences (> 2048) at head_dim 64 on 16-token blocks, contexts up to 700 tokens.  With
    # 1024-token partitions every context is one partition and the batch takes the per-partition
    # MFMA kernel (one workgroup per sequence and KV head, no merge); with 256-token partitions the
    # split kernel runs once per slice of 2048 sequences.
    import paged_kv_cache_358_amd as pa
    lens = np.random.default_rng(11).integers(1, 700, size=2100)
    cfg = synth.DecodeConfig("many_seqs", 41, 2100, 8, 2, 64, "bf16", "fixed", tuple(int(x) for x in lens),
                             partition_size=1024)
    pd = PagedDecode(cfg)
    picks = sorted(set(np.random.default_rng(12).choice(cfg.num_seqs, size=60, replace=False).tolist())
                   | {0, 2047, 2048, 2099})
    for part, kernel in ((1024, "decode_mfma_kernel"), (256, "decode_split_kernel")):
        out = torch.empty(pd.q.shape, dtype=torch.float32, device="cuda")
        assert pa.paged_attention_decode_kernel(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, out,
                                                pd.max_context_len, part) == kernel
        out = pd.run(partition_size=part)
        assert torch.isfinite(out).all()
        assert max_err(out, pd, seqs=picks) <= 5e-3, part


def test_per_partition_mfma_kernel_with_merges():
    # A block table so wide that the split kernel's int32 tile index could overflow (2049 sequences
    # x 8 KV heads x 131072 entries) sends the batch to the per-partition MFMA kernel even with
    # contexts over several partitions: partials and the merge kernel.  Table entries past each
    # context are zero, and never read.
    import paged_kv_cache_358_amd as pa
    lens = np.random.default_rng(15).integers(1, 40, size=2049)
    lens[[0, 1, 2, 1000, 2048]] = [1500, 512, 513, 1100, 2000]
    cfg = synth.DecodeConfig("wide_table", 46, 2049, 32, 8, 128, "bf16", "fixed", tuple(int(x) for x in lens))
    pd = PagedDecode(cfg, keep_truth=False)
    wide = torch.zeros(cfg.num_seqs, 131072, dtype=torch.int32, device="cuda")
    wide[:, :pd.block_tables.shape[1]] = pd.block_tables
    out = torch.empty(pd.q.shape, dtype=torch.float32, device="cuda")
    assert pa.paged_attention_decode_kernel(pd.q, pd.k_cache, pd.v_cache, wide, out, pd.max_context_len,
                                            512) == "decode_mfma_kernel"
    out = pd.run(block_tables=wide).cpu().numpy()
    heads = [0, 13, 31]
    for s in (0, 1, 2, 1000, 2048):
        assert np.max(np.abs(out[s, heads] - pd.oracle_sampled(s, heads))) <= 5e-3, s
    del wide
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,B,D,hq,hkv", [
    ("bf16", 32, 128, 8, 2),   # 32-token blocks
    ("f16", 8, 64, 8, 2),      # 8-token blocks, two to a 16-token tile
    ("bf16", 16, 96, 8, 2),    # head_dim 96
    ("bf16", 16, 128, 32, 1),  # 32 query heads per KV head: groups of one sequence
    ("f16", 32, 256, 4, 1),    # head_dim 256
])
def test_more_sequences_than_one_split_launch_covers(dtype, B, D, hq, hkv):
    # 4500 sequences on shapes the per-partition MFMA kernel does not take: the split kernel runs
    # once per slice of 2048 sequences (2048, 2048, 404), each on its own rows of q, out, the
    # tables and the lengths.  Sequences at the slice edges, empty ones, one longer than a
    # partition, and random picks from every slice.
    rng = np.random.default_rng(14)
    lens = rng.integers(1, 300, size=4500)
    edges = {0: 1, 2047: 299, 2048: 700, 2049: 0, 4095: 17, 4096: 513, 4499: 64}
    for s, n in edges.items():
        lens[s] = n
    cfg = synth.DecodeConfig("many_seqs_split", 44, 4500, hq, hkv, D, dtype, "fixed",
                             tuple(int(x) for x in lens), block_size=B)
    pd = PagedDecode(cfg, keep_truth=False)
    out = pd.run()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    assert np.all(o[2049] == 0)
    picks = sorted(set(rng.choice(cfg.num_seqs, size=36, replace=False).tolist()) | set(edges) - {2049})
    heads = [0, hq // 2, hq - 1]
    for s in picks:
        if lens[s] == 0:
            assert np.all(o[s] == 0)
            continue
        ref = pd.oracle_sampled(s, heads)
        assert np.max(np.abs(o[s, heads] - ref)) <= tol_for(dtype), s
    # a call with another partition size over the same cache reuses the workspace with new tags
    o2 = pd.run(partition_size=4 * B).cpu().numpy()
    for s in (2047, 2048, 4096):
        assert np.max(np.abs(o2[s, heads] - pd.oracle_sampled(s, heads))) <= tol_for(dtype), s


def test_mixed_empty_short_and_long_contexts():
    # Zero-length, one-token, partial-block and multi-partition contexts side by side:
    # the persistent split cuts runs inside long contexts and the merge recombines them.
    rng = np.random.default_rng(13)
    lens = [0, 1, 17, 5000, 0, 2, 3000, 16, 700, 4097] + rng.integers(1, 300, size=50).tolist()
    cfg = synth.scaled(synth.C3, lens=lens)
    pd = PagedDecode(cfg)
    out = pd.run()
    o = out.cpu().numpy()
    assert np.all(o[0] == 0) and np.all(o[4] == 0)
    assert max_err(out, pd, seqs=[s for s in range(cfg.num_seqs) if lens[s] > 0]) <= 5e-3


def test_fewer_blocks_than_workgroups():
    # A few blocks in all: most workgroups of the persistent grid own no partition.
    cfg = synth.DecodeConfig("tiny_bf16", 42, 2, 4, 4, 128, "bf16", "fixed", (3, 40))
    pd = PagedDecode(cfg)
    out = pd.run()
    assert max_err(out, pd) <= 5e-3


@pytest.mark.parametrize("part", [16, 128])
def test_long_context_small_partitions(part):
    # Many partitions per context: runs hold several partitions merged on chip.
    cfg = synth.scaled(synth.C5, lens=[20000, 7777], partition_size=part)
    pd = PagedDecode(cfg, keep_truth=False)
    out = pd.run().cpu().numpy()
    for s in range(2):
        heads = [0, 9, 63]
        ref = pd.oracle_sampled(s, heads)
        assert np.max(np.abs(out[s, heads] - ref)) <= 5e-3


def test_workspace_shared_by_calls_with_other_queries_and_partitions():
    # The split kernel's per-context arrival counters live in the workspace and are never
    # cleared: each call tags them.  Calls with other queries and partition sizes reuse one
    # workspace that starts as garbage; every call must match the oracle.
    from paged_setup import to_torch
    import paged_kv_cache_358_amd as pa
    cfg = synth.scaled(synth.C5, lens=[9000, 3000, 0, 5000], partition_size=32)
    pd = PagedDecode(cfg, keep_truth=False)
    out = torch.empty(pd.q.shape, dtype=torch.float32, device=pd.q.device)
    need = pa.paged_attention_workspace_bytes(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, out,
                                              pd.max_context_len, 32)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=pd.q.device)
    heads = [0, 13, 63]
    for step, part in enumerate([32, 512, 32, 16 * 7]):
        pd.q_np = synth.queries(cfg, step=step + 1)
        pd.q = to_torch(pd.q_np, cfg.dtype, pd.q.device)
        pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens,
                                  cfg.softmax_scale, out, max_context_len=pd.max_context_len,
                                  partition_size=part, workspace=ws)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(o[2] == 0)
        for s in (0, 1, 3):
            ref = pd.oracle_sampled(s, heads)
            assert np.max(np.abs(o[s, heads] - ref)) <= 5e-3, (step, part, s)


@pytest.mark.parametrize("part", [512, 16])
def test_start_and_stop_events_bracket_the_kernels(part):
    # The events travel with the launches; the per-partition path (more sequences than the
    # split kernel indexes) ends with the merge kernel, which carries the stop event.
    import paged_kv_cache_358_amd as pa
    # fp32 beyond 2048 sequences: the per-partition VALU kernel and the merge kernel
    many = synth.DecodeConfig("many_seqs_ev", 43, 2050, 8, 2, 64, "f32", "fixed", (40, 600) * 1025)
    # 32-token blocks beyond 2048 sequences: two launches of the split kernel, the start event on
    # the first and the stop event on the second
    sliced = synth.DecodeConfig("many_seqs_ev32", 45, 2050, 8, 2, 64, "bf16", "fixed", (40, 600) * 1025,
                                block_size=32)
    for cfg in (synth.scaled(synth.C2, lens=[700, 33, 2048]), many, sliced):
        pd = PagedDecode(cfg, keep_truth=False)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        stop.record()
        out = torch.empty(pd.q.shape, dtype=torch.float32, device=pd.q.device)
        pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens,
                                  cfg.softmax_scale, out, max_context_len=pd.max_context_len,
                                  partition_size=max(part, cfg.block_size), start_event=start, stop_event=stop)
        stop.synchronize()
        ms = start.elapsed_time(stop)
        assert 0.0 < ms < 1000.0
        for s in (0, 1):
            ref = pd.oracle_sampled(s, [0, cfg.num_q_heads - 1])
            assert np.max(np.abs(out[s, [0, cfg.num_q_heads - 1]].cpu().numpy() - ref)) <= 5e-3
    # nothing to launch: both events are still recorded, in stream order
    empty = torch.empty(0, 4, 128, dtype=torch.bfloat16, device="cuda")
    kc, vc = pa.alloc_kv_cache(4, 4, 128, torch.bfloat16, "cuda")
    start.record()
    stop.record()
    pa.paged_attention_decode(empty, kc, vc, torch.zeros(0, 1, dtype=torch.int32, device="cuda"),
                              torch.zeros(0, dtype=torch.int32, device="cuda"), 0.1, empty.float(),
                              max_context_len=0, start_event=start, stop_event=stop)
    stop.synchronize()
    assert start.elapsed_time(stop) >= 0.0


@pytest.mark.parametrize("dtype,B", [("bf16", 8), ("bf16", 32), ("f32", 32), ("f16", 64), ("f32", 8)])
def test_other_block_sizes(dtype, B):
    # fp32 caches take the VALU kernel (and the partition merge); bf16/fp16 blocks of 8 tokens take
    # the split kernel two to a 16-token tile, and blocks of 32 and 64 tokens as 16-token tiles (a
    # partition of 4 * 8 = 32 tokens holds two tiles).  Lengths around the block size, several
    # blocks and several partitions.
    lens = [1, B - 1, B, B + 1, 2 * B + 3, 300, 1000]
    cfg = synth.scaled(synth.C3, lens=lens, dtype=dtype, block_size=B)
    pd = PagedDecode(cfg)
    assert pd.k_cache.shape[3] == B
    out = pd.run()
    assert max_err(out, pd) <= tol_for(dtype)
    out2 = pd.run(partition_size=4 * B)
    assert max_err(out2, pd) <= tol_for(dtype)


@pytest.mark.parametrize("base,dtype,B,D", [(synth.C3, "bf16", 32, 128), (synth.C2, "bf16", 64, 128),
                                           (synth.C3, "f16", 128, 64), (synth.C2, "f16", 32, 64)])
def test_multi_tile_blocks(base, dtype, B, D):
    # Blocks of 16 << j tokens go to the split kernel, which streams each as 16-token tiles:
    # contexts ending inside a block's first tile, on a tile edge inside a block, on a block edge,
    # and spanning several blocks and 512-token partitions.
    lens = [1, 15, 16, 17, B - 1, B, B + 1, B + 16, 3 * B + 5, 511, 512, 513, 1500, 2047]
    cfg = synth.scaled(base, lens=lens, dtype=dtype, block_size=B, head_dim=D)
    pd = PagedDecode(cfg)
    assert pd.k_cache.shape[3] == B
    assert max_err(pd.run(), pd) <= tol_for(dtype)
    # partitions of one block and of 1024 tokens; bf16 output
    assert max_err(pd.run(partition_size=B), pd) <= tol_for(dtype)
    assert max_err(pd.run(partition_size=1024), pd) <= tol_for(dtype)
    # 16-bit output: the fp32 result rounded once, and within 5e-3 plus half an output ulp of the oracle
    o16 = pd.run(out_dtype=pd.q.dtype).float().cpu().numpy()
    check_16bit_output(o16, pd.run().cpu().numpy(), dtype)
    for s in range(cfg.num_seqs):
        ref = pd.oracle(s)
        assert np.all(np.abs(o16[s] - ref) <= bound_16bit(ref, dtype)), s


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_multi_tile_blocks_match_16_token_blocks(dtype):
    # The split kernel computes the same 16-token tiles whatever the cache's block size; only the
    # order in which a workgroup's waves sum them changes (a wave takes all tiles of its block).  The
    # same sequences in caches of 16-, 32- and 64-token blocks agree to fp32 rounding.
    lens = [1, 16, 33, 200, 511, 512, 513, 777, 1024, 1500, 2047, 3000]
    outs = []
    for B in (16, 32, 64):
        pd = PagedDecode(synth.scaled(synth.C3, lens=lens, dtype=dtype, block_size=B))
        outs.append(pd.run().cpu().numpy())
    assert float(np.max(np.abs(outs[1] - outs[0]))) <= 1e-5
    assert float(np.max(np.abs(outs[2] - outs[0]))) <= 1e-5
    assert max_err(torch.from_numpy(outs[2]), pd) <= tol_for(dtype)


@pytest.mark.parametrize("base,dtype,D", [(synth.C3, "bf16", 128), (synth.C2, "f16", 128), (synth.C3, "f16", 64),
                                         (synth.C2, "bf16", 64)])
def test_eight_token_blocks(base, dtype, D):
    # Blocks of 8 tokens go to the split kernel, two to a 16-token tile: contexts ending inside a
    # tile's first block, on the block edge inside a tile, on a tile edge, and spanning several
    # 512-token partitions.  Partitions of one tile and of 1024 tokens; a partition of 8 tokens
    # (half a tile) takes the VALU kernel.
    import paged_kv_cache_358_amd as pa
    lens = [1, 7, 8, 9, 15, 16, 17, 23, 24, 25, 511, 512, 513, 1500, 2047]
    cfg = synth.scaled(base, lens=lens, dtype=dtype, block_size=8, head_dim=D)
    pd = PagedDecode(cfg)
    assert pd.k_cache.shape[3] == 8
    out = torch.empty(pd.q.shape, dtype=torch.float32, device="cuda")
    args = (pd.q, pd.k_cache, pd.v_cache, pd.block_tables, out, pd.max_context_len)
    assert pa.paged_attention_decode_kernel(*args) == "decode_split_kernel"
    assert pa.paged_attention_decode_kernel(*args, partition_size=8) == "decode_generic_kernel"
    for part in (None, 16, 1024, 8):
        assert max_err(pd.run(partition_size=part), pd) <= tol_for(dtype), part
    o16 = pd.run(out_dtype=pd.q.dtype).float().cpu().numpy()
    check_16bit_output(o16, pd.run().cpu().numpy(), dtype)
    for s in range(cfg.num_seqs):
        ref = pd.oracle(s)
        assert np.all(np.abs(o16[s] - ref) <= bound_16bit(ref, dtype)), s


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_eight_token_blocks_match_16_token_blocks(dtype):
    # Two 8-token blocks make the same 16-token tile as one 16-token block, and the waves take the
    # tiles in the same order: the same sequences in caches of 8- and 16-token blocks give the same
    # bits.
    lens = [1, 8, 16, 33, 200, 511, 512, 513, 777, 1024, 1500, 2047, 3000]
    outs = []
    for B in (16, 8):
        pd = PagedDecode(synth.scaled(synth.C3, lens=lens, dtype=dtype, block_size=B))
        outs.append(pd.run())
    assert torch.equal(outs[0], outs[1])


def test_eight_token_blocks_ignore_table_entries_past_the_context():
    # Past each context the table may hold anything, also in the second block of the context's last
    # tile; a context ending on a block edge inside a tile leaves that block unread.
    cfg = synth.scaled(synth.C3, lens=[8, 20, 300, 1, 24], block_size=8)
    pd = PagedDecode(cfg)
    ref = pd.run()
    t = pd.tables_np.copy()
    for s, n in enumerate(pd.lens):
        t[s, -(-int(n) // 8):] = 2 ** 30
    assert torch.equal(ref, pd.run(block_tables=torch.from_numpy(t).cuda()))
    t[:, :] = np.where(t == 2 ** 30, -1, t)
    assert torch.equal(ref, pd.run(block_tables=torch.from_numpy(t).cuda()))


@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 16, 4), ("f16", 8, 8), ("bf16", 32, 2)])
def test_head_dim_256_split_kernel(dtype, hq, hkv):
    # head_dim 256 on 16-token blocks: the split kernel, one wave per SIMD.  Lengths around block and
    # partition edges, several partitions; partitions of one block and of 1024 tokens; with a
    # shared-prefix description of groups sharing no blocks, the group mode gives the same attention.
    import paged_kv_cache_358_amd as pa
    lens = [1, 15, 16, 17, 300, 511, 512, 513, 1600, 2500]
    cfg = synth.DecodeConfig("d256_split", 35, len(lens), hq, hkv, 256, dtype, "fixed", tuple(lens))
    pd = PagedDecode(cfg)
    out = pd.run()
    assert max_err(out, pd) <= tol_for(dtype)
    for part in (16, 1024):
        assert max_err(pd.run(partition_size=part), pd) <= tol_for(dtype)
    # groups of consecutive sequences, at most 32 / g members each (the description's limit)
    m = min(4, 32 // (hq // hkv))
    sh = torch.tensor([[f, min(m, len(lens) - f), 0] for f in range(0, len(lens), m)], dtype=torch.int32,
                      device="cuda")
    o2 = torch.empty_like(out)
    pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens,
                              cfg.softmax_scale, o2, max_context_len=pd.max_context_len, shared=sh)
    torch.cuda.synchronize()
    assert max_err(o2, pd) <= tol_for(dtype)
    assert float((o2 - out).abs().max()) <= tol_for(dtype)


def test_index_arrays_in_pinned_host_memory():
    # Block tables, context lengths and shared-prefix groups may live in pinned host memory (the engine's
    # staging buffer): the kernels read them over the bus and the results are bitwise those of device copies.
    import paged_kv_cache_358_amd as pa
    lens = [5000, 1, 700, 0, 1600, 16]
    pd = PagedDecode(synth.scaled(synth.C3, lens=lens))
    host_t = pd.block_tables.cpu().pin_memory()
    host_l = pd.context_lens.cpu().pin_memory()
    assert pa.device_address(host_t) != 0
    for part in (512, 64):
        ref = pd.run(partition_size=part)
        out = torch.empty_like(ref)
        pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, host_t, host_l, pd.cfg.softmax_scale, out,
                                  max_context_len=pd.max_context_len, partition_size=part)
        torch.cuda.synchronize()
        assert torch.equal(ref, out)
    groups = torch.tensor([[0, 1, 0], [1, 2, 0], [3, 3, 0]], dtype=torch.int32)
    ref = torch.empty(pd.q.shape, dtype=torch.float32, device="cuda")
    pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens, pd.cfg.softmax_scale,
                              ref, max_context_len=pd.max_context_len, shared=groups.cuda())
    out = torch.empty_like(ref)
    pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, host_t, host_l, pd.cfg.softmax_scale, out,
                              max_context_len=pd.max_context_len, shared=groups.pin_memory())
    torch.cuda.synchronize()
    assert torch.equal(ref, out)
    with pytest.raises(ValueError, match="pinned"):
        pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables.cpu(), pd.context_lens,
                                  pd.cfg.softmax_scale, out, max_context_len=pd.max_context_len)

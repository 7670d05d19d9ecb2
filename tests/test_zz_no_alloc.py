"""paged_attention_decode_noalloc (the entry point that allocates nothing) against
paged_attention_decode on the same inputs, through the C ABI.

Both run the same kernel on the same inputs; only where the partials live differs (the library's
per-GPU scratch array against a caller workspace), so the outputs must be identical bit for bit, and
within the fp64 oracle's bound.  Two calls in a row, the second with a smaller input, show that the
scratch needs no clearing between calls.
"""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_358_amd as pa
import synth
from paged_setup import PagedDecode, tol_for

pytestmark = pytest.mark.gpu


def _noalloc(pd, partition_size=None, shared=None):
    out = torch.full(pd.q.shape, float("nan"), dtype=torch.float32, device=pd.q.device)
    pa.paged_attention_decode_noalloc(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens,
                                      pd.cfg.softmax_scale, out, max_context_len=pd.max_context_len,
                                      partition_size=pd.cfg.partition_size if partition_size is None
                                      else partition_size, shared=shared)
    torch.cuda.synchronize()
    return out


def _worst(out, pd, seqs, heads):
    o = out.cpu().numpy()
    return max(float(np.max(np.abs(o[s, heads] - pd.oracle_sampled(s, heads)))) for s in seqs)


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    # First call: GQA with contexts that span many partitions and workgroup runs (partials and merges);
    # second call: fewer, shorter sequences on the same scratch, which still holds the first call's data.
    big = PagedDecode(synth.scaled(synth.C3, lens=[20000, 7, 5000, 16, 3000, 1, 9000, 2048], partition_size=256),
                      keep_truth=False)
    small = PagedDecode(synth.scaled(synth.C3, lens=[600, 33, 1500], partition_size=512), keep_truth=False)
    for pd in (big, small):
        ref = pd.run()
        got = _noalloc(pd)
        assert torch.equal(ref, got)
        heads = [0, 9, 63]
        assert _worst(got, pd, range(pd.cfg.num_seqs), heads) <= tol_for(pd.cfg.dtype)


def test_noalloc_groups_and_mha():
    # Forked samples read through shared-prefix groups (32 query columns per run slot), then an MHA batch.
    cfg = synth.scaled(synth.C3, lens=[700] * 4 + [1300, 40])
    pd = PagedDecode(cfg, keep_truth=False)
    t = pd.tables_np.copy()
    t[1:4, :40] = t[0, :40]                    # sequences 1..3 read sequence 0's first 40 blocks
    pd.block_tables = torch.from_numpy(t).cuda()
    groups = torch.tensor([[0, 4, 40], [4, 1, 0], [5, 1, 0]], dtype=torch.int32, device="cuda")
    ref = torch.empty(pd.q.shape, dtype=torch.float32, device="cuda")
    pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens, cfg.softmax_scale,
                              ref, max_context_len=pd.max_context_len, shared=groups)
    got = _noalloc(pd, shared=groups)
    assert torch.equal(ref, got)
    mha = PagedDecode(synth.scaled(synth.C2, lens=[2048, 1, 513, 1000]), keep_truth=False)
    ref, got = mha.run(), _noalloc(mha)
    assert torch.equal(ref, got)
    assert _worst(got, mha, range(4), [0, 31]) <= tol_for("bf16")


def test_noalloc_groups_on_8_token_blocks():
    # Group mode streams 8-token blocks two to a tile; an odd shared count (81 blocks) puts the last shared
    # block in each member's first own tile.  Two calls in a row: grouped, then plain on fewer sequences.
    cfg = synth.scaled(synth.C3, lens=[700] * 4 + [1300, 40], block_size=8)
    pd = PagedDecode(cfg, keep_truth=False)
    t = pd.tables_np.copy()
    t[1:4, :81] = t[0, :81]                    # sequences 1..3 read sequence 0's first 81 blocks
    pd.block_tables = torch.from_numpy(t).cuda()
    groups = torch.tensor([[0, 4, 81], [4, 1, 0], [5, 1, 0]], dtype=torch.int32, device="cuda")
    ref = torch.empty(pd.q.shape, dtype=torch.float32, device="cuda")
    pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens, cfg.softmax_scale,
                              ref, max_context_len=pd.max_context_len, shared=groups)
    got = _noalloc(pd, shared=groups)
    assert torch.isfinite(got).all()
    assert torch.equal(ref, got)
    small = PagedDecode(synth.scaled(synth.C3, lens=[600, 33, 1500], block_size=8), keep_truth=False)
    ref, got = small.run(), _noalloc(small)
    assert torch.equal(ref, got)
    assert _worst(got, small, range(3), [0, 9, 63]) <= tol_for(small.cfg.dtype)


def test_noalloc_groups_at_head_dim_256():
    # The largest partial slots a call can need (32 columns of 258 floats per slot) fit the scratch.
    cfg = synth.scaled(synth.C3, lens=[700] * 4 + [1300, 40], head_dim=256)
    pd = PagedDecode(cfg, keep_truth=False)
    t = pd.tables_np.copy()
    t[1:4, :40] = t[0, :40]                    # sequences 1..3 read sequence 0's first 40 blocks
    pd.block_tables = torch.from_numpy(t).cuda()
    groups = torch.tensor([[0, 4, 40], [4, 1, 0], [5, 1, 0]], dtype=torch.int32, device="cuda")
    ref = torch.empty(pd.q.shape, dtype=torch.float32, device="cuda")
    pa.paged_attention_decode(pd.q, pd.k_cache, pd.v_cache, pd.block_tables, pd.context_lens, cfg.softmax_scale,
                              ref, max_context_len=pd.max_context_len, shared=groups)
    got = _noalloc(pd, shared=groups)
    assert torch.isfinite(got).all()
    assert torch.equal(ref, got)
    assert _worst(got, pd, [4, 5], [0, 63]) <= tol_for(cfg.dtype)


def test_noalloc_rejects_what_its_scratch_cannot_hold():
    # fp32 caches with many partitions: the per-partition kernel would need more partial rows than the
    # scratch holds.  Rejected before anything is launched (the pointers below are not device memory,
    # so the sizes are checked first and the call is made only when the rejection is certain).
    S, hq, D, parts = 4096, 64, 128, 16
    need = S * hq * parts * (D + 2) * 4
    c = pa.CacheDesc(1024, 8, D, 16, pa.PA_F32)
    p = pa.DecodeParams(S, hq, 512, 512 * parts, 512, pa.PA_F32, c, None, 0, None, None)
    assert pa.lib.paged_attention_decode_kernel(ctypes.byref(p)) == b"decode_generic_kernel"
    assert pa.lib.paged_attention_workspace_bytes(ctypes.byref(p)) == need
    assert need > pa.lib.paged_attention_noalloc_scratch_bytes()
    fake = ctypes.c_void_p(256)
    assert pa.lib.paged_attention_decode_noalloc(fake, fake, fake, fake, fake, 0.1, fake, ctypes.byref(p)) == \
        pa.PA_ERR_WORKSPACE


def test_noalloc_batches_beyond_2048_sequences():
    # 4500 sequences on 32-token blocks: the split kernel once per slice of 2048 sequences, each slice
    # reusing the scratch; then a smaller batch (2100 sequences, one partition each at head_dim 64 on
    # 16-token blocks: the per-partition kernel, no partials).
    rng = np.random.default_rng(16)
    lens = rng.integers(1, 300, size=4500)
    lens[[0, 2047, 2048, 4096, 4499]] = [700, 513, 1100, 600, 1]
    big = PagedDecode(synth.DecodeConfig("noalloc_many", 47, 4500, 8, 2, 128, "bf16", "fixed",
                                         tuple(int(x) for x in lens), block_size=32), keep_truth=False)
    assert pa.paged_attention_workspace_bytes(big.q, big.k_cache, big.v_cache, big.block_tables,
                                              torch.empty(big.q.shape, device="cuda"), big.max_context_len,
                                              big.cfg.partition_size) <= pa.lib.paged_attention_noalloc_scratch_bytes()
    ref, got = big.run(), _noalloc(big)
    assert torch.equal(ref, got)
    assert _worst(got, big, [0, 2047, 2048, 4096, 4499], [0, 7]) <= tol_for("bf16")
    lens2 = rng.integers(1, 500, size=2100)
    small = PagedDecode(synth.DecodeConfig("noalloc_many_small", 48, 2100, 8, 2, 64, "bf16", "fixed",
                                           tuple(int(x) for x in lens2)), keep_truth=False)
    ref, got = small.run(), _noalloc(small)
    assert torch.equal(ref, got)
    assert _worst(got, small, [0, 2047, 2048, 2099], [0, 7]) <= tol_for("bf16")

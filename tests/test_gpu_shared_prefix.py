"""Decode with shared prefixes on the GPU against the fp64 oracle.

Prompts are written once, forked into samples that keep the prompt's blocks
("Stop Wasting GPU Memory" page, Technical Details, "Copy-on-Write for Parallel
Sampling"), and each sample appends its own tokens (the first write into the
shared partial block copies it).  The batch is laid out prompt by prompt, with
lone sequences in between; pa_shared_prefixes cuts the batch into groups and
paged_attention_decode reads each group's shared blocks once, with each
member's own blocks scored only for that member's query heads.  The oracle
sees only each sequence's contiguous truth (prefix + own tokens).

Tolerance: max abs error 5e-3 (bf16/fp16 inputs, fp32 accumulation) against the
oracle, for the shared call and the plain call alike.  Free pool memory and
slots past each context hold NaN.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_358_amd as pa
import synth
from oracle.attention import decode_attention_seq
from paged_setup import TORCH_DTYPE, to_torch

pytestmark = pytest.mark.gpu
B = 16


class ForkedBatch:
    def __init__(self, seed, hq, hkv, D, dtype, prompts, lone=(), partition_size=512, block_size=B):
        """prompts: list of (prefix_len, [tokens appended by each sample]).  lone: context lengths of
        unforked sequences placed after each prompt's samples in turn."""
        rng = np.random.default_rng(seed)
        self.hq, self.hkv, self.D, self.dtype, self.part = hq, hkv, D, dtype, partition_size
        self.bs = bs = block_size
        need = sum(-(-L // bs) + len(sm) * (-(-max(sm) // bs) + 1) for L, sm in prompts) + \
            sum(-(-n // bs) for n in lone)
        nblocks = need + 8
        self.alloc = pa.BlockAllocator(nblocks, bs, rng.permutation(nblocks).astype(np.int32))
        tdt = TORCH_DTYPE[dtype]
        self.k_cache, self.v_cache = pa.alloc_kv_cache(nblocks, hkv, D, tdt, "cuda", block_size=bs)
        self.k_cache.fill_(float("nan"))
        self.v_cache.fill_(float("nan"))

        def draw(n):
            return (synth.encode(rng.standard_normal((n, hkv, D), dtype=np.float32), dtype),
                    synth.encode(rng.standard_normal((n, hkv, D), dtype=np.float32), dtype))

        def write(sid, k, v):
            slots, pairs = self.alloc.append(sid, k.shape[0])
            if len(pairs):
                pa.block_copy(self.k_cache, self.v_cache, torch.from_numpy(pairs).cuda())
            pa.kv_append(to_torch(k, dtype), to_torch(v, dtype), torch.from_numpy(slots).cuda(), self.k_cache,
                         self.v_cache)

        self.order, self.truth = [], {}
        sid = 0
        lone = list(lone)
        for L, samples in prompts:
            root = sid
            pk, pv = draw(L)
            self.alloc.add(root)
            write(root, pk, pv)
            for c in range(1, len(samples)):
                self.alloc.fork(root, root + c)
            for c, n in enumerate(samples):
                k, v = draw(n)
                if n:
                    write(root + c, k, v)
                self.truth[root + c] = (np.concatenate([pk, k]), np.concatenate([pv, v]))
                self.order.append(root + c)
            sid += len(samples)
            if lone:
                n = lone.pop(0)
                k, v = draw(n)
                self.alloc.add(sid)
                if n:
                    write(sid, k, v)
                self.truth[sid] = (k, v)
                self.order.append(sid)
                sid += 1
        S = len(self.order)
        self.lens_np = np.array([self.truth[s][0].shape[0] for s in self.order], np.int32)
        self.max_blocks = int(max(1, -(-self.lens_np.max() // bs)))
        tables, lens = self.alloc.build_batch(self.order, self.max_blocks)
        assert np.array_equal(lens, self.lens_np)
        self.tables_np = tables.copy()
        self.tables = torch.from_numpy(self.tables_np).cuda()
        self.lens = torch.from_numpy(self.lens_np.copy()).cuda()
        self.q_np = synth.encode(rng.standard_normal((S, hq, D), dtype=np.float32), dtype)
        self.q = to_torch(self.q_np, dtype)
        self.scale = float(np.float32(1.0 / np.sqrt(D)))

    def groups(self, max_members=None, min_blocks=1):
        mm = 32 // (self.hq // self.hkv) if max_members is None else max_members
        return pa.shared_prefixes(self.tables_np, self.lens_np, mm, min_blocks, block_size=self.bs)

    def run(self, shared=None, out_dtype=torch.float32):
        out = torch.empty(self.q.shape, dtype=out_dtype, device="cuda")
        sh = None if shared is None else torch.from_numpy(np.ascontiguousarray(shared)).cuda()
        pa.paged_attention_decode(self.q, self.k_cache, self.v_cache, self.tables, self.lens, self.scale, out,
                                  max_context_len=int(self.lens_np.max()), partition_size=self.part, shared=sh)
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    def max_err(self, o):
        worst = 0.0
        for i, s in enumerate(self.order):
            k, v = self.truth[s]
            ref = decode_attention_seq(synth.decode_f64(self.q_np[i], self.dtype), synth.decode_f64(k, self.dtype),
                                       synth.decode_f64(v, self.dtype), self.scale)
            assert np.all(np.isfinite(o[i])), s
            worst = max(worst, float(np.max(np.abs(o[i] - ref))))
        return worst


def check(fb, **kw):
    gr = fb.groups(**kw)
    assert np.any(gr[:, 1] > 1)
    o_sh = fb.run(gr)
    o_plain = fb.run()
    assert fb.max_err(o_sh) <= 5e-3
    assert fb.max_err(o_plain) <= 5e-3
    assert float(np.max(np.abs(o_sh - o_plain))) <= 5e-3
    return gr, o_sh


def test_gqa_samples_ragged_suffixes():
    # 32 query / 8 KV heads: up to eight samples per group.  Prompt 2's sample 0 appends nothing to a
    # 512-token prompt, so its whole context is the group's shared blocks.
    prompts = [(1000, [200, 1, 17, 0, 64, 300, 5, 16]), (37, [3, 40, 100]), (512, [0, 15, 16, 600, 1, 2])]
    fb = ForkedBatch(1, 32, 8, 128, "bf16", prompts, lone=[700, 1])
    gr, _ = check(fb)
    # prompt 0: samples 0..7 (62 blocks; sample 3 appended nothing and fills 62 blocks too), then the
    # lone sequence, prompt 1's three samples (2 shared blocks), the other lone one, prompt 2's six
    # samples (32 blocks)
    assert gr.tolist() == [[0, 8, 62], [8, 1, 0], [9, 3, 2], [12, 1, 0], [13, 6, 32]]
    # groups of at most four: one column tile per group
    check(fb, max_members=4)


def test_mha_sixteen_members_multi_partition_prefix_and_rest():
    # g = 1: up to 32 members per group (here 20, then 16 and 4); a 1500-token prefix spans three
    # 512-token partitions, suffixes up to 1100 tokens span three more.
    rng = np.random.default_rng(5)
    prompts = [(1500, rng.integers(0, 1100, 20).tolist()), (800, rng.integers(1, 40, 3).tolist())]
    fb = ForkedBatch(2, 8, 8, 128, "f16", prompts, lone=[2000, 33])
    gr, _ = check(fb)
    assert gr[0].tolist() == [0, 20, 1500 // B]
    gr, _ = check(fb, max_members=16)
    assert gr[:2].tolist() == [[0, 16, 1500 // B], [16, 4, 1500 // B]]


@pytest.mark.parametrize("part", [16, 48, 1024])
def test_partition_sizes_and_head_dim_64(part):
    prompts = [(333, [40, 0, 500, 7, 16, 16, 1, 90]), (200, [1, 2])]
    fb = ForkedBatch(3, 16, 8, 64, "bf16", prompts, lone=[1], partition_size=part)
    check(fb)


def test_bf16_output_and_min_blocks():
    prompts = [(640, [10, 20, 30, 40]), (100, [1, 1, 1, 1])]
    fb = ForkedBatch(4, 32, 8, 128, "bf16", prompts)
    # min_blocks 8: prompt 1's 6 full blocks are not shared
    gr = fb.groups(min_blocks=8)
    assert gr.tolist() == [[0, 4, 40], [4, 1, 0], [5, 1, 0], [6, 1, 0], [7, 1, 0]]
    o = torch.empty(fb.q.shape, dtype=torch.bfloat16, device="cuda")
    sh = torch.from_numpy(gr.copy()).cuda()
    pa.paged_attention_decode(fb.q, fb.k_cache, fb.v_cache, fb.tables, fb.lens, fb.scale, o,
                              max_context_len=int(fb.lens_np.max()), shared=sh)
    torch.cuda.synchronize()
    o32 = fb.run(gr)
    ob = o.float().cpu().numpy()
    # bf16 output is the fp32 result rounded once: within half a bf16 ulp of it
    assert np.all(np.abs(ob - o32) <= np.abs(o32) * 2.0 ** -8 + 1e-30)


def test_workspace_reuse_between_shared_and_plain_calls():
    prompts = [(700, [5, 300, 9, 900]), (1200, [1, 2, 3, 4, 5, 6, 7, 8])]
    fb = ForkedBatch(6, 32, 8, 128, "bf16", prompts, lone=[1300])
    gr = fb.groups()
    need = pa.paged_attention_workspace_bytes(fb.q, fb.k_cache, fb.v_cache, fb.tables,
                                              torch.empty(1, device="cuda"), int(fb.lens_np.max()), 512, shared=True)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    sh = torch.from_numpy(gr.copy()).cuda()
    outs = []
    for use in (True, False, True, True):
        o = torch.empty(fb.q.shape, dtype=torch.float32, device="cuda")
        pa.paged_attention_decode(fb.q, fb.k_cache, fb.v_cache, fb.tables, fb.lens, fb.scale, o,
                                  max_context_len=int(fb.lens_np.max()), workspace=ws, shared=sh if use else None)
        outs.append(o)
    torch.cuda.synchronize()
    outs = [o.cpu().numpy() for o in outs]
    # the same call gives the same bits every time
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[0], outs[3])
    assert fb.max_err(outs[0]) <= 5e-3 and fb.max_err(outs[1]) <= 5e-3


def test_groups_of_one_and_an_empty_context():
    # every sequence alone (the cover without sharing) gives the plain call's bits; samples that
    # own one or two tokens beyond the shared blocks; an empty sequence alone gives 0
    prompts = [(48, [0, 1, 2, 16, 17, 100])]
    fb = ForkedBatch(7, 32, 8, 128, "bf16", prompts, lone=[0])
    alone = np.array([[s, 1, 0] for s in range(len(fb.order))], np.int32)
    o_alone, o_plain = fb.run(alone), fb.run()
    assert np.array_equal(o_alone, o_plain)
    gr = fb.groups()
    assert gr.tolist() == [[0, 6, 3], [6, 1, 0]]
    o = fb.run(gr)
    errs = []
    for i, s in enumerate(fb.order):
        k, v = fb.truth[s]
        if k.shape[0] == 0:
            assert np.all(o[i] == 0)
            continue
        ref = decode_attention_seq(synth.decode_f64(fb.q_np[i], "bf16"), synth.decode_f64(k, "bf16"),
                                   synth.decode_f64(v, "bf16"), fb.scale)
        errs.append(float(np.max(np.abs(o[i] - ref))))
    assert max(errs) <= 5e-3


@pytest.mark.parametrize("bs", [32, 64])
def test_blocks_of_several_tiles(bs):
    # Blocks of 32 or 64 tokens: the groups count whole blocks, the kernel streams 16-token tiles of
    # them (a shared block is several shared tiles; a member's own blocks start on a block edge).
    prompts = [(700, [0, 1, 31, 32, 33, 100, 500, 9]), (96, [1, 64, 2])]
    fb = ForkedBatch(8, 32, 8, 128, "bf16", prompts, lone=[65, 0], block_size=bs)
    assert fb.k_cache.shape[3] == bs
    gr, _ = check(fb)
    assert gr.tolist() == [[0, 8, 700 // bs], [8, 1, 0], [9, 3, 96 // bs], [12, 1, 0]]
    check(fb, max_members=3)


@pytest.mark.parametrize("hq,hkv", [(24, 8), (12, 2)])
def test_member_heads_straddling_column_tiles(hq, hkv):
    # g = 3 (ten members, 30 columns) and g = 6 (five members): a member's query heads can sit in
    # both 16-column tiles, so its own blocks are computed on both
    prompts = [(400, [3, 0, 50, 17, 200, 1, 16, 90, 5, 33]), (150, [2, 40])]
    fb = ForkedBatch(9, hq, hkv, 128, "bf16", prompts, lone=[77])
    gr, _ = check(fb)
    g = hq // hkv
    assert gr[0].tolist() == [0, min(10, 32 // g), 400 // B]


@pytest.mark.parametrize("hq,hkv,part", [(32, 8, 512), (24, 8, 48), (8, 8, 16)])
def test_eight_token_blocks(hq, hkv, part):
    # 8-token blocks stream two to a 16-token tile.  Prompt 0 shares 87 full blocks (an odd count: the
    # last shared block sits in a member's first own tile and is read through each member's row),
    # prompt 1 shares 12; samples own 0 to 500 tokens, so a member's last tile may hold one block.
    prompts = [(700, [0, 1, 4, 5, 12, 13, 500, 9, 31, 2]), (96, [1, 8, 9])]
    fb = ForkedBatch(10, hq, hkv, 128, "bf16", prompts, lone=[65, 0], partition_size=part, block_size=8)
    assert fb.k_cache.shape[3] == 8
    gr, _ = check(fb)
    g = hq // hkv
    assert gr[0].tolist() == [0, min(10, 32 // g), 700 // 8]
    check(fb, max_members=3)


def test_eight_token_blocks_group_spans_two_partitions():
    # MHA, three samples of 168 tokens that share one block: 11 tiles each, 33 in all, so the
    # group's context needs two 512-token partitions (and the partial slots that go with them).
    fb = ForkedBatch(11, 4, 4, 64, "f16", [(8, [160, 160, 160])], block_size=8)
    gr, _ = check(fb)
    assert gr.tolist() == [[0, 3, 1]]


def test_head_dim_64_one_workgroup_per_group_context():
    # 64 prompts x 2 samples, 8 KV heads, head_dim 64: 512 group contexts, at least two per CU and fewer
    # than the resident workgroups, so the grid is one workgroup per context (none cut into runs).
    prompts = [(100 + 7 * i, [5 + i % 3, 9]) for i in range(64)]
    fb = ForkedBatch(12, 16, 8, 64, "bf16", prompts)
    gr, _ = check(fb)
    assert len(gr) == 64 and np.all(gr[:, 1] == 2)


def test_head_dim_96():
    # head_dim 96 (three 32-dim score chunks, six 16-dim output tiles) in group mode
    prompts = [(333, [40, 0, 500, 7, 16, 16, 1, 90]), (200, [1, 2])]
    fb = ForkedBatch(13, 16, 8, 96, "bf16", prompts, lone=[1])
    check(fb)


@pytest.mark.parametrize("bs,hq,hkv,dtype", [(16, 16, 4, "bf16"), (32, 8, 8, "f16"), (8, 32, 8, "bf16")])
def test_head_dim_256(bs, hq, hkv, dtype):
    # head_dim 256 in group mode (one wave per SIMD, part of the state spilled): 16-, 32- and 8-token
    # blocks, MHA and GQA, groups of up to 32 / g members
    prompts = [(333, [40, 0, 500, 7, 16, 16, 1, 90][: 32 // (hq // hkv)]), (200, [1, 2])]
    fb = ForkedBatch(21, hq, hkv, 256, dtype, prompts, lone=[1], block_size=bs)
    check(fb)

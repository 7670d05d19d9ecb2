"""A seeded sweep of decode shapes on the GPU against the fp64 oracle.

Each case draws its shape from a fixed list (block size 8, 16, 32 or 64 tokens, head_dim 64, 96,
128 or 256, query heads per KV head 1..24, bf16 or fp16 inputs, fp32 or input-dtype output, the
default partition or one of 16 * 2^k tokens) and its context lengths from a seeded mix of
short, block-edge and multi-partition lengths, so that every kernel form the library
dispatches to (split kernel in plain mode on 16-token tiles, on pairs of 8-token blocks or on
32-token units, head_dim 256, the VALU kernel for the rest) meets ragged tails.  Tolerance: max
abs error 5e-3 with fp32 output (bf16/fp16 inputs, fp32 accumulation); a 16-bit output must be the
fp32 result rounded once: within half an ulp of the output type at the value (half the subnormal
spacing for fp16's smallest values).
"""
import numpy as np
import pytest
import torch

import synth
from paged_setup import PagedDecode, check_16bit_output, tol_for

pytestmark = pytest.mark.gpu

# (block size, head_dim, H_q, H_kv, dtype)
SHAPES = [
    (16, 128, 8, 8, "bf16"), (16, 128, 16, 4, "f16"), (16, 64, 16, 1, "bf16"), (16, 256, 8, 2, "f16"),
    (16, 256, 16, 16, "bf16"), (16, 128, 24, 8, "bf16"), (32, 128, 8, 8, "f16"), (32, 64, 32, 4, "bf16"),
    (32, 128, 16, 1, "bf16"), (64, 128, 12, 4, "bf16"), (64, 64, 8, 8, "f16"), (32, 256, 4, 2, "bf16"),
    (8, 128, 16, 2, "bf16"), (8, 64, 8, 8, "f16"), (8, 128, 24, 8, "f16"),
    (16, 96, 32, 32, "bf16"), (32, 96, 8, 2, "f16"), (8, 96, 12, 4, "bf16"), (16, 96, 24, 1, "bf16"),
    (8, 256, 8, 2, "f16"), (64, 256, 2, 1, "bf16"),
]


def lengths(rng, B, n):
    pick = [1, B - 1, B, B + 1, 16, 17, 511, 512, 513, 1024, 1025]
    out = [int(x) for x in rng.choice(pick, size=n // 2)]
    out += [int(x) for x in rng.integers(1, 3000, size=n - n // 2)]
    rng.shuffle(out)
    return out


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_decode_shape_sweep(case):
    B, D, hq, hkv, dtype = SHAPES[case]
    rng = np.random.default_rng(1000 + case)
    lens = lengths(rng, B, 7)
    cfg = synth.DecodeConfig(f"sweep{case}", 40 + case, len(lens), hq, hkv, D, dtype, "fixed", tuple(lens),
                             block_size=B)
    pd = PagedDecode(cfg)
    part = [0, 16 * B if 16 * B <= 1024 else B, max(B, 256)][case % 3]
    out = pd.run(partition_size=part or None)
    o = out.float().cpu().numpy()
    worst = 0.0
    for s in range(cfg.num_seqs):
        ref = pd.oracle(s)
        assert np.all(np.isfinite(o[s]))
        worst = max(worst, float(np.max(np.abs(o[s] - ref))))
    assert worst <= tol_for(dtype), (SHAPES[case], lens, part, worst)
    # 16-bit output: the fp32 result rounded once (within half an ulp of the type; fp16 below 2^-14 is
    # subnormal, spaced 2^-24)
    o16 = pd.run(out_dtype=pd.q.dtype, partition_size=part or None).float().cpu().numpy()
    check_16bit_output(o16, o, dtype)


def test_head_dim_64_one_workgroup_per_context():
    # 20 sequences x 32 heads at head_dim 64: 640 contexts, at least two per CU and fewer than the
    # resident workgroups, so the grid is one workgroup per context.
    rng = np.random.default_rng(77)
    lens = lengths(rng, 16, 20)
    cfg = synth.DecodeConfig("grid64", 77, len(lens), 32, 32, 64, "bf16", "fixed", tuple(lens))
    pd = PagedDecode(cfg)
    o = pd.run().float().cpu().numpy()
    worst = max(float(np.max(np.abs(o[s] - pd.oracle(s)))) for s in range(cfg.num_seqs))
    assert np.all(np.isfinite(o)) and worst <= tol_for("bf16"), (lens, worst)

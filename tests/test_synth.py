"""Checks of the shared seeded input module (encodings and workload shapes)."""
import math

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1.0, 3.0e38, 1e-40], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())
    assert np.isnan(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_decode_f64_is_exact():
    x = np.array([1.5, -2.25, 65504.0], np.float16)
    assert list(synth.decode_f64(x, "f16")) == [1.5, -2.25, 65504.0]


def test_context_lengths_follow_the_configs():
    assert list(synth.context_lens(synth.C1)) == [1, 15, 16, 33]
    l2 = synth.context_lens(synth.C2)
    assert l2.size == 64 and l2.min() >= 128 and l2.max() <= 2048
    l3 = synth.context_lens(synth.C3)
    assert l3.size == 256 and l3.min() >= 16 and l3.max() <= 8192
    assert 700 < np.median(l3) < 1500
    assert list(synth.context_lens(synth.C5)) == [131072] * 4


def test_pool_plans():
    p1 = synth.pool_plan(synth.C1)
    assert p1.num_blocks == 32 and sorted(p1.free_order) == list(range(32))
    l3 = synth.context_lens(synth.C3)
    p3 = synth.pool_plan(synth.C3, l3)
    need = int(synth.blocks_for(l3 + synth.C3.pool_slack_tokens).sum())
    assert p3.num_blocks == math.ceil(need / 0.7)
    assert p3.preoccupy_blocks == round(0.3 * p3.num_blocks)
    assert synth.C4.pool_blocks() == 64 * (62 + 8 * 13) + synth.C4.slack_blocks


def test_per_head_streams_are_independent():
    k_all, v_all = synth.seq_kv(synth.C3, 5, 40)
    k_one, v_one = synth.seq_kv(synth.C3, 5, 40, kv_heads=[6])
    assert np.array_equal(k_all[:, 6], k_one[:, 0]) and np.array_equal(v_all[:, 6], v_one[:, 0])

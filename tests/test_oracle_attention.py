"""Pins for the fp64 attention oracle.

Each test ties the oracle to something other than itself: a closed form, a
scalar brute force written with math.fsum/math.exp, PyTorch's own attention in
float64, or an invariant of softmax attention.  Together they fail on a dropped
scale, a missing normalisation, a sign error in the exponent, a wrong GQA head
mapping or a transposed operand.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import attend_one_head, decode_attention, decode_attention_seq
import synth


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force(q, keys, values, scale):
    """Scalar loops, math.fsum for every sum, math.exp for every weight."""
    S, hq, D = q.shape
    scale = float(np.float32(scale))          # the value the library receives
    out = np.zeros((S, hq, D))
    for s in range(S):
        K, V = keys[s], values[s]
        n, hkv, _ = K.shape
        g = hq // hkv
        for j in range(hq):
            h = j // g
            if n == 0:
                continue
            x = [scale * math.fsum(q[s, j, d] * K[t, h, d] for d in range(D)) for t in range(n)]
            m = max(x)
            w = [math.exp(xt - m) for xt in x]
            den = math.fsum(w)
            for d in range(D):
                out[s, j, d] = math.fsum(w[t] * V[t, h, d] for t in range(n)) / den
    return out


def test_single_token_returns_v_exactly():
    # ctx = 1: the only weight is exp(0) = 1, so out is V_0 bit for bit.
    q = _rand((3, 8, 64), 1)
    keys = [_rand((1, 2, 64), 10 + s) for s in range(3)]
    vals = [_rand((1, 2, 64), 20 + s) for s in range(3)]
    out = decode_attention(q, keys, vals, 0.125)
    for s in range(3):
        for j in range(8):
            assert np.array_equal(out[s, j], vals[s][0, j // 4])


def test_brute_force_tiny_c1_shapes():
    # The tiny fp32 workload: ctx {1, 15, 16, 33}, 4 MHA heads, D = 64.
    cfg = synth.C1
    lens = synth.context_lens(cfg)
    q = synth.decode_f64(synth.queries(cfg), cfg.dtype)
    keys, vals = [], []
    for s, n in enumerate(lens):
        k, v = synth.seq_kv(cfg, s, int(n))
        keys.append(synth.decode_f64(k, cfg.dtype))
        vals.append(synth.decode_f64(v, cfg.dtype))
    ref = brute_force(q, keys, vals, cfg.softmax_scale)
    out = decode_attention(q, keys, vals, cfg.softmax_scale)
    assert np.max(np.abs(out - ref)) < 1e-13


def test_brute_force_gqa_small():
    q = _rand((2, 6, 8), 3)
    keys = [_rand((n, 3, 8), 30 + n) for n in (5, 17)]
    vals = [_rand((n, 3, 8), 40 + n) for n in (5, 17)]
    ref = brute_force(q, keys, vals, 0.3)
    out = decode_attention(q, keys, vals, 0.3)
    assert np.max(np.abs(out - ref)) < 1e-13


def test_matches_torch_sdpa_float64():
    # Library special case: PyTorch's scaled_dot_product_attention in float64 on the
    # CPU, GQA expanded by repeating each KV head over its query group.
    hq, hkv, D = 16, 4, 32
    g = hq // hkv
    for n in (1, 7, 64, 300):
        q = _rand((1, hq, D), 50 + n)
        K = _rand((n, hkv, D), 60 + n)
        V = _rand((n, hkv, D), 70 + n)
        out = decode_attention(q, [K], [V], 0.17)[0]
        qt = torch.from_numpy(q[0]).unsqueeze(1)                     # [hq, 1, D]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)  # [hq, n, D]
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.contiguous(), vt.contiguous(), scale=float(np.float32(0.17)))[:, 0, :].numpy()
        assert np.max(np.abs(out - ref)) < 1e-12


def test_zero_scale_is_mean_of_values():
    V = _rand((37, 1, 16), 5)
    K = _rand((37, 1, 16), 6)
    out = attend_one_head(_rand(16, 7), K[:, 0], V[:, 0], 0.0)
    assert np.max(np.abs(out - V[:, 0].mean(axis=0))) < 1e-14


def test_identical_keys_is_mean_of_values():
    k = _rand(16, 8)
    K = np.tile(k, (25, 1))
    V = _rand((25, 16), 9)
    out = attend_one_head(_rand(16, 10), K, V, 0.9)
    assert np.max(np.abs(out - V.mean(axis=0))) < 1e-14


def test_two_tokens_closed_form():
    # out = (v0 + e^delta v1) / (1 + e^delta), delta = scale * q.(k1 - k0).
    rng = np.random.default_rng(11)
    for _ in range(20):
        q, k0, k1, v0, v1 = (rng.standard_normal(8) for _ in range(5))
        scale = rng.uniform(0.05, 2.0)
        delta = scale * float(np.dot(q, k1 - k0))
        expect = (v0 + math.exp(delta) * v1) / (1.0 + math.exp(delta))
        out = attend_one_head(q, np.stack([k0, k1]), np.stack([v0, v1]), scale)
        assert np.max(np.abs(out - expect)) < 1e-13


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(12)
    K = rng.standard_normal((50, 8))
    V = rng.standard_normal((50, 8))
    q = rng.standard_normal(8)
    K[17] = 60.0 * q / np.linalg.norm(q)          # score ~ 60*|q| above the rest
    out = attend_one_head(q, K, V, 1.0)
    assert np.max(np.abs(out - V[17])) < 1e-12


def test_large_scores_stay_finite():
    # Scores near 1e3 would overflow exp() without the max shift; the result is the
    # two-token closed form with delta = 1.
    q = np.array([1.0])
    out = attend_one_head(q, np.array([[1000.0], [1001.0]]), np.array([[0.0], [1.0]]), 1.0)
    assert abs(out[0] - math.e / (1 + math.e)) < 1e-13


def test_shift_invariance_of_keys():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 4, 16))
    K = rng.standard_normal((40, 2, 16))
    V = rng.standard_normal((40, 2, 16))
    u = rng.standard_normal((1, 2, 16))
    a = decode_attention(q, [K], [V], 0.25)
    b = decode_attention(q, [K + u], [V], 0.25)
    assert np.max(np.abs(a - b)) < 1e-12


def test_linearity_in_values():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 2, 16))
    K = rng.standard_normal((33, 2, 16))
    V1 = rng.standard_normal((33, 2, 16))
    V2 = rng.standard_normal((33, 2, 16))
    lhs = decode_attention(q, [K], [2.5 * V1 - 0.5 * V2], 0.25)
    rhs = 2.5 * decode_attention(q, [K], [V1], 0.25) - 0.5 * decode_attention(q, [K], [V2], 0.25)
    assert np.max(np.abs(lhs - rhs)) < 1e-12


def test_token_order_does_not_matter():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((1, 4, 16))
    K = rng.standard_normal((50, 4, 16))
    V = rng.standard_normal((50, 4, 16))
    p = rng.permutation(50)
    a = decode_attention(q, [K], [V], 0.3)
    b = decode_attention(q, [K[p]], [V[p]], 0.3)
    assert np.max(np.abs(a - b)) < 1e-13


def test_gqa_groups_are_contiguous():
    # 8 query heads over 2 KV heads: heads 0..3 read KV head 0, heads 4..7 KV head 1.
    n, D = 9, 4
    rng = np.random.default_rng(16)
    K = rng.standard_normal((n, 2, D))
    V = np.zeros((n, 2, D))
    V[:, 0, :] = 1.0
    V[:, 1, :] = -1.0
    out = decode_attention_seq(rng.standard_normal((8, D)), K, V, 0.5)
    assert np.all(out[:4] == 1.0) and np.all(out[4:] == -1.0)


def test_empty_context_is_zero():
    out = decode_attention(np.ones((1, 2, 4)), [np.zeros((0, 2, 4))], [np.zeros((0, 2, 4))], 1.0)
    assert np.all(out == 0.0)


def test_scale_is_taken_at_float32():
    # The library receives scale as a float32; the oracle must use that value.
    q = np.array([[[1.0]]])
    K = np.array([[[0.0]], [[1.0]]])
    V = np.array([[[0.0]], [[1.0]]])
    s = 0.1                                   # not representable in float32
    out = decode_attention(q, [K], [V], s)[0, 0, 0]
    d = float(np.float32(s))
    assert out == pytest.approx(math.exp(d) / (1 + math.exp(d)), abs=1e-15)
    assert abs(out - math.exp(s) / (1 + math.exp(s))) > 1e-10

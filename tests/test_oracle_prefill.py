"""Pins for the fp64 causal prefill oracle.

Each test ties the oracle to something other than itself: PyTorch's own causal attention
in float64 (with its built-in causal mask, and with an explicit mask for a chunk at the end
of a longer context), a scalar brute force with math.fsum/math.exp, the closed form of the
first position, and causality itself.  A wrong mask direction, an off-by-one in the
position, a dropped scale or a wrong GQA head mapping fails one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle.prefill import prefill_attention_seq


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_whole_sequence_matches_torch_causal_sdpa(hq, hkv):
    n, d = 37, 16
    q, k, v = _rand((n, hq, d), 1), _rand((n, hkv, d), 2), _rand((n, hkv, d), 3)
    scale = 0.3
    out = prefill_attention_seq(q, k, v, scale)
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                           # [H_q, n, D]
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=float(np.float32(scale)))
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_chunk_at_the_end_of_a_context_matches_explicit_mask():
    n, c, hq, hkv, d = 50, 9, 6, 3, 8
    q, k, v = _rand((c, hq, d), 4), _rand((n, hkv, d), 5), _rand((n, hkv, d), 6)
    scale = 0.25
    out = prefill_attention_seq(q, k, v, scale)
    g = hq // hkv
    pos = np.arange(n - c, n)
    mask = torch.from_numpy(np.arange(n)[None, :] <= pos[:, None])    # [c, n], True = attend
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)))
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_brute_force_scalar_loops():
    n, c, hq, hkv, d = 7, 4, 2, 1, 5
    q, k, v = _rand((c, hq, d), 7), _rand((n, hkv, d), 8), _rand((n, hkv, d), 9)
    scale = float(np.float32(0.7))
    out = prefill_attention_seq(q, k, v, 0.7)
    for i in range(c):
        p = n - c + i
        for j in range(hq):
            x = [scale * math.fsum(q[i, j, e] * k[t, 0, e] for e in range(d)) for t in range(p + 1)]
            m = max(x)
            w = [math.exp(xt - m) for xt in x]
            for e in range(d):
                want = math.fsum(w[t] * v[t, 0, e] for t in range(p + 1)) / math.fsum(w)
                assert abs(out[i, j, e] - want) < 1e-13


def test_first_position_returns_its_own_value():
    # a chunk that is the whole sequence: row 0 sees only token 0, so out = V_0 exactly
    n, hq, hkv, d = 12, 4, 2, 8
    q, k, v = _rand((n, hq, d), 10), _rand((n, hkv, d), 11), _rand((n, hkv, d), 12)
    out = prefill_attention_seq(q, k, v, 0.5)
    for j in range(hq):
        assert np.array_equal(out[0, j], v[0, j // 2])


def test_later_tokens_never_reach_earlier_rows():
    n, c, hq, d = 30, 10, 2, 8
    q, k, v = _rand((c, hq, d), 13), _rand((n, hq, d), 14), _rand((n, hq, d), 15)
    base = prefill_attention_seq(q, k, v, 0.4)
    k2, v2 = k.copy(), v.copy()
    k2[25:] += 100.0
    v2[25:] = -v2[25:]
    moved = prefill_attention_seq(q, k2, v2, 0.4)
    first_changed = 25 - (n - c)          # chunk row whose position is 25
    assert np.array_equal(base[:first_changed], moved[:first_changed])
    assert not np.allclose(base[first_changed:], moved[first_changed:])


def test_rows_and_heads_selection():
    n, c, hq, d = 20, 6, 4, 4
    q, k, v = _rand((c, hq, d), 16), _rand((n, hq, d), 17), _rand((n, hq, d), 18)
    full = prefill_attention_seq(q, k, v, 0.3)
    part = prefill_attention_seq(q, k, v, 0.3, rows=[5, 0], heads=[3, 1])
    assert np.array_equal(part, full[[5, 0]][:, [3, 1]])
    with pytest.raises(ValueError):
        prefill_attention_seq(_rand((21, hq, d), 19), k, v, 0.3)

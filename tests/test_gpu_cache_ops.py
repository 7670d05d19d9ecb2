"""kv_append and block_copy on the GPU against the oracle's paged-layout model,
byte for byte."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_358_amd as pa
import synth
from oracle import paged_layout as pl
from paged_setup import TORCH_DTYPE, raw_view, storage_raw, to_torch

pytestmark = pytest.mark.gpu


def random_cache(num_blocks, H, D, dtype, seed, block_size=16):
    k_cache, v_cache = pa.alloc_kv_cache(num_blocks, H, D, TORCH_DTYPE[dtype], block_size=block_size)
    rng = synth.rng(100, seed)
    kh = synth.encode(rng.standard_normal(k_cache.numel(), dtype=np.float32), dtype)
    vh = synth.encode(rng.standard_normal(v_cache.numel(), dtype=np.float32), dtype)
    k_cache.copy_(to_torch(kh, dtype).view(k_cache.shape))
    v_cache.copy_(to_torch(vh, dtype).view(v_cache.shape))
    return k_cache, v_cache, kh, vh


@pytest.mark.parametrize("dtype,H,D,B", [("f32", 4, 64, 16), ("bf16", 8, 128, 16), ("f16", 3, 64, 16),
                                          ("bf16", 32, 128, 16), ("bf16", 8, 128, 32), ("f32", 2, 64, 8)])
def test_kv_append_bitwise(dtype, H, D, B):
    N = 40
    k_cache, v_cache, kh, vh = random_cache(N, H, D, dtype, 1, B)
    rng = np.random.default_rng(2)
    T = 300
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int32)
    slots[::7] = -1                     # padding tokens are skipped
    slots[3] = N * B + 5                # out of range: skipped, never written
    k_new = synth.encode(rng.standard_normal((T, H, D), dtype=np.float32), dtype)
    v_new = synth.encode(rng.standard_normal((T, H, D), dtype=np.float32), dtype)
    pa.kv_append(to_torch(k_new, dtype), to_torch(v_new, dtype), torch.from_numpy(slots).cuda(), k_cache, v_cache)
    torch.cuda.synchronize()
    valid = [s if 0 <= s < N * B else -1 for s in slots]
    ek, ev = pl.apply_kv_append(storage_raw(kh, dtype), storage_raw(vh, dtype), valid,
                                storage_raw(k_new, dtype), storage_raw(v_new, dtype), H, D, B, synth.ELEM_BYTES[dtype])
    assert np.array_equal(raw_view(k_cache), ek)
    assert np.array_equal(raw_view(v_cache), ev)


def test_kv_append_empty_and_single():
    k_cache, v_cache, kh, vh = random_cache(4, 2, 64, "bf16", 3)
    empty = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    pa.kv_append(empty, empty, torch.empty(0, dtype=torch.int32, device="cuda"), k_cache, v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(raw_view(k_cache), storage_raw(kh, "bf16"))
    one = synth.encode(np.arange(128, dtype=np.float32).reshape(1, 2, 64), "bf16")
    pa.kv_append(to_torch(one, "bf16"), to_torch(one, "bf16"), torch.tensor([63], dtype=torch.int32, device="cuda"),
                 k_cache, v_cache)
    torch.cuda.synchronize()
    k, v = pl.gather_sequence(raw_view(k_cache), raw_view(v_cache), [3], 16, 2, 64, 16, 2)
    assert np.array_equal(k[15], storage_raw(one[0], "bf16")) and np.array_equal(v[15], storage_raw(one[0], "bf16"))


@pytest.mark.parametrize("dtype,H,D,npairs", [("bf16", 8, 128, 448), ("f32", 4, 64, 5), ("f16", 2, 64, 1)])
def test_block_copy_bitwise(dtype, H, D, npairs):
    N = 2 * npairs + 8
    k_cache, v_cache, kh, vh = random_cache(N, H, D, dtype, 4)
    rng = np.random.default_rng(5)
    perm = rng.permutation(N)
    pairs = np.stack([perm[:npairs], perm[npairs:2 * npairs]], axis=1).astype(np.int32)
    pairs_dev = torch.from_numpy(np.vstack([pairs, [[N + 3, 0], [0, -1]]]).astype(np.int32)).cuda()  # last two skipped
    pa.block_copy(k_cache, v_cache, pairs_dev)
    torch.cuda.synchronize()
    ek, ev = pl.apply_block_copy(storage_raw(kh, dtype), storage_raw(vh, dtype), pairs.tolist(), H, D, 16)
    assert np.array_equal(raw_view(k_cache), ek)
    assert np.array_equal(raw_view(v_cache), ev)


def test_block_copy_empty():
    k_cache, v_cache, kh, _ = random_cache(4, 2, 64, "bf16", 6)
    pa.block_copy(k_cache, v_cache, torch.empty(0, 2, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(raw_view(k_cache), storage_raw(kh, "bf16"))


def test_stage_copy_moves_pinned_host_words():
    import paged_kv_cache_358_amd as pa
    host = torch.arange(1, 1 + 4099, dtype=torch.int32).pin_memory()  # 4099 words: vector part + tail
    dev = torch.full((4100,), -7, dtype=torch.int32, device="cuda")
    pa.stage_copy(dev, host, 4099 * 4)
    torch.cuda.synchronize()
    got = dev.cpu()
    assert torch.equal(got[:4099], host) and got[4099].item() == -7


def test_stage_copy_rejects_pageable_source():
    import paged_kv_cache_358_amd as pa
    host = torch.arange(64, dtype=torch.int32)  # pageable: not addressable by the device
    dev = torch.empty(64, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        pa.stage_copy(dev, host, 256)
    rc = pa.lib.pa_stage_copy(ctypes.c_void_p(dev.data_ptr()), ctypes.c_void_p(host.data_ptr()), 256, None)
    assert rc == pa.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("dtype,H,D,slots_on", [("bf16", 8, 128, "host"), ("f32", 4, 64, "device"),
                                                 ("f16", 32, 128, "host")])
def test_stage_append_copies_and_appends_in_one_launch(dtype, H, D, slots_on):
    # The copy part moves the staging words; the append part writes the cache exactly as
    # kv_append does, with the slot mapping read from pinned host memory or the device.
    B, N = 16, 40
    k_cache, v_cache, kh, vh = random_cache(N, H, D, dtype, 4)
    rng = np.random.default_rng(5)
    T = 200
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int32)
    slots[::9] = -1
    slots[5] = N * B + 3
    k_new = synth.encode(rng.standard_normal((T, H, D), dtype=np.float32), dtype)
    v_new = synth.encode(rng.standard_normal((T, H, D), dtype=np.float32), dtype)
    host = torch.arange(7, 7 + 10003, dtype=torch.int32).pin_memory()
    dev = torch.full((10004,), -3, dtype=torch.int32, device="cuda")
    slot_t = torch.from_numpy(slots).pin_memory() if slots_on == "host" else torch.from_numpy(slots).cuda()
    pa.stage_append(dev, host, 10003 * 4, to_torch(k_new, dtype), to_torch(v_new, dtype), slot_t, k_cache, v_cache)
    torch.cuda.synchronize()
    got = dev.cpu()
    assert torch.equal(got[:10003], host) and got[10003].item() == -3
    valid = [s if 0 <= s < N * B else -1 for s in slots]
    ek, ev = pl.apply_kv_append(storage_raw(kh, dtype), storage_raw(vh, dtype), valid,
                                storage_raw(k_new, dtype), storage_raw(v_new, dtype), H, D, B, synth.ELEM_BYTES[dtype])
    assert np.array_equal(raw_view(k_cache), ek)
    assert np.array_equal(raw_view(v_cache), ev)


def test_stage_append_either_part_empty_and_bad_slots():
    k_cache, v_cache, kh, vh = random_cache(4, 2, 64, "bf16", 6)
    host = torch.arange(64, dtype=torch.int32).pin_memory()
    dev = torch.zeros(64, dtype=torch.int32, device="cuda")
    empty = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    pa.stage_append(dev, host, 64 * 4, empty, empty, torch.empty(0, dtype=torch.int32).pin_memory(), k_cache, v_cache)
    torch.cuda.synchronize()
    assert torch.equal(dev.cpu(), host) and np.array_equal(raw_view(k_cache), storage_raw(kh, "bf16"))
    one = synth.encode(np.arange(128, dtype=np.float32).reshape(1, 2, 64), "bf16")
    pa.stage_append(dev, host, 0, to_torch(one, "bf16"), to_torch(one, "bf16"),
                    torch.tensor([63], dtype=torch.int32).pin_memory(), k_cache, v_cache)
    torch.cuda.synchronize()
    k, v = pl.gather_sequence(raw_view(k_cache), raw_view(v_cache), [3], 16, 2, 64, 16, 2)
    assert np.array_equal(k[15], storage_raw(one[0], "bf16")) and np.array_equal(v[15], storage_raw(one[0], "bf16"))
    # pageable host slots: not addressable by the device, refused before any launch
    with pytest.raises(ValueError):
        pa.stage_append(dev, host, 0, to_torch(one, "bf16"), to_torch(one, "bf16"),
                        torch.tensor([1], dtype=torch.int32), k_cache, v_cache)
    c = pa.cache_desc(k_cache, v_cache)
    pageable = torch.tensor([1], dtype=torch.int32)
    kt = to_torch(one, "bf16")
    rc = pa.lib.pa_stage_append(ctypes.c_void_p(dev.data_ptr()), ctypes.c_void_p(host.data_ptr()), 0,
                                ctypes.c_void_p(kt.data_ptr()), ctypes.c_void_p(kt.data_ptr()),
                                ctypes.c_void_p(pageable.data_ptr()), 1, ctypes.c_void_p(k_cache.data_ptr()),
                                ctypes.c_void_p(v_cache.data_ptr()), ctypes.byref(c), None)
    assert rc == pa.PA_ERR_INVALID_ARG


def test_debug_checks_reject_undefined_copies_and_appends(monkeypatch):
    # With PA_DEBUG_CHECKS set, block_copy and kv_append read their index arrays back and refuse what
    # the kernels leave undefined, launching nothing; valid calls still copy byte for byte.
    k_cache, v_cache, kh, vh = random_cache(16, 2, 64, "bf16", 7)
    before_k, before_v = raw_view(k_cache), raw_view(v_cache)

    def pairs(rows):
        return torch.tensor(rows, dtype=torch.int32, device="cuda")

    bad_pairs = ([[3, 3]],                    # source is the destination
                 [[1, 5], [2, 5]],            # two copies onto one block
                 [[1, 5], [5, 6]])            # a destination that another pair reads
    for rows in bad_pairs:                    # without the checks these are the caller's problem
        monkeypatch.setenv("PA_DEBUG_CHECKS", "1")
        with pytest.raises(pa.PagedAttnError) as e:
            pa.block_copy(k_cache, v_cache, pairs(rows))
        assert e.value.status == pa.PA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert np.array_equal(raw_view(k_cache), before_k) and np.array_equal(raw_view(v_cache), before_v)
    # out-of-range pairs are skipped, not errors; a valid call copies
    pa.block_copy(k_cache, v_cache, pairs([[1, 5], [2, 6], [99, 3], [-1, 4]]))
    torch.cuda.synchronize()
    ek, ev = pl.apply_block_copy(storage_raw(kh, "bf16"), storage_raw(vh, "bf16"), [(1, 5), (2, 6)], 2, 64, 16)
    assert np.array_equal(raw_view(k_cache), ek) and np.array_equal(raw_view(v_cache), ev)

    new = to_torch(synth.encode(np.ones((3, 2, 64), np.float32), "bf16"), "bf16")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.kv_append(new, new, torch.tensor([17, 40, 17], dtype=torch.int32, device="cuda"), k_cache, v_cache)
    assert e.value.status == pa.PA_ERR_INVALID_ARG
    pa.kv_append(new, new, torch.tensor([17, -1, -1], dtype=torch.int32, device="cuda"), k_cache, v_cache)  # -1: skipped
    monkeypatch.setenv("PA_DEBUG_CHECKS", "0")
    pa.block_copy(k_cache, v_cache, pairs([[7, 8]]))                    # checks off: plain launch
    torch.cuda.synchronize()


def test_index_arrays_in_pinned_host_memory():
    # kv_append's slots and block_copy's pairs read from pinned host memory: the same bytes as from the device.
    k1, v1, kh, vh = random_cache(24, 4, 64, "bf16", 9)
    k2, v2 = k1.clone(), v1.clone()
    rng = np.random.default_rng(10)
    slots = torch.from_numpy(rng.choice(24 * 16, size=50, replace=False).astype(np.int32))
    new = to_torch(synth.encode(rng.standard_normal((50, 4, 64), dtype=np.float32), "bf16"), "bf16")
    pairs = torch.tensor([[1, 20], [2, 21], [3, 22]], dtype=torch.int32)
    pa.kv_append(new, new, slots.cuda(), k1, v1)
    pa.block_copy(k1, v1, pairs.cuda())
    pa.kv_append(new, new, slots.pin_memory(), k2, v2)
    pa.block_copy(k2, v2, pairs.pin_memory())
    torch.cuda.synchronize()
    assert np.array_equal(raw_view(k1), raw_view(k2)) and np.array_equal(raw_view(v1), raw_view(v2))

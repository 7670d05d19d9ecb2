"""Paged KV-cache decode attention for MI355X (gfx950): Python binding.

A thin ctypes layer over ``libpagedattn.so`` (C ABI in ``include/pagedattn.h``):
argument marshalling only.  Every step of the hot path runs in the library's HIP
kernels or its C++ allocator; there is no CPU or PyTorch fallback, and importing
this package fails if the library has not been built
(``python paged_kv_cache_358_amd/build.py``).

PyTorch supplies device memory and streams: tensors are passed by data pointer,
the stream is torch's current stream unless one is given.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# PAGEDATTN_LIB names another build of the same library (the host-sanitizer build of the tests).
LIB_PATH = os.environ.get("PAGEDATTN_LIB") or os.path.join(_PKG, "libpagedattn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_OUT_OF_BLOCKS, PA_ERR_HIP, PA_ERR_WORKSPACE = range(6)
PA_F32, PA_BF16, PA_F16 = 0, 1, 2
# The most sequences one decode call reads through a shared-prefix description (PA_MAX_GROUPED_SEQS).
PA_MAX_GROUPED_SEQS = 2048
BLOCK_SIZE = 16

# Every symbol the header declares, with its ctypes signature.
_i32, _i64, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_P32 = ctypes.POINTER(ctypes.c_int32)
_P64 = ctypes.POINTER(ctypes.c_int64)


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", _i64), ("num_kv_heads", _i32), ("head_dim", _i32), ("block_size", _i32),
                ("dtype", _i32)]


class SharedPrefix(ctypes.Structure):
    _fields_ = [("groups", _vp), ("num_groups", _i32)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_q_heads", _i32), ("max_blocks_per_seq", _i32), ("max_context_len", _i32),
                ("partition_size", _i32), ("out_dtype", _i32), ("cache", CacheDesc), ("workspace", _vp),
                ("workspace_bytes", _sz), ("stream", _vp), ("start_event", _vp),
                ("stop_event", _vp), ("shared", ctypes.POINTER(SharedPrefix))]


class PrefillParams(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_tokens", _i32), ("num_q_heads", _i32), ("max_blocks_per_seq", _i32),
                ("max_query_len", _i32), ("out_dtype", _i32), ("cache", CacheDesc), ("stream", _vp),
                ("start_event", _vp), ("stop_event", _vp), ("seq_order", _vp)]


_PAllocPtr = ctypes.POINTER(_vp)
SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_version": (_i32, []),
    "pa_last_error": (ctypes.c_char_p, []),
    "paged_attention_workspace_bytes": (_sz, [ctypes.POINTER(DecodeParams)]),
    "paged_attention_decode_kernel": (ctypes.c_char_p, [ctypes.POINTER(DecodeParams)]),
    "paged_attention_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, ctypes.POINTER(DecodeParams)]),
    "paged_attention_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _f32, _vp, ctypes.POINTER(DecodeParams)]),
    "paged_attention_noalloc_scratch_bytes": (_sz, []),
    "kv_append": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, ctypes.POINTER(CacheDesc), _vp]),
    "block_copy": (_i32, [_vp, _vp, _vp, _i32, ctypes.POINTER(CacheDesc), _vp]),
    "pa_stage_copy": (_i32, [_vp, _vp, _sz, _vp]),
    "pa_device_address": (_i32, [_vp, ctypes.POINTER(_vp)]),
    "paged_attention_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                       ctypes.POINTER(PrefillParams)]),
    "pa_stage_append": (_i32, [_vp, _vp, _sz, _vp, _vp, _vp, _i32, _vp, _vp, ctypes.POINTER(CacheDesc), _vp]),
    "pa_alloc_create": (_i32, [_i32, _i32, _P32, _PAllocPtr]),
    "pa_alloc_destroy": (None, [_vp]),
    "pa_seq_add": (_i32, [_vp, _i64]),
    "pa_seq_fork": (_i32, [_vp, _i64, _i64]),
    "pa_seq_append": (_i32, [_vp, _i64, _i32, _P32, _P32, _i32, _P32]),
    "pa_seq_append_batch": (_i32, [_vp, _P64, _i32, _P32, _P32, _P32, _i32, _P32]),
    "pa_seq_free": (_i32, [_vp, _i64]),
    "pa_seq_table": (_i32, [_vp, _i64, _P32, _i32, _P32]),
    "pa_seq_len": (_i64, [_vp, _i64]),
    "pa_num_free": (_i32, [_vp]),
    "pa_refcount": (_i32, [_vp, _i32]),
    "pa_free_list": (_i32, [_vp, _P32, _i32, _P32]),
    "pa_build_batch": (_i32, [_vp, _P64, _i32, _i32, _P32, _P32]),
    "pa_shared_prefixes": (_i32, [_P32, _P32, _i32, _i32, _i32, _i32, _i32, _P32, _i32, _P32]),
    "pa_prefill_order": (_i32, [_P32, _P32, _i32, _P32]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_cache_358_amd/build.py` "
                          "(the library has no CPU fallback)")
    # torch ships its own HIP runtime.  Loading it first makes the library's
    # libamdhip64.so.7 dependency resolve (by soname) to that same runtime; the
    # other order puts two HIP/HSA runtimes in the process and the second one
    # finds no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        self.status_name = lib.pa_status_string(status).decode()
        detail = f" ({lib.pa_last_error().decode()})" if status == PA_ERR_HIP else ""
        super().__init__(f"{what}: {self.status_name}{detail}")


def _check(status: int, what: str):
    if status != PA_OK:
        raise PagedAttnError(status, what)


# ----------------------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def torch_dtype_code(dt) -> int:
    torch = _torch()
    return {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float16: PA_F16}[dt]


def x_of(dtype_code: int) -> int:
    return 4 if dtype_code == PA_F32 else 8


def cache_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, dtype_code: int, block_size: int = BLOCK_SIZE):
    """Shapes of the K and V cache tensors in the library's layout."""
    x = x_of(dtype_code)
    return (num_blocks, num_kv_heads, head_dim // x, block_size, x), (num_blocks, num_kv_heads, head_dim, block_size)


def alloc_kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device="cuda",
                   block_size: int = BLOCK_SIZE):
    """Allocate an (uninitialised) K and V cache pair with torch."""
    torch = _torch()
    ks, vs = cache_shapes(num_blocks, num_kv_heads, head_dim, torch_dtype_code(dtype), block_size)
    return torch.empty(ks, dtype=dtype, device=device), torch.empty(vs, dtype=dtype, device=device)


def cache_desc(k_cache, v_cache) -> CacheDesc:
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("k_cache must be [N, H, D/X, B, X] and v_cache [N, H, D, B]")
    n, h, dx, b, x = k_cache.shape
    code = torch_dtype_code(k_cache.dtype)
    if v_cache.dtype != k_cache.dtype or x != x_of(code):
        raise ValueError("k_cache / v_cache dtype or chunk width mismatch")
    if tuple(v_cache.shape) != (n, h, dx * x, b):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} does not match k_cache {tuple(k_cache.shape)}")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    return CacheDesc(n, h, dx * x, b, code)


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _event_ptr(ev):
    """Raw hipEvent_t of a recorded torch.cuda.Event (None -> NULL)."""
    if ev is None:
        return None
    if ev.cuda_event == 0:
        raise ValueError("record the event once before passing it (torch creates events lazily)")
    return ev.cuda_event


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require_index(*ts):
    """Index arrays (tables, lengths, groups, slots, pairs) may be device tensors or pinned host tensors."""
    for t in ts:
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError("index arrays must be on the GPU or in pinned host memory")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _iptr(t):
    """Kernel address of an index array (device tensor, or pinned host tensor read over the bus)."""
    return ctypes.c_void_p(device_address(t)) if t is not None else ctypes.c_void_p(0)


def _require_device(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


# ----------------------------------------------------------------------------- kernels
def device_address(t) -> int:
    """The address a kernel uses for a device tensor or a pinned host tensor (read over the bus)."""
    if t.is_cuda:
        return t.data_ptr()
    if not t.is_pinned():
        raise ValueError("host memory must be pinned for the device to read it")
    out = _vp()
    _check(lib.pa_device_address(_ptr(t), ctypes.byref(out)), "pa_device_address")
    return out.value


def decode_params(q, k_cache, v_cache, block_tables, out, max_context_len: int, partition_size: int = 0,
                  workspace=None, stream=None, start_event=None, stop_event=None, shared=None) -> DecodeParams:
    """``shared`` is a SharedPrefix (kept alive by the caller for the call) or None."""
    c = cache_desc(k_cache, v_cache)
    S, hq, d = q.shape
    if d != c.head_dim:
        raise ValueError("q head_dim does not match the cache")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return DecodeParams(S, hq, block_tables.shape[1], int(max_context_len), int(partition_size),
                        torch_dtype_code(out.dtype), c, _ptr(workspace).value, ws_bytes,
                        _stream_ptr(stream).value, _event_ptr(start_event), _event_ptr(stop_event),
                        None if shared is None else ctypes.pointer(shared))


def paged_attention_workspace_bytes(q, k_cache, v_cache, block_tables, out, max_context_len: int,
                                    partition_size: int = 0, shared: bool = False) -> int:
    """Workspace bytes of a decode call; ``shared=True`` sizes it for calls with shared prefixes."""
    sh = SharedPrefix(None, 0) if shared else None
    p = decode_params(q, k_cache, v_cache, block_tables, out, max_context_len, partition_size, shared=sh)
    return int(lib.paged_attention_workspace_bytes(ctypes.byref(p)))


def paged_attention_decode_kernel(q, k_cache, v_cache, block_tables, out, max_context_len: int,
                                  partition_size: int = 0) -> str:
    """Name of the kernel that streams K/V for a decode call with these arguments, as the library
    chooses it ("" when nothing would be launched).  Shared-prefix groups change the kernel's mode,
    not the kernel."""
    p = decode_params(q, k_cache, v_cache, block_tables, out, max_context_len, partition_size)
    return lib.paged_attention_decode_kernel(ctypes.byref(p)).decode()


def shared_prefixes(tables, lens, max_members: int, min_blocks: int = 1, block_size: int = BLOCK_SIZE,
                    groups_out=None):
    """The batch (host block tables int32 [S, max_blocks], lengths int32 [S]) cut into groups of
    consecutive sequences that share leading full blocks: int32 [G, 3] rows of (first sequence,
    members, shared blocks), covering the batch in order (a sequence that shares nothing is a group
    of one with 0 shared blocks).  ``max_members`` is at most 32 // (H_q / H_kv) for
    paged_attention_decode.  ``groups_out`` (C-contiguous int32 [>= S, 3]) receives it in place."""
    t, tptr = _as_i32(tables)
    ln, lptr = _as_i32(lens)
    S = int(ln.size)
    if t.ndim != 2 or t.shape[0] < S:
        raise ValueError("tables must be int32 [S, max_blocks]")
    gr = np.empty((max(S, 1), 3), np.int32) if groups_out is None else groups_out
    if gr.dtype != np.int32 or not gr.flags.c_contiguous or gr.ndim != 2 or gr.shape[1] != 3 or gr.shape[0] < S:
        raise ValueError("shared_prefixes: groups_out must be C-contiguous int32 [>= S, 3]")
    ng = ctypes.c_int32(0)
    _check(lib.pa_shared_prefixes(tptr, lptr, S, int(t.shape[1]), int(block_size), int(max_members), int(min_blocks),
                                  gr.ctypes.data_as(_P32), gr.shape[0], ctypes.byref(ng)), "pa_shared_prefixes")
    return gr[:ng.value]


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out, *,
                           max_context_len: int, partition_size: int = 0, workspace=None, stream=None,
                           start_event=None, stop_event=None, shared=None):
    """out[s, j] = softmax attention of q[s, j] over sequence s's cached tokens.

    q [S, H_q, D] and out [S, H_q, D] (fp32 or the cache dtype), block_tables int32
    [S, max_blocks], context_lens int32 [S]; ``max_context_len`` is a host-known upper
    bound of context_lens.  ``workspace`` (any device tensor of at least
    ``paged_attention_workspace_bytes`` bytes) is allocated here if omitted.
    ``start_event`` / ``stop_event`` (torch.cuda.Events recorded once before) mark the
    start of the call's first kernel and the end of its last one.
    ``shared`` = device int32 [G, 3] groups from ``shared_prefixes`` (covering the batch): each
    group's shared leading blocks are read once for all its members.
    """
    torch = _torch()
    # Shapes first: the kernels read context_lens[s] and table row s (row stride block_tables.shape[1]) for
    # every s < S, so undersized metadata would send them outside its allocation.
    if q.dim() != 3:
        raise ValueError("q must be [S, H_q, D]")
    S = q.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != S or block_tables.shape[1] < 1:
        raise ValueError(f"block_tables must be [S={S}, max_blocks >= 1], got {tuple(block_tables.shape)}")
    if context_lens.dim() != 1 or context_lens.numel() != S:
        raise ValueError(f"context_lens must be [S={S}], got {tuple(context_lens.shape)}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _require_device(q, k_cache, v_cache, out)
    _require_index(block_tables, context_lens)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if q.dtype != k_cache.dtype:
        raise ValueError("q must have the cache dtype")
    sh = None
    if shared is not None:
        _require_index(shared)
        if shared.dtype != torch.int32 or (shared.numel() and (shared.dim() != 2 or shared.shape[1] != 3)):
            raise ValueError("shared must be int32 [G, 3]")
        sh = SharedPrefix(_iptr(shared).value, shared.shape[0] if shared.numel() else 0)
    if workspace is None:
        need = paged_attention_workspace_bytes(q, k_cache, v_cache, block_tables, out, max_context_len,
                                               partition_size, shared=sh is not None)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    p = decode_params(q, k_cache, v_cache, block_tables, out, max_context_len, partition_size, workspace, stream,
                      start_event, stop_event, sh)
    _check(lib.paged_attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _iptr(block_tables),
                                      _iptr(context_lens), float(scale), _ptr(out), ctypes.byref(p)),
           "paged_attention_decode")
    return out


def paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out, *,
                                   max_context_len: int, partition_size: int = 0, stream=None, start_event=None,
                                   stop_event=None, shared=None):
    """paged_attention_decode without a workspace: the library's per-GPU scratch array holds the partials
    (nothing is allocated; calls that overlap on one GPU race).  Same arguments otherwise."""
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [S, H_q, D]")
    S = q.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != S or block_tables.shape[1] < 1:
        raise ValueError(f"block_tables must be [S={S}, max_blocks >= 1], got {tuple(block_tables.shape)}")
    if context_lens.dim() != 1 or context_lens.numel() != S:
        raise ValueError(f"context_lens must be [S={S}], got {tuple(context_lens.shape)}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    _require_device(q, k_cache, v_cache, out)
    _require_index(block_tables, context_lens)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if q.dtype != k_cache.dtype:
        raise ValueError("q must have the cache dtype")
    sh = None
    if shared is not None:
        _require_index(shared)
        if shared.dtype != torch.int32 or (shared.numel() and (shared.dim() != 2 or shared.shape[1] != 3)):
            raise ValueError("shared must be int32 [G, 3]")
        sh = SharedPrefix(_iptr(shared).value, shared.shape[0] if shared.numel() else 0)
    p = decode_params(q, k_cache, v_cache, block_tables, out, max_context_len, partition_size, None, stream,
                      start_event, stop_event, sh)
    _check(lib.paged_attention_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _iptr(block_tables),
                                              _iptr(context_lens), float(scale), _ptr(out), ctypes.byref(p)),
           "paged_attention_decode_noalloc")
    return out


def paged_attention_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float, out, *,
                            max_query_len: int, stream=None, start_event=None, stop_event=None, seq_order=None):
    """out[row, j] = causal attention of chunk row `row` over its sequence's cached tokens.

    q / out [T, H_q, D]; query_start int32 [S + 1] (device) gives each sequence's first row;
    context_lens int32 [S] counts the sequence's tokens including its chunk (already appended);
    ``max_query_len`` is a host-known upper bound of the chunk lengths.  ``seq_order`` (int32 [S],
    device or pinned host, from ``prefill_order``) starts the heaviest sequences first; it changes
    the launch's tail, not the results.
    """
    torch = _torch()
    _require_device(q, k_cache, v_cache, block_tables, context_lens, query_start, out)
    for t in (block_tables, context_lens, query_start):
        if t.dtype != torch.int32:
            raise ValueError("block_tables, context_lens and query_start must be int32")
    if q.dtype != k_cache.dtype:
        raise ValueError("q must have the cache dtype")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    c = cache_desc(k_cache, v_cache)
    T, hq, d = q.shape
    if d != c.head_dim:
        raise ValueError("q head_dim does not match the cache")
    S = block_tables.shape[0]
    if query_start.numel() != S + 1 or context_lens.numel() != S:
        raise ValueError("query_start must have S + 1 entries and context_lens S")
    if seq_order is not None:
        _require_index(seq_order)
        if seq_order.dtype != torch.int32 or seq_order.numel() != S:
            raise ValueError("seq_order must be int32 with S entries")
    p = PrefillParams(S, T, hq, block_tables.shape[1], int(max_query_len), torch_dtype_code(out.dtype), c,
                      _stream_ptr(stream).value, _event_ptr(start_event), _event_ptr(stop_event),
                      _iptr(seq_order).value)
    _check(lib.paged_attention_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                                       _ptr(query_start), float(scale), _ptr(out), ctypes.byref(p)),
           "paged_attention_prefill")
    return out


def prefill_order(context_lens, query_start):
    """Host int32 [S]: the sequences by descending prefill work (the (row, token) pairs of their chunk),
    ties in batch order, for ``paged_attention_prefill(..., seq_order=...)``.  context_lens [S] and
    query_start [S + 1] are host arrays."""
    ln, lptr = _as_i32(context_lens)
    qs, qptr = _as_i32(query_start)
    S = int(ln.size)
    if qs.size != S + 1:
        raise ValueError("query_start must have S + 1 entries")
    order = np.empty(S, dtype=np.int32)
    _check(lib.pa_prefill_order(lptr, qptr, S, order.ctypes.data_as(_P32)), "pa_prefill_order")
    return order


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, *, stream=None):
    """Write k_new/v_new [T, H_kv, D] into the cache slots slot_mapping[T] (int32, -1 = skip; a device
    tensor or a pinned host tensor)."""
    torch = _torch()
    _require_device(k_new, v_new, k_cache, v_cache)
    _require_index(slot_mapping)
    if slot_mapping.dtype != torch.int32:
        raise ValueError("slot_mapping must be int32")
    c = cache_desc(k_cache, v_cache)
    T = slot_mapping.numel()
    if tuple(k_new.shape) != (T, c.num_kv_heads, c.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new / v_new must be [T, H_kv, D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise ValueError("k_new / v_new must have the cache dtype")
    _check(lib.kv_append(_ptr(k_new), _ptr(v_new), _iptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache),
                         ctypes.byref(c), _stream_ptr(stream)), "kv_append")


def block_copy(k_cache, v_cache, pairs, *, stream=None):
    """Copy whole blocks pairs[i, 0] -> pairs[i, 1] (int32 [n, 2], a device tensor or a pinned host
    tensor), K and V."""
    torch = _torch()
    _require_device(k_cache, v_cache)
    _require_index(pairs)
    if pairs.dtype != torch.int32 or (pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2)):
        raise ValueError("pairs must be int32 [n, 2]")
    c = cache_desc(k_cache, v_cache)
    n = pairs.shape[0] if pairs.numel() else 0
    _check(lib.block_copy(_ptr(k_cache), _ptr(v_cache), _iptr(pairs), n, ctypes.byref(c), _stream_ptr(stream)),
           "block_copy")


def stage_copy(dst, src, nbytes: int, *, stream=None):
    """Copy nbytes from pinned host tensor src to device tensor dst with one kernel on the stream."""
    if not dst.is_cuda or src.is_cuda or not src.is_pinned():
        raise ValueError("stage_copy copies a pinned host tensor into a device tensor")
    if nbytes > min(dst.numel() * dst.element_size(), src.numel() * src.element_size()):
        raise ValueError("nbytes exceeds a buffer")
    _check(lib.pa_stage_copy(_ptr(dst), _ptr(src), int(nbytes), _stream_ptr(stream)), "pa_stage_copy")


def stage_append(dst, src, nbytes: int, k_new, v_new, slot_mapping, k_cache, v_cache, *, stream=None):
    """stage_copy(dst, src, nbytes) and kv_append(k_new, v_new, slot_mapping, ...) in one launch.
    slot_mapping (int32 [T]) may be a device tensor or a pinned host tensor (read over the bus)."""
    torch = _torch()
    if not dst.is_cuda or src.is_cuda or not src.is_pinned():
        raise ValueError("stage_append copies a pinned host tensor into a device tensor")
    if nbytes > min(dst.numel() * dst.element_size(), src.numel() * src.element_size()):
        raise ValueError("nbytes exceeds a buffer")
    _require_device(k_new, v_new, k_cache, v_cache)
    T = slot_mapping.numel()
    if slot_mapping.dtype != torch.int32 or (T and not (slot_mapping.is_cuda or slot_mapping.is_pinned())):
        raise ValueError("slot_mapping must be int32, on the device or in pinned host memory")
    c = cache_desc(k_cache, v_cache)
    if tuple(k_new.shape) != (T, c.num_kv_heads, c.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new / v_new must be [T, H_kv, D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise ValueError("k_new / v_new must have the cache dtype")
    _check(lib.pa_stage_append(_ptr(dst), _ptr(src), int(nbytes), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T,
                               _ptr(k_cache), _ptr(v_cache), ctypes.byref(c), _stream_ptr(stream)), "pa_stage_append")


# ----------------------------------------------------------------------------- allocator
def _as_i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_P32)


class BlockAllocator:
    """Host block allocator (C++): free pool, reference counts, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, free_order=None):
        h = _vp()
        if free_order is None:
            st = lib.pa_alloc_create(num_blocks, block_size, None, ctypes.byref(h))
        else:
            arr, ptr = _as_i32(free_order)
            if arr.size != num_blocks:
                raise ValueError("free_order must have num_blocks entries")
            st = lib.pa_alloc_create(num_blocks, block_size, ptr, ctypes.byref(h))
        _check(st, "pa_alloc_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self, _destroy=lib.pa_alloc_destroy):
        # _destroy is bound when the class is made: at interpreter exit the module's globals may
        # already be gone when the last allocators are collected.
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _destroy(h)
            self._h = None

    def add(self, seq: int):
        _check(lib.pa_seq_add(self._h, seq), "pa_seq_add")

    def fork(self, parent: int, child: int):
        _check(lib.pa_seq_fork(self._h, parent, child), "pa_seq_fork")

    def append(self, seq: int, n: int = 1):
        """Returns (slots int32[n], pairs int32[k, 2])."""
        slots = np.empty(max(n, 1), np.int32)
        pairs = np.empty((1, 2), np.int32)
        npairs = ctypes.c_int32(0)
        _check(lib.pa_seq_append(self._h, seq, n, slots.ctypes.data_as(_P32), pairs.ctypes.data_as(_P32), 1,
                                 ctypes.byref(npairs)), "pa_seq_append")
        return slots[:n], pairs[:npairs.value]

    def append_batch(self, seqs, counts, slots_out=None, pairs_out=None):
        """One decode step: seqs[i] appends counts[i] tokens.  Returns (slots, pairs)."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        cnt, cptr = _as_i32(counts)
        total = int(cnt.sum())
        slots = np.empty(max(total, 1), np.int32) if slots_out is None else slots_out
        cap = len(ids) if pairs_out is None else pairs_out.shape[0]
        pairs = np.empty((max(cap, 1), 2), np.int32) if pairs_out is None else pairs_out
        npairs = ctypes.c_int32(0)
        _check(lib.pa_seq_append_batch(self._h, ids.ctypes.data_as(_P64), len(ids), cptr, slots.ctypes.data_as(_P32),
                                       pairs.ctypes.data_as(_P32), cap, ctypes.byref(npairs)),
               "pa_seq_append_batch")
        return slots[:total], pairs[:npairs.value]

    def free(self, seq: int):
        _check(lib.pa_seq_free(self._h, seq), "pa_seq_free")

    def table(self, seq: int):
        n = ctypes.c_int32(0)
        ln = self.seq_len(seq)
        cap = max(1, -(-max(ln, 0) // self.block_size))
        out = np.empty(cap, np.int32)
        _check(lib.pa_seq_table(self._h, seq, out.ctypes.data_as(_P32), cap, ctypes.byref(n)), "pa_seq_table")
        return out[:n.value].tolist()

    def seq_len(self, seq: int) -> int:
        return int(lib.pa_seq_len(self._h, seq))

    def num_free(self) -> int:
        return int(lib.pa_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(lib.pa_refcount(self._h, block))

    def free_list(self):
        out = np.empty(max(self.num_blocks, 1), np.int32)
        n = ctypes.c_int32(0)
        _check(lib.pa_free_list(self._h, out.ctypes.data_as(_P32), self.num_blocks, ctypes.byref(n)),
               "pa_free_list")
        return out[:n.value].tolist()

    def build_batch(self, seqs, max_blocks: int, tables_out=None, lens_out=None):
        """(tables int32[n, max_blocks] padded with -1, lens int32[n]).  ``tables_out`` /
        ``lens_out`` (C-contiguous int32 of at least that shape) receive them in place."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(ids)
        if tables_out is None:
            tables_out = np.empty((max(n, 1), max(max_blocks, 1)), np.int32)
        if lens_out is None:
            lens_out = np.empty(max(n, 1), np.int32)
        for arr, shape in ((tables_out, (n, max_blocks)), (lens_out, (n,))):
            if (arr.dtype != np.int32 or not arr.flags.c_contiguous or arr.ndim != len(shape)
                    or any(a < b for a, b in zip(arr.shape, shape))
                    or (arr.ndim == 2 and n > 1 and arr.shape[1] != max_blocks)):
                raise ValueError(f"build_batch: output must be C-contiguous int32 of shape >= {shape}")
        _check(lib.pa_build_batch(self._h, ids.ctypes.data_as(_P64), n, max_blocks,
                                  tables_out.ctypes.data_as(_P32), lens_out.ctypes.data_as(_P32)), "pa_build_batch")
        return tables_out[:n, :max_blocks], lens_out[:n]


__all__ = ["paged_attention_decode", "device_address", "paged_attention_decode_noalloc", "paged_attention_workspace_bytes", "paged_attention_decode_kernel", "shared_prefixes", "SharedPrefix", "paged_attention_prefill", "kv_append", "block_copy", "stage_copy",
           "stage_append",
           "BlockAllocator",
           "alloc_kv_cache", "cache_shapes", "cache_desc", "PagedAttnError", "lib", "LIB_PATH", "SIGNATURES",
           "PA_F32", "PA_BF16", "PA_F16", "BLOCK_SIZE"]

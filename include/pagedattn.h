/*
 * pagedattn.h — C ABI of the paged KV-cache decode library (gfx950 / MI355X).
 *
 * The KV cache of one attention layer is cut into fixed-size blocks of
 * block_size tokens (16 here); a per-sequence block table maps the sequence's
 * logical blocks to physical blocks anywhere in the pool ("Stop Wasting GPU
 * Memory: A Deep Dive Into vLLM's PagedAttention", Technical Details, "Core
 * Architecture"; the ml-canon page "49 vLLM / PagedAttention", box "Paging for
 * the KV cache" and its block-table sketch).  This library provides:
 *
 *   paged_attention_decode  single-query attention per head, gathering K/V
 *                           through the block tables (zhichai.net page "How
 *                           Virtual Memory Paging Solved LLM KV Cache Waste",
 *                           "Why it matters": the kernel gathers scattered
 *                           blocks; Key points: transformer math unchanged);
 *   kv_append               write each new token's K/V into its cache slot
 *                           (the sketch's write into the last block; Technical
 *                           Details, "Single Sequence Generation");
 *   block_copy              the copy-on-write block copy at divergence
 *                           (Technical Details, "Copy-on-Write for Parallel
 *                           Sampling");
 *   pa_alloc_* / pa_seq_*   the host block allocator: free pool, per-block
 *                           reference counts, copy-on-write, release at zero
 *                           (Technical Details, "Copy-on-Write ..." and "Beam
 *                           Search Optimization").
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory (e.g. torch tensors); the
 *     library never allocates or frees device memory.  Host pointers are
 *     caller-owned host memory.
 *   - GPU entry points are asynchronous on the given HIP stream (a hipStream_t
 *     passed as void*; NULL = the null stream).  Argument errors are detected
 *     synchronously on the host and nothing is launched.
 *   - Every call returns a pa_status; no C++ exception crosses the ABI.
 *
 * Cache layout (all tensors densely packed, element type = dtype):
 *   k_cache  [num_blocks][num_kv_heads][head_dim / X][block_size][X]
 *   v_cache  [num_blocks][num_kv_heads][head_dim][block_size]
 *   X = 16 / sizeof(element)  (8 for bf16/fp16, 4 for fp32)
 * i.e. each (block, kv head) is one contiguous tile of block_size tokens; K is
 * stored in 16-byte token-interleaved chunks and V transposed (tokens fastest),
 * so that one wavefront load instruction reads a contiguous run.  A token at
 * logical position p of a sequence with table T lives in block T[p / B] at
 * slot p % B; its flat slot number is T[p / B] * B + p % B.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,    /* null pointer, negative size, bad shape, unknown sequence */
  PA_ERR_UNSUPPORTED = 2,    /* valid request outside the compiled fast paths (dtype, block size, head_dim) */
  PA_ERR_OUT_OF_BLOCKS = 3,  /* allocator pool exhausted; allocator state unchanged */
  PA_ERR_HIP = 4,            /* a HIP launch or runtime call failed */
  PA_ERR_WORKSPACE = 5       /* workspace missing or smaller than paged_attention_workspace_bytes() */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_F16 = 2 } pa_dtype;

/* Shape of one layer's paged KV cache (see layout above). */
typedef struct pa_cache_desc {
  int64_t num_blocks;    /* physical blocks in the pool, > 0 */
  int32_t num_kv_heads;  /* H_kv, > 0 */
  int32_t head_dim;      /* D, a multiple of X; the decode MFMA path covers 64, 96, 128 and 256 */
  int32_t block_size;    /* tokens per block, <= 1024.  Decode takes 8 (two to a 16-token tile: partitions
                            of whole tiles) and 16 << j (16, 32, ..., 1024) on the MFMA path (bf16/fp16,
                            head_dim 64, 96 or 128, H_q / H_kv <= 32), with or without a pa_shared_prefix
                            description; other sizes on the VALU kernel; prefill likewise (8 and 16 << j on
                            its MFMA kernel, other sizes up to 1024 on its VALU kernel) */
  int32_t dtype;         /* pa_dtype of K and V */
} pa_cache_desc;

/*
 * Sequences of a decode batch that read the same leading blocks (forked samples or beams of one
 * prompt: "Stop Wasting GPU Memory" page, Technical Details, "Copy-on-Write for Parallel Sampling" and
 * "Beam Search Optimization").  The batch is cut into groups of consecutive sequences, in order: group i
 * is sequences first .. first + members - 1, whose block tables hold the same physical ids in entries
 * [0, prefix_blocks), each of which every member fills completely (prefix_blocks * block_size <=
 * context_lens[s]); a sequence that shares nothing is a group of one with prefix_blocks 0.
 * paged_attention_decode then treats a group as one context: its shared blocks followed by each member's
 * own blocks, with a block's scores counted only for the query heads of the sequences that hold it.
 * Each shared block is read once for all members; every output is the same softmax attention as
 * without the description, within rounding.  pa_shared_prefixes builds the groups from host copies of
 * the tables and lengths.
 *   groups   int32 [num_groups][3] (device or pinned host memory): first sequence, members, prefix_blocks
 * members * (H_q / H_kv) must not exceed 32 (the query columns of two matrix-core tiles).  A description
 * that does not match the tables gives undefined results (never out-of-bounds accesses).  Used by the split
 * kernel at head_dim 64/96/128 (bf16/fp16) in batches of up to PA_MAX_GROUPED_SEQS sequences; larger
 * batches and the other kernels ignore it.  A caller with a larger batch can cut it at group
 * boundaries into calls of at most PA_MAX_GROUPED_SEQS sequences each, with the groups' first sequences
 * counted from the call's first sequence (the Python engine does so).
 */
#define PA_MAX_GROUPED_SEQS 2048

typedef struct pa_shared_prefix {
  const int32_t* groups;
  int32_t num_groups;  /* 0 (= no sharing) or the number of groups covering the batch, <= num_seqs */
} pa_shared_prefix;

/* Parameters of one paged_attention_decode call. */
typedef struct pa_decode_params {
  int32_t num_seqs;            /* S >= 0 */
  int32_t num_q_heads;         /* H_q, a multiple of num_kv_heads; query head j reads KV head j / (H_q / H_kv) */
  int32_t max_blocks_per_seq;  /* row stride (in int32) of block_tables, >= 1 */
  int32_t max_context_len;     /* host-known upper bound of context_lens[]; sizes the grid without a device->host copy */
  int32_t partition_size;      /* tokens per split-context partition, a multiple of block_size, at most 1024;
                                  0 = 512 rounded down to whole blocks */
  int32_t out_dtype;           /* PA_F32, or the cache dtype */
  pa_cache_desc cache;
  void* workspace;             /* device scratch for partition partials, >= paged_attention_workspace_bytes(); may be
                                  NULL when that is 0 */
  size_t workspace_bytes;
  void* stream;                /* hipStream_t */
  void* start_event;           /* hipEvent_t or NULL: marks the start of the call's first kernel */
  void* stop_event;            /* hipEvent_t or NULL: marks the end of the call's last kernel.  Both travel with
                                  the kernel launches (no marker packets between kernels, which would delay the
                                  stream); the events must already exist.  Elapsed time between them is the
                                  call's GPU time; a caller can also wait on stop_event for the call's end.
                                  With num_seqs = 0 nothing is launched and both are recorded on the stream. */
  const pa_shared_prefix* shared; /* host pointer or NULL: shared leading blocks (see above).  When not NULL
                                  the workspace holds partials for whole groups (see the workspace size) */
} pa_decode_params;

/* Human-readable name of a status code (static string). */
const char* pa_status_string(int32_t status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t pa_version(void);

/* Text of the HIP error behind the most recent PA_ERR_HIP returned on the calling thread ("" if none).
 * The string is owned by the library and valid until the thread's next failing call. */
const char* pa_last_error(void);

/* ----------------------------------------------------------------------- decode attention */

/* Device workspace bytes paged_attention_decode needs for these parameters (0 when no context can span more
 * than one partition).  The call takes one of three kernels (paged_attention_decode_kernel names it):
 *   decode_split_kernel (bf16/fp16; head_dim 64, 96, 128 or 256 on blocks of 8 or 16 << j tokens;
 *     H_q / H_kv <= 32 (<= 16 at head_dim 256)): at most 1024 workgroups ("runs") each write at most two
 *     partials, so the workspace is 1024 * 2 * C fp32 rows of head_dim + 2 values (C = H_q / H_kv query
 *     columns, or 32 when p->shared is set or H_q / H_kv > 16), then num_seqs * H_kv uint64 arrival
 *     counters.  Its size does not grow with the batch's context lengths.  A batch of more than 2048
 *     sequences runs as one launch per 2048, in stream order, sharing the workspace.
 *   decode_mfma_kernel (batches of more than 2048 sequences on 16-token blocks, head_dim 64 or 128,
 *     H_q / H_kv <= 16, whose contexts all fit one partition; or a block table too wide for the split
 *     kernel's int32 tile index) / decode_generic_kernel (other shapes): P = num_seqs * H_q * n fp32
 *     partial rows of head_dim + 2 values, n = ceil(min(max_context_len, max_blocks_per_seq * block_size) /
 *     partition_size), when n > 1.
 * Returns 0 for invalid parameters (the decode call then reports the error).  The contents need no
 * initialisation (the counters carry a per-call tag) and are scratch between calls; two calls in flight at
 * once must not share a workspace. */
size_t paged_attention_workspace_bytes(const pa_decode_params* p);

/* Name of the kernel that streams the K/V blocks of a paged_attention_decode call with these parameters:
 * "decode_split_kernel", "decode_mfma_kernel" or "decode_generic_kernel" (the last two are followed by
 * reduce_partitions_kernel when a context spans several partitions).  The decode call chooses its kernel
 * with the same host rule.  "" for invalid parameters or num_seqs = 0 (nothing is launched).  A static
 * string; no device is touched. */
const char* paged_attention_decode_kernel(const pa_decode_params* p);

/*
 * Single-query decode attention over a paged KV cache.
 *
 * For each sequence s (context length n = context_lens[s]), query head j and
 * its KV head h = j / (H_q / H_kv):
 *     out[s, j, :] = sum_t softmax_t(scale * q[s, j, :] . K_s[t, h, :]) * V_s[t, h, :],   t < n
 * where K_s[t] / V_s[t] are read from block block_tables[s * max_blocks_per_seq + t / B], slot t % B.
 * A sequence with n == 0 gets out = 0.  Contexts longer than one partition are split into partitions whose
 * softmax partials (max, sum, normalised output) go to the workspace; the bf16/fp16 path merges them in the
 * same kernel launch, the other paths with a second kernel.
 *
 *   q             device [num_seqs][H_q][head_dim], cache dtype
 *   k_cache/v_cache  device, layout above
 *   block_tables  int32 [num_seqs][max_blocks_per_seq], device memory or pinned host memory (see
 *                 pa_device_address); entries past ceil(n / B) are never read
 *   context_lens  int32 [num_seqs], device or pinned host memory; values are clamped to [0,
 *                 min(max_context_len, max_blocks_per_seq * B)]
 *   scale         softmax scale (usually 1/sqrt(head_dim)), taken as float32
 *   out           device [num_seqs][H_q][head_dim], out_dtype
 * Table entries outside [0, num_blocks) are a caller error: the kernel never dereferences them and treats
 * their tokens as absent.  Slots of a block past n, and blocks not in any table, are never read, so they may
 * hold anything (including NaN).  Results are deterministic (no floating-point atomics) and do not depend on
 * which physical blocks hold the tokens.
 */
int32_t paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, float scale,
                               void* out, const pa_decode_params* p);

/*
 * paged_attention_decode_noalloc: paged_attention_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments
 * and results; p->workspace and p->workspace_bytes are ignored.  The partials and arrival counters live in
 * a scratch array of paged_attention_noalloc_scratch_bytes() (72 MiB) that the library keeps on each GPU
 * it runs on until the process ends.  Nothing is allocated per call (no hipMalloc, hipFree or allocating
 * library routine).  The scratch needs no clearing (the counters carry a per-call tag) and holds the last
 * call's contents.  Returns PA_ERR_WORKSPACE, launching nothing, when paged_attention_workspace_bytes(p)
 * exceeds the scratch (large batches on the per-partition kernels); every decode_split_kernel call fits.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time on one GPU (on different
 * streams, or from different threads) race and give undefined results.
 */
int32_t paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens, float scale,
                                       void* out, const pa_decode_params* p);

/* Bytes of the per-GPU scratch array of paged_attention_decode_noalloc. */
size_t paged_attention_noalloc_scratch_bytes(void);

/* ----------------------------------------------------------------------- cache writes */

/*
 * kv_append: for i in [0, num_tokens): if slot_mapping[i] is in [0, num_blocks * B), write
 * k_new[i, :, :] and v_new[i, :, :] into that slot (block slot / B, offset slot % B) of k_cache / v_cache;
 * other slots (-1 = padding) are skipped.
 *   k_new, v_new   device [num_tokens][num_kv_heads][head_dim], cache dtype
 *   slot_mapping   int32 [num_tokens], device or pinned host memory
 * Two tokens naming the same slot race (which one lands is undefined); the allocator never produces that.
 * With the environment variable PA_DEBUG_CHECKS set (and not "0") the call first copies slot_mapping back
 * to the host, synchronously, and returns PA_ERR_INVALID_ARG without launching if two in-range slots are
 * equal.
 */
int32_t kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, int32_t num_tokens,
                  void* k_cache, void* v_cache, const pa_cache_desc* cache, void* stream);

/*
 * block_copy: for each pair i in [0, num_pairs), copy physical block pairs[2i] (source) onto block
 * pairs[2i + 1] (destination): every slot, every KV head, K and V.  Pairs with an index outside
 * [0, num_blocks) are skipped.  Destinations must be distinct and must not be a source of the same call
 * (the allocator's copy-on-write pairs satisfy both); otherwise the result is undefined.  With the
 * environment variable PA_DEBUG_CHECKS set (and not "0") the call first copies pairs back to the host,
 * synchronously, and returns PA_ERR_INVALID_ARG without launching if an in-range pair has src == dst, two
 * share a destination, or a destination is also a source.
 *   pairs   int32 [num_pairs][2], device or pinned host memory
 */
int32_t block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                   const pa_cache_desc* cache, void* stream);

/* Parameters of one paged_attention_prefill call. */
typedef struct pa_prefill_params {
  int32_t num_seqs;            /* S >= 0 */
  int32_t num_tokens;          /* T = rows of q and out (query_start[S]) */
  int32_t num_q_heads;         /* H_q, a multiple of num_kv_heads */
  int32_t max_blocks_per_seq;  /* row stride (in int32) of block_tables, >= 1 */
  int32_t max_query_len;       /* host-known upper bound of the chunk lengths; sizes the grid */
  int32_t out_dtype;           /* PA_F32, or the cache dtype */
  pa_cache_desc cache;
  void* stream;                /* hipStream_t */
  void* start_event;           /* hipEvent_t or NULL, as for paged_attention_decode */
  void* stop_event;            /* hipEvent_t or NULL, as for paged_attention_decode */
  const int32_t* seq_order;    /* NULL, or [S] int32 (device or pinned host): the order in which the sequences'
                                  workgroups are started, a permutation of 0 .. S-1 (pa_prefill_order gives
                                  the heaviest first).  It changes the launch's tail, never the results;
                                  sequences it names twice are computed twice, sequences it leaves out are
                                  not written, entries outside 0 .. S-1 are skipped */
} pa_prefill_params;

/*
 * paged_attention_prefill: causal attention of each sequence's newest tokens (a chunk whose K/V
 * kv_append has already written) over the sequence's cached tokens, through its block table.
 * The prefill phase fills a sequence's blocks ("Stop Wasting GPU Memory" page, Technical
 * Details, "Single Sequence Generation"); the attention math is unchanged by paging
 * ("PagedAttention: How Virtual Memory Paging Solved LLM KV Cache Waste" page, Key points).
 * Chunk row i of sequence s (q row query_start[s] + i), with n = context_lens[s] tokens of
 * which c = query_start[s+1] - query_start[s] are the chunk, is position n - c + i and attends to
 * tokens 0 .. n - c + i:
 *   out[row, j, :] = sum_t softmax_t(scale * q[row, j, :] . K[t, j / g, :]) V[t, j / g, :]
 *   q            [T][H_q][D] (the cache dtype), device
 *   block_tables [S][max_blocks_per_seq] int32; context_lens [S] int32 (tokens including the chunk)
 *   query_start  [S + 1] int32, non-decreasing, query_start[0] = 0, query_start[S] = T, device
 *   out          [T][H_q][D] fp32 or the cache dtype
 * Rows whose position would be negative (a chunk longer than its context) are left unwritten.
 * bf16 / fp16 caches with head_dim 64, 96, 128 or 256 and blocks of 8 or 16 << j tokens run the MFMA kernel;
 * fp32 caches and the other 16-bit shapes up to head_dim 256 (a multiple of X) and blocks of up to 1024 tokens
 * run a VALU kernel (one wavefront per chunk row and query head); else PA_ERR_UNSUPPORTED.  Asynchronous on
 * the stream.
 */
int32_t paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start, float scale, void* out,
                                const pa_prefill_params* p);

/*
 * pa_prefill_order: the scheduling order for paged_attention_prefill's seq_order, on the host: sequences by
 * descending work (the (row, token) pairs their chunk attends over), ties in batch order.
 *   context_lens [S], query_start [S + 1]  host int32, as for paged_attention_prefill
 *   order        [S] host int32, written with a permutation of 0 .. S-1
 * PA_ERR_INVALID_ARG for S < 0 or a NULL pointer with S > 0.
 */
int32_t pa_prefill_order(const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs, int32_t* order);

/*
 * pa_device_address: the address a kernel uses for p, which is device memory (returned as is) or pinned host
 * memory (hipHostMalloc, torch pin_memory: the device-side address of the same bytes, read over the bus).
 * The index arrays of the GPU entry points (block tables, context lengths, shared-prefix groups, slot
 * mappings, copy pairs) may live in pinned host memory given by such an address; K/V, q, out and the
 * workspace must be device memory.  PA_ERR_INVALID_ARG for NULL or memory HIP does not know.
 */
int32_t pa_device_address(const void* p, const void** out);

/*
 * pa_stage_copy: copy `bytes` (a multiple of 4) from src to dst with one kernel on `stream`.  It moves
 * the host allocator's per-step output (block tables, context lengths, slot mapping, copy pairs) to
 * the device ahead of kv_append / block_copy / paged_attention_decode, on the same queue as those
 * kernels, so they need not wait on a separate copy engine.
 *   src   pinned host memory the device can address (hipHostMalloc, torch pin_memory), 16-byte aligned;
 *         it must stay unchanged until the copy has run (record an event after the call)
 *   dst   device memory, 16-byte aligned
 */
int32_t pa_stage_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * pa_stage_append: pa_stage_copy and kv_append in one kernel launch, for a decode step whose
 * allocator output needs no block copies first.  One part of the grid copies `bytes` from pinned
 * host `src` to device `dst`; the other writes k_new / v_new into the cache slots, as kv_append
 * does (the append of each new token: "Stop Wasting GPU Memory" page, Technical Details,
 * "Single Sequence Generation").  The append does not read `dst`: `slot_mapping` may be device
 * memory or pinned host memory (the staging buffer itself), read over the bus.  One launch fewer
 * per step than the two calls; the copy and the append run side by side.
 *   src, dst, bytes     as for pa_stage_copy (bytes may be 0)
 *   other arguments     as for kv_append (num_tokens may be 0)
 * Errors as for the two calls; PA_ERR_INVALID_ARG if slot_mapping is neither device nor pinned host
 * memory.
 */
int32_t pa_stage_append(void* dst, const void* src, size_t bytes, const void* k_new, const void* v_new,
                        const int32_t* slot_mapping, int32_t num_tokens, void* k_cache, void* v_cache,
                        const pa_cache_desc* cache, void* stream);

/* ----------------------------------------------------------------------- host block allocator */

typedef struct pa_allocator pa_allocator;

/* Create an allocator over blocks [0, num_blocks).  free_order (nullable, host int32[num_blocks], a
 * permutation) is the order a fresh pool hands blocks out; NULL = 0, 1, 2, ...  The pool is a LIFO stack:
 * freed blocks are handed out again first.  num_blocks * block_size must fit in int32. */
int32_t pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);

/* New empty sequence.  PA_ERR_INVALID_ARG if the id exists. */
int32_t pa_seq_add(pa_allocator* a, int64_t id);

/* child shares all of parent's blocks (each block's reference count + 1) and its length. */
int32_t pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child);

/*
 * Append n tokens to sequence id.  A token opens a fresh block when the last block is full (length % B == 0);
 * a token written into a partial last block that other sequences share (reference count > 1) first moves
 * the sequence onto a private copy: a fresh block is taken, (old, new) is emitted as a copy pair, the old
 * block's count drops by one.  slots_out[i] (host int32[n]) receives each token's flat slot; pairs_out
 * (host int32[pairs_cap][2], at most one pair per call) the copy pairs, *n_pairs their count.  If the pool
 * lacks the blocks the call needs it returns PA_ERR_OUT_OF_BLOCKS and changes nothing.
 */
int32_t pa_seq_append(pa_allocator* a, int64_t id, int32_t n, int32_t* slots_out, int32_t* pairs_out,
                      int32_t pairs_cap, int32_t* n_pairs);

/*
 * Batched form of pa_seq_append for one decode step: sequences ids[0..n_seqs) in order append counts[i]
 * tokens each; slots_out receives all slots concatenated in that order, pairs_out all copy pairs in order.
 * Atomic: if the whole batch does not fit in the pool (or in pairs_cap), nothing changes.
 */
int32_t pa_seq_append_batch(pa_allocator* a, const int64_t* ids, int32_t n_seqs, const int32_t* counts,
                            int32_t* slots_out, int32_t* pairs_out, int32_t pairs_cap, int32_t* n_pairs);

/* Release a sequence: each block of its table (in logical order) loses one reference; blocks reaching zero
 * go back to the free pool at once. */
int32_t pa_seq_free(pa_allocator* a, int64_t id);

/* Copy a sequence's block table into out (host int32[cap]); *n = its length in blocks. */
int32_t pa_seq_table(const pa_allocator* a, int64_t id, int32_t* out, int32_t cap, int32_t* n);

/* Tokens held by a sequence, or -1 if unknown. */
int64_t pa_seq_len(const pa_allocator* a, int64_t id);

/* Blocks in the free pool. */
int32_t pa_num_free(const pa_allocator* a);

/* Reference count of a block, or -1 if out of range. */
int32_t pa_refcount(const pa_allocator* a, int32_t block);

/* The free pool, bottom of the stack first (the last entry is handed out next). */
int32_t pa_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n);

/* Block tables of sequences ids[0..n) as rows of max_blocks int32 padded with -1 (host
 * tables_out[n][max_blocks]), and their lengths (host lens_out[n]). */
int32_t pa_build_batch(const pa_allocator* a, const int64_t* ids, int32_t n, int32_t max_blocks,
                       int32_t* tables_out, int32_t* lens_out);

/*
 * The groups of pa_shared_prefix for a batch (host arrays).  full(s) = min(lens[s] / block_size,
 * max_blocks).  A run starts at the first sequence i not yet grouped with k = full(i); the next sequence j
 * joins while the run has fewer than max_members members and k' = min(k, full(j), leading entries where
 * rows i and j agree) >= min_blocks (then k = k').  A run of two or more is a group (i, members, k); every
 * other sequence is a group (i, 1, 0) of its own.  The groups cover the batch in order.
 *   tables  host int32 [num_seqs][max_blocks];  lens  host int32 [num_seqs]
 *   groups  host int32 [groups_cap][3] (out);  *num_groups (out)
 * PA_ERR_INVALID_ARG for null pointers, num_seqs < 0, block_size, max_blocks, max_members or min_blocks < 1,
 * or groups_cap < num_seqs.
 */
int32_t pa_shared_prefixes(const int32_t* tables, const int32_t* lens, int32_t num_seqs, int32_t max_blocks,
                           int32_t block_size, int32_t max_members, int32_t min_blocks, int32_t* groups,
                           int32_t groups_cap, int32_t* num_groups);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */

// Paged single-query decode attention for gfx950 (MI355X).
//
// What is computed: per sequence, query head and its KV head, softmax attention of
// the one decode query over the sequence's cached tokens.  Paging does not change
// this math (zhichai.net page, Key points, "Engineering insight"); the kernel only
// follows each sequence's block table to find the scattered blocks, 16 tokens each by
// default (zhichai.net page, "Why it matters"; "Stop Wasting GPU Memory" page, Technical
// Details, "Core Architecture").  Softmax is taken online, block by block, as in the
// FlashAttention kernels the ml-canon page's "Connections" section says vLLM uses.
//
// Work decomposition.  A context is split into partitions of P tokens; a workgroup's
// waves take a partition's blocks in turn.  Each wave keeps a running max, sum and
// unnormalised output per query head; the waves merge through LDS.  The main (split)
// kernel runs one workgroup per resident slot over a balanced run of partitions and
// merges contexts that span several runs in the same launch (the last run to finish
// merges them with the log-sum-exp rule).  The per-partition kernels for the other
// shapes write each partition's (max, sum, normalised output) to the workspace and a
// second kernel merges them.
//
// bf16/fp16 fast path (MFMA).  All g = H_q / H_kv query heads of a KV head share
// each K/V block, so a 16-token tile is one dense contraction on the matrix cores:
//   S^T[16 tokens x 16 heads] = K[16 x D] . Q^T[D x 16]     (D/32 v_mfma_f32_16x16x32)
//   O^T[D x 16 heads]        += V^T[D x 16] . P^T[16 x 16]  (D/16 v_mfma_f32_16x16x32)
// Query heads beyond g are zero columns.  The lane that holds S for (head, 4 tokens)
// after the first product is exactly the lane that must supply P for them in the
// second, so scores never leave registers.  P is split as P_hi + P_lo, both in the
// input's 16-bit type, and one PV MFMA contracts over (token, half) pairs, so the
// probabilities enter with ~16 significant bits instead of 8 while V and the accumulation
// stay exact fp32.  Blocks of 32 or more tokens (plain mode) take 32 tokens per step with
// 16x16x32 PV MFMAs per half; 8-token blocks are taken two to a 16-token tile.
// The cache layout makes every load a contiguous run per instruction: K is stored in
// 16-byte chunks [D/8][B tokens][8], so the 64 lanes of one QK operand load read 16
// tokens of 4 chunks; V is stored transposed [D][B tokens], so a PV operand load reads
// 16 dims x 16 tokens.
//
// fp32 (and any shape outside the fast path): a plain VALU kernel, one wavefront per
// (partition, query head, sequence).
#include <math.h>

#include <algorithm>
#include <cmath>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <map>
#include <mutex>
#include <utility>

#include <hip/hip_ext.h>

#include "pa_device.h"
#include "pa_mfma.h"
#include "pa_status.h"

namespace pa {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* part_o;   // normalised partial outputs: [S][H_q][max_parts][D] (per-partition kernels) or per run (split)
  float* part_ml;  // (max in log2 units, sum) of each partial: [S][H_q][max_parts][2] or per run (split)
  float scale_log2;
  int32_t num_seqs;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t head_dim;
  int32_t max_blocks;   // block-table row stride
  int32_t ctx_limit;    // min(max_context_len, max_blocks * block_tokens)
  int32_t part_blocks;  // blocks per partition
  int32_t block_tokens; // tokens per block (16 on the MFMA paths)
  int32_t max_parts;
  int32_t out_f32;
  int64_t num_blocks;
  int32_t run_grid;   // split: chunks (workgroups) of the main kernel; 0 = one run per partition
  int32_t run_rounds; // split: rounds of the chunk schedule
  int32_t part_cost;  // split: balance weight of a partition beyond its blocks, in blocks
  int32_t ctx_cost;   // split: balance weight of a (sequence, KV head) context's end, in blocks
  uint64_t* run_done; // split: per (sequence, KV head) arrival counters [S * H_kv] (workspace); tag << 32 | partitions
  uint32_t launch_tag; // split: this launch's counter tag
  // Groups of sequences sharing leading blocks (split kernel only): [num_groups][3] = first
  // sequence, members, prefix blocks; the groups cover the batch in order.  Null with num_groups =
  // num_seqs: every sequence is a group of its own (more than 16 query heads per KV head).
  const int32_t* share_groups;
  int32_t num_groups;
  // split: query columns per partial slot.  The split kernel's partials are indexed by run: run k writes
  // at most two, [k][slot][column][D] (and [k][slot][column][2]), slot 0 for the run's last segment and
  // slot 1 for its first segment when another context follows it in the run.
  int32_t part_cols;
  // split: log2 of the 16-token tiles per cache block (block_tokens = 16 << sub_log2), or -1 for
  // 8-token blocks, two to a tile; the split kernel counts blocks and partitions (part_blocks) in
  // 16-token tiles.
  int32_t sub_log2;
};

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int s) {
  const int n = a.context_lens[s];
  return n < 0 ? 0 : (n > a.ctx_limit ? a.ctx_limit : n);
}

__device__ __forceinline__ int num_parts(int n, int part_blocks, int block_tokens) {
  const int pt = part_blocks * block_tokens;
  const int p = (n + pt - 1) / pt;
  return p < 1 ? 1 : p;
}

template <int DT>
__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t idx, float val) {
  if (a.out_f32) {
    static_cast<float*>(a.out)[idx] = val;
  } else {
    static_cast<typename Elem<DT>::storage*>(a.out)[idx] = Elem<DT>::from_float(val);
  }
}

// Four consecutive outputs (16-byte aligned for fp32, 8-byte for 16-bit types).
template <int DT>
__device__ __forceinline__ void store_out4(const DecodeArgs& a, int64_t idx, const f32x4_t& v) {
  if (a.out_f32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + idx) = v;
  } else {
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = Elem<DT>::from_float(v[e]);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + idx) = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
}

// ------------------------------------------------------------------ MFMA fast path

constexpr int kWaves = 4;
constexpr int kRing = 2;                // register sets per wave (blocks in flight + 1)

// One workgroup = kWaves wavefronts per (partition, KV head, sequence).  Each wave walks
// its blocks with a ring of NBUF register sets: block i+NBUF-1 is being fetched while
// block i computes.  Every (block, KV head) tile is read through a buffer resource
// covering exactly that tile; a slot of the ring past the wave's last block, or a block
// id outside the pool, gets an empty resource, whose loads return zeros and touch no
// memory.  So each iteration issues the same loads, and the compiler's wait counts
// cover exactly the block about to be used.
template <int DT, int D, int NBUF>
__global__ __launch_bounds__(kWaves * kWave) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;
  constexpr int NV = D / 16;
  constexpr int kTileBytes = D * kBlockTokens * 2;
  __shared__ float sm_o[kWaves][16][D];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];

  const int wg = blockIdx.x;
  const int p = wg % a.max_parts;
  const int rest = wg / a.max_parts;
  const int h = rest % a.hkv;
  const int s = rest / a.hkv;
  const int n = clamp_ctx(a, s);
  const int nparts = num_parts(n, a.part_blocks, kBlockTokens);
  if (p >= nparts) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform by construction
  const int col = lane & 15;  // MFMA row/column index of this lane
  const int grp = lane >> 4;  // MFMA k-group of this lane
  const int g = a.group;

  if (n == 0) {  // empty context: out = 0 (nparts == 1 here)
    for (int i = tid; i < g * D; i += kWaves * kWave) {
      const int c = i / D, d = i % D;
      store_out<DT>(a, (static_cast<int64_t>(s) * a.hq + h * g + c) * D + d, 0.0f);
    }
    return;
  }

  const int nblk = (n + kBlockTokens - 1) / kBlockTokens;
  const int b0 = p * a.part_blocks;
  const int b1 = min(nblk, b0 + a.part_blocks);
  const int my_n = (b1 - b0 > w) ? (b1 - b0 - w + kWaves - 1) / kWaves : 0;  // <= 16

  // Physical ids of this wave's blocks b0 + w + 4 i, one per lane; -1 past the last.
  int32_t my_id = -1;
  if (lane < my_n) my_id = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + b0 + w + kWaves * lane];

  // Q^T operand: lane (column = head col, k-group grp) holds dims (kk*4 + grp)*8 .. +8.
  using st = uint16_t;
  const st* q = static_cast<const st*>(a.q);
  u32x4_t qop[KK];
  {
    const bool real = col < g;
    const int64_t qrow = (static_cast<int64_t>(s) * a.hq + h * g + (real ? col : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(q + qrow + (kk * 4 + grp) * 8);
      qop[kk] = real ? x : u32x4_t{0, 0, 0, 0};
    }
  }

  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + static_cast<int64_t>(h) * kTileBytes;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + static_cast<int64_t>(h) * kTileBytes;
  const int64_t blk_stride = static_cast<int64_t>(a.hkv) * kTileBytes;
  // K tile [D/8][16 tokens][8]: lane reads 16 B at lane*16 (+1 KiB per QK MFMA).
  // V tile [D][16 tokens]: lane reads tokens grp*4..+3 of dim col (+16 dims per PV MFMA).
  const int k_off = lane * 16;
  const int v_off = col * 32 + grp * 8;

  auto load = [&](KVRegs<D>& r, int i) {
    const int32_t phys = __builtin_amdgcn_readlane(my_id, i < 63 ? i : 63);
    const bool ok = i < my_n && phys >= 0 && phys < a.num_blocks;
    const int64_t off = ok ? static_cast<int64_t>(phys) * blk_stride : 0;
    const int nrec = ok ? kTileBytes : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kbase + off), 0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vbase + off), 0, nrec, kRsrcWord3);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      r.k[kk] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off, kk * 1024, kLoadNT));
#pragma unroll
    for (int nn = 0; nn < NV; ++nn)
      r.v[nn] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off, nn * 512, kLoadNT));
  };

  f32x4_t o[NV];
#pragma unroll
  for (int nn = 0; nn < NV; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float l = 0.f;

  // Branch-free: a block whose id is out of range counts as empty (nv = 0), and the
  // masking below then leaves m, l and o unchanged.
  auto compute = [&](const KVRegs<D>& r, int i) {
    const int bl = b0 + w + kWaves * i;
    const int32_t phys = __builtin_amdgcn_readlane(my_id, i);
    int nv = n - bl * kBlockTokens;
    nv = nv > kBlockTokens ? kBlockTokens : nv;
    if (phys < 0 || phys >= a.num_blocks) nv = 0;

    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sacc = mfma_qk<DT>(r.k[kk], qop[kk], sacc);

    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (grp * 4 + e < nv) ? sacc[e] * a.scale_log2 : -INFINITY;
    const float bm = rows4_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float m_new = fmaxf(m, bm);
    const float alpha = (m == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = (x[e] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[e] - m_new);
    l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = m_new;
    u32x2_t p_hi, p_lo;
    PSplit<DT>::split(pr, p_hi, p_lo);

    // Absent tokens' V may hold anything, even NaN: select them out (P is 0 there too).
    uint32_t keep[2];
#pragma unroll
    for (int wd = 0; wd < 2; ++wd) {
      const int t0 = grp * 4 + 2 * wd;
      keep[wd] = (t0 < nv ? 0x0000ffffu : 0u) | (t0 + 1 < nv ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) {
      const u32x2_t vv = {r.v[nn][0] & keep[0], r.v[nn][1] & keep[1]};
      o[nn] *= alpha;
      o[nn] = mfma_pv<DT>(vv, p_hi, o[nn]);
      o[nn] = mfma_pv<DT>(vv, p_lo, o[nn]);
    }
  };

  KVRegs<D> ring[NBUF];
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) load(ring[j], j);
  for (int i0 = 0; i0 < my_n; i0 += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (i0 + j >= my_n) break;
      load(ring[(j + NBUF - 1) % NBUF], i0 + j + NBUF - 1);
      compute(ring[j], i0 + j);
    }
  }

  // Per-wave totals: the sum over the four k-groups of this head column.
  l = rows4_sum(l);
  if (grp == 0) {
    sm_m[w][col] = m;
    sm_l[w][col] = l;
  }
#pragma unroll
  for (int nn = 0; nn < NV; ++nn)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_o[w][col][nn * 16 + grp * 4 + e] = o[nn][e];
  __syncthreads();

  // Merge the four waves; thread i covers (head c, dim d) pairs.
  const bool single = nparts == 1;
  for (int i = tid; i < g * D; i += kWaves * kWave) {
    const int c = i / D, d = i % D;
    float mx = sm_m[0][c];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mx = fmaxf(mx, sm_m[ww][c]);
    float L = 0.f, O = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float e = __builtin_amdgcn_exp2f(sm_m[ww][c] - mx);
        L += e * sm_l[ww][c];
        O += e * sm_o[ww][c][d];
      }
    }
    const float res = L > 0.f ? O / L : 0.f;
    const int64_t row = static_cast<int64_t>(s) * a.hq + h * g + c;
    if (single) {
      store_out<DT>(a, row * D + d, res);
    } else {
      const int64_t prow = row * a.max_parts + p;
      a.part_o[prow * D + d] = res;
      if (d == 0) {
        a.part_ml[prow * 2] = mx;
        a.part_ml[prow * 2 + 1] = L;
      }
    }
  }
}

// ------------------------------------------------------------------ split MFMA path

constexpr float kLazyLog2 = 8.0f;  // how far (log2 units) a score may exceed the softmax reference point
constexpr int kMaxScanSeqs = PA_MAX_GROUPED_SEQS;  // sequences the split kernel's in-LDS index covers
constexpr int kPersistRing = 2;     // ring depth of the split kernel
constexpr int kXcds = 8;            // accelerator complex dies of an MI355X, each with its own L2
constexpr int kMaxRuns = 1024;      // chunks (workgroups, runs) of the split kernel, at most
constexpr int kMaxCols = 32;        // query columns of a context in the split kernel (two 16-column tiles)

// Modes of the split kernel.  kPlain: one context per sequence.  kGroup: one context per group of
// consecutive sequences whose block tables share their first k blocks (forked samples or beams of
// one prompt).  A group's query columns are its (member, query head of the KV head) pairs, and its
// context is the shared blocks (read through the first member's table) followed by each member's
// own blocks k .. in member order.  Scores of a member's own block count only in that member's
// columns (the others see -inf there), so every column's online softmax runs over exactly its
// sequence's tokens, and each shared block is read once for all members.  A group has up to 32
// query columns: two 16-column MFMA tiles that share every K/V block's registers.
constexpr int kPlain = 0;
constexpr int kGroup = 1;

// Work split.  The partitions of all (sequence, KV head) pairs are laid end to end in
// (sequence, KV head, partition) order, each weighted by its block count plus a fixed cost
// per partition (its query and table loads, the ring's minimum depth, the segment's merge
// and stores, which blocks alone do not account for); W is the total.
// The split cuts [0, W) into chunks of decreasing size: NR rounds of R chunks (R = the
// workgroups resident at once), round r covering [W - W/2^r, W - W/2^(r+1)) (the last round
// runs to W), so the first chunks take half the work and the last ones fill the tail.  One
// workgroup per chunk owns the partitions whose weighted start lies in the chunk: a contiguous
// run.  Consecutive partitions of one (sequence, KV head) inside a run are merged on chip
// (the online softmax simply continues); only where a run ends inside a sequence's context
// is a partial (max, sum, output) written, to the slot of the run's first partition; the
// run that finishes such a context last merges its runs' partials (chunk_owner finds them).
__device__ __forceinline__ int64_t chunk_lo(int64_t j, int64_t W, int R, int NR) {
  const int r = static_cast<int>(j / R), t = static_cast<int>(j % R);
  if (r >= NR) return W;
  const int64_t T0 = W - (W >> r);
  const int64_t T1 = (r + 1 >= NR) ? W : W - (W >> (r + 1));
  return T0 + (T1 - T0) * t / R;
}
// The chunk whose range holds global block offset off (0 <= off < W).
__device__ __forceinline__ int64_t chunk_owner(int64_t off, int64_t W, int R, int NR) {
  int r = 0;
  while (r + 1 < NR && W - (W >> (r + 1)) <= off) ++r;
  const int64_t T0 = W - (W >> r);
  const int64_t T1 = (r + 1 >= NR) ? W : W - (W >> (r + 1));
  return static_cast<int64_t>(r) * R + ((off - T0 + 1) * R - 1) / (T1 - T0);
}

// Arrival count of one (sequence, KV head): the high 32 bits hold the tag of the launch
// that last wrote it, the low 32 the partitions whose runs have published their partials.
// The workspace is never cleared: a counter still holding another launch's tag counts as 0.
// Returns the partitions published before this call's `add`.
// A run first reads the counter.  If it carries another launch's tag (or garbage), the run
// swaps in (tag, add); exactly one swap per launch succeeds, since the tag never changes back
// within a launch, and a run whose swap fails has re-read the counter and finds the tag there.
// Only then does a run fetch-add, so every add lands on a counter with this launch's tag and a
// count of at most the context's partitions: no add can carry out of the low word into the tag
// (an add on a stale counter whose low word is near 2^32 could forge this launch's tag).
__device__ __forceinline__ uint32_t arrive(uint64_t* ctr, uint32_t tag, uint32_t add) {
  const uint64_t mine = static_cast<uint64_t>(tag) << 32;
  uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((old >> 32) != tag) {
    if (__hip_atomic_compare_exchange_strong(ctr, &old, mine | add, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return 0u;
  }
  old = __hip_atomic_fetch_add(ctr, static_cast<uint64_t>(add), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return static_cast<uint32_t>(old);
}

// One partition of one (sequence, KV head) as a workgroup sees it.
struct Item {
  int32_t s, h, p, n;  // sequence, KV head, partition, context length
  int32_t b0, my_n;    // first block (tile) of the partition; ring positions of this wave
  int32_t np, len;     // partitions of the sequence; blocks in this partition
  int32_t nt;          // column tiles holding query heads (group mode: members * g / 16, rounded up)
};

// Split form of the MFMA kernel: one workgroup per chunk of the schedule above walks its run
// of partitions.  Each wave keeps a ring of NBUF register sets that looks NBUF-1 positions
// ahead across partition boundaries, so the next partition's first blocks are already
// loading while the current one finishes.  The next partition's block ids and query are
// loaded one partition ahead into the other of two slots (A/B), so no loaded value is copied
// before it is used.  Per-block arithmetic is that of decode_mfma_kernel.
// At least two waves per SIMD for head_dim 64 and 128: the compiler keeps the kernel within 256
// VGPRs.  Head_dim 256 (4 wavefronts) runs one wave per SIMD with the accumulators partly in AGPRs:
// twice the bytes per ring slot keep as many bytes in flight per CU.
// Block kinds of the split kernel.  kBk16: 16-token cache blocks, one per ring position.
// kBkMulti: cache blocks of 16 << a.sub_log2 tokens (32, 64, ...), streamed as 16-token tiles:
// tile b of a row is tile b % SB of the row's cache block b / SB (SB = 1 << sub_log2).  kBkHalf:
// 8-token cache blocks (plain mode), two to a 16-token tile: tile b of a row is its cache blocks
// 2b and 2b + 1.  Every count below (blocks, partitions, shared blocks) is in 16-token tiles.
constexpr int kBk16 = 0, kBkMulti = 1, kBkHalf = 2;
template <int DT, int D, int NBUF, int MODE, int WV, int BK>
__global__ __launch_bounds__(WV * kWave) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2))) void decode_split_kernel(
    DecodeArgs a) {
  constexpr int KK = D / 32;
  constexpr int NV = D / 16;
  constexpr int kTileBytes = D * kBlockTokens * 2;  // one 16-token tile of one KV head
  constexpr int kThreads = WV * kWave;
  constexpr int NT = MODE == kGroup ? 2 : 1;  // 16-column MFMA tiles of query columns
  constexpr bool MULTI = BK == kBkMulti;
  constexpr bool HALF = BK == kBkHalf;
  __shared__ __attribute__((aligned(16))) float sm_o[WV][16][D];
  __shared__ float sm_m[WV][16];
  __shared__ float sm_l[WV][16];
  __shared__ int32_t blkpre[kMaxScanSeqs + 1];  // H_kv * (weight of the sequences before s)
  __shared__ int32_t nb_s[kMaxScanSeqs];        // blocks of sequence s
  __shared__ int32_t ctx_s[kMaxScanSeqs];       // clamped context length of sequence s (both modes)
  __shared__ int32_t scan[WV];  // per-wave totals of the prologue's scan
  __shared__ int32_t merge_flag[2];  // thread 0's arrivals completed these contexts
  static_assert(WV * 16 * D > kMaxRuns, "run starts of one context fit in sm_o");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int S = MODE == kGroup ? a.num_groups : a.num_seqs;  // contexts: groups or sequences
  const int PB = a.part_blocks;
  const int hkv = a.hkv;
  const int lsb = MULTI ? a.sub_log2 : 0;  // log2 of the tiles per cache block
  const int sbm = (1 << lsb) - 1;
  // PAIR (plain mode on blocks of 32 or more tokens): a ring position holds 32 tokens, two
  // tiles, so that every V load covers 32 consecutive tokens of each V row (the whole row of a
  // 32-token block) and the PV product runs on 16x16x32 MFMAs; waves take the pairs in turn.
  // Group mode keeps one tile per position and per turn: a member's own tiles need not start on a
  // block boundary of the group's tile sequence.
  constexpr bool PAIR = MULTI && MODE == kPlain;
  constexpr int kUnitTokens = PAIR ? 2 * kBlockTokens : kBlockTokens;  // tokens per ring position
  const int lu = PAIR ? lsb - 1 : lsb;  // log2 of the ring units per cache block
  const int um = (1 << lu) - 1;
  // Unit (from the partition's first) of this wave's ring position i.
  auto unit_of = [&](int i) { return w + WV * i; };
  const int g = a.group;
  const int J = gridDim.x;          // chunks = NR rounds of R
  const int C = a.part_cost;        // fixed cost of a partition, in blocks of streaming
  const int CE = a.ctx_cost;        // fixed cost of a context's end (merge and stores)
  const int PW = PB + C;            // weighted stride of partitions within a context
  // Weight of one (sequence, KV head) context with nb blocks: its blocks, C per partition
  // and CE once, after its last partition.
  auto wnb_of = [&](int nb) { return nb == 0 ? 0 : nb + C * ((nb + PB - 1) / PB) + CE; };
  const int NR = a.run_rounds;
  const int R = J / NR;
  // Chunk k of the split.  Workgroups are dealt to the 8 XCDs round-robin (workgroup i on XCD
  // i % 8); within a round, giving XCD x the chunks [x*R/8, (x+1)*R/8) keeps neighbouring
  // runs (e.g. samples forked from one prompt, which share its blocks) on one XCD and its L2
  // while they run.
  int k = blockIdx.x;
  if (R % kXcds == 0) {
    const int r = k / R, t = k % R;
    k = r * R + (t % kXcds) * (R / kXcds) + t / kXcds;
  }

  // kGroup: group v's first sequence, members and shared blocks, clamped so that every row stays
  // inside the batch, the columns inside the NT 16-wide tiles and the shared blocks inside a table row.
  auto group_first = [&](int v) {
    if (!a.share_groups) return v;
    const int f = a.share_groups[3 * v];
    return f < 0 ? 0 : (f >= a.num_seqs ? a.num_seqs - 1 : f);
  };
  auto group_members = [&](int v, int first) {
    if (!a.share_groups) return 1;
    const int mm = a.share_groups[3 * v + 1];
    return max(1, min(min(mm, a.num_seqs - first), 16 * NT / g));
  };
  // The description counts cache blocks; the context counts tiles.
  auto group_shared = [&](int v) {
    if (!a.share_groups) return 0;
    if constexpr (MULTI) {
      return max(0, min(a.share_groups[3 * v + 2], (a.ctx_limit / kBlockTokens) >> lsb)) << lsb;
    } else if constexpr (HALF) {
      // Whole tiles of shared 8-token blocks; an odd last shared block is read through each member's
      // own row (which holds the same id).
      return max(0, min(a.share_groups[3 * v + 2], min(a.max_blocks, a.ctx_limit / (kBlockTokens / 2)))) >> 1;
    } else {
      return max(0, min(a.share_groups[3 * v + 2], min(a.max_blocks, a.ctx_limit / kBlockTokens)));
    }
  };
  // Blocks of a member with n tokens beyond the k shared ones.
  auto own_blocks = [&](int n, int k) { return max(0, (n + kBlockTokens - 1) / kBlockTokens - k); };
  // Blocks to stream of context s; a group reads its members' lengths from ctx_s.
  auto blocks_of = [&](int s) {
    if constexpr (MODE == kGroup) {
      const int f = group_first(s), mm = group_members(s, f), k = group_shared(s);
      int nb = k;
      for (int j = 0; j < mm; ++j) nb += own_blocks(ctx_s[f + j], k);
      return nb;
    } else {
      return (ctx_s[s] + kBlockTokens - 1) / kBlockTokens;
    }
  };

  // ---- prefix sums of context weights over sequences (every workgroup builds its own copy).
  // Every sequence's clamped length goes to LDS first (one round of global loads), then each
  // thread sizes its contexts once (nb_s) and the second pass reads only LDS.
  for (int s = tid; s < a.num_seqs; s += kThreads) ctx_s[s] = clamp_ctx(a, s);
  __syncthreads();
  const int per = (S + kThreads - 1) / kThreads;
  int cnt = 0;
  for (int j = 0; j < per; ++j) {
    const int s = tid * per + j;
    if (s < S) {
      const int nb = blocks_of(s);
      nb_s[s] = nb;
      cnt += wnb_of(nb);
    }
  }
  // Inclusive scan of the per-thread counts: within each wave by shuffles, then across the
  // four waves through their totals in LDS.
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) scan[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int ww = 0; ww < WV; ++ww) {
    const int t = scan[ww];
    before += ww < w ? t : 0;
    total += t;
  }
  {
    int base = before + incl - cnt;
    for (int j = 0; j < per; ++j) {
      const int s = tid * per + j;
      if (s < S) {
        blkpre[s] = base * hkv;
        base += wnb_of(nb_s[s]);
      }
    }
    if (tid == kThreads - 1) blkpre[S] = total * hkv;
  }
  __syncthreads();
  const int W = __builtin_amdgcn_readfirstlane(blkpre[S]);

  // Zero-length contexts own no partition: their output is 0 (all members' rows for a group).
  for (int s = blockIdx.x; s < S; s += J) {
    if (nb_s[s] == 0) {
      int f = s, mm = 1;
      if constexpr (MODE == kGroup) {
        f = group_first(s);
        mm = group_members(s, f);
      }
      for (int i = tid; i < mm * a.hq * D; i += kThreads)
        store_out<DT>(a, static_cast<int64_t>(f) * a.hq * D + i, 0.0f);
    }
  }
  if (W == 0) return;

  const int64_t lo = chunk_lo(k, W, R, NR);
  const int64_t hi = chunk_lo(k + 1, W, R, NR);
  if (lo >= hi) return;  // an empty chunk (small W): no partition starts in it

  // Sequence holding weighted offset off: the last s with blkpre[s] <= off (that skips
  // zero-length sequences, which share their successor's prefix).
  auto seq_of = [&](int64_t off) {
    int lo_s = 0, hi_s = S - 1;
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(blkpre[mid]) <= off) lo_s = mid; else hi_s = mid - 1;
    }
    return lo_s;
  };

  // One partition (off = the global offset of its first block) and the data loaded for
  // it ahead of time.
  struct Slot {
    Item it;
    bool ok;
    int32_t ids;    // this wave's block ids, one per lane; lanes >= my_n are never used
    // per lane: tile of its cache block << 16 (MULTI), and in kGroup
    // (owning member + 1) << 8 | tokens of the block (owner 0 = shared)
    int32_t meta;
    u32x4_t q[NT][KK];  // Q^T operand of each column tile
  };
  using st = uint16_t;
  const st* qp = static_cast<const st*>(a.q);
  // Decode the partition starting at off and issue the loads of its block ids and query
  // without waiting for them.  The table read is clamped into the row so that it is
  // issued unconditionally; query columns >= g repeat head 0 of the group (their scores
  // only feed their own, discarded, columns).
  // Fill a slot with partition p of (sequence s, KV head h) and issue the loads of its block
  // ids and query without waiting for them.  ok = false gives an empty slot (its loads still
  // go to valid addresses, row 0).
  auto fill = [&](Slot& sl, bool ok, int s, int h, int p) {
    Item& it = sl.it;
    it = Item{0, 0, 0, 0, 0, 0, 1, 0, 1};
    sl.ok = ok;
    if (ok) {
      const int nb = __builtin_amdgcn_readfirstlane(nb_s[s]);
      it.s = s;
      it.h = h;
      it.p = p;
      it.n = MODE == kGroup ? 0 : __builtin_amdgcn_readfirstlane(ctx_s[s]);  // group: per member
      it.np = (nb + PB - 1) / PB;
      it.len = min(PB, nb - p * PB);
      it.b0 = p * PB;
      // This wave's share of the partition's ring units (pairs of tiles in PAIR; only a context's
      // last pair can be half full), dealt to the waves in turn.
      const int lenu = PAIR ? (it.len + 1) >> 1 : it.len;
      it.my_n = (lenu > w) ? (lenu - w + WV - 1) / WV : 0;
    }
    int64_t qrow[NT];
    if constexpr (MODE == kGroup) {
      // This lane's block b of the group's context: shared block b (first member's row) while
      // b < k, else block k + r of the member whose own blocks hold position r = b - k.
      const int first = __builtin_amdgcn_readfirstlane(group_first(it.s));
      const int mm = __builtin_amdgcn_readfirstlane(group_members(it.s, first));
      const int k = __builtin_amdgcn_readfirstlane(group_shared(it.s));
      it.nt = (mm * g + 15) / 16;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int c = t * 16 + col < mm * g ? t * 16 + col : 0;
        qrow[t] = (static_cast<int64_t>(first + c / g) * a.hq + it.h * g + c % g) * D;
      }
      // kBkHalf: lane i and lane 32 + i hold ring position i's two 8-token blocks.
      const int b = it.b0 + w + WV * (HALF ? (lane & 31) : lane);
      int row = first, pos = b, owner = 0, nv = kBlockTokens;
      if (b >= k) {
        int r = b - k;
        for (int j = 0; j < mm; ++j) {
          const int nj = ctx_s[first + j];
          const int oj = own_blocks(nj, k);
          if (r < oj || j == mm - 1) {
            row = first + j;
            pos = k + r;
            owner = j + 1;
            nv = min(kBlockTokens, max(0, nj - pos * kBlockTokens));
            break;
          }
          r -= oj;
        }
      }
      sl.meta = (owner << 8) | nv;
      if constexpr (MULTI) sl.meta |= (pos & sbm) << 16;
      const int tb = HALF ? 2 * max(pos, 0) + (lane >> 5) : max(pos, 0) >> lsb;
      sl.ids = a.block_tables[static_cast<int64_t>(row) * a.max_blocks + min(tb, a.max_blocks - 1)];
    } else {
      qrow[0] = (static_cast<int64_t>(it.s) * a.hq + it.h * g + (col < g ? col : 0)) * D;
      if constexpr (HALF) {
        // Lane i < 32: the first cache block of ring position i's tile; lane 32 + i: its second (a
        // wave holds at most 64 tiles / 4 waves = 16 positions of a partition).
        const int u = it.b0 + unit_of(lane & 31);
        sl.meta = 0;
        sl.ids = a.block_tables[static_cast<int64_t>(it.s) * a.max_blocks + min(2 * u + (lane >> 5), a.max_blocks - 1)];
      } else {
        const int u = (PAIR ? it.b0 >> 1 : it.b0) + unit_of(lane);  // partitions start on a block
        sl.meta = (u & um) << 16;
        sl.ids = a.block_tables[static_cast<int64_t>(it.s) * a.max_blocks + min(u >> lu, a.max_blocks - 1)];
      }
    }
    // Keep the id load ahead of the query loads: the lookahead waits for it while the
    // query loads may still be in flight.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        sl.q[t][kk] = *reinterpret_cast<const u32x4_t*>(qp + qrow[t] + (kk * 4 + grp) * 8);
  };
  // The partition after `cur` in (sequence, KV head, partition) order, at weighted offset
  // off (= cur's offset + its weighted length); empty when off reaches the end of the run.
  auto prepare_next = [&](const Item& cur, int64_t off, Slot& sl) {
    int s = cur.s, h = cur.h, p = cur.p + 1;
    if (p >= cur.np) {
      p = 0;
      if (++h >= hkv) {
        h = 0;
        const bool more = off < hi;  // then a sequence with blocks follows
        do ++s; while (more && s < S && __builtin_amdgcn_readfirstlane(nb_s[s]) == 0);
        if (s >= S) s = 0;
      }
    }
    fill(sl, off < hi, s, h, p);
  };

  const uint8_t* kc = static_cast<const uint8_t*>(a.k);
  const uint8_t* vc = static_cast<const uint8_t*>(a.v);
  // A (cache block, KV head) holds 16 * SB tokens: K as [D/8][16 * SB][8] and V as [D][16 * SB]
  // (SB = 1 without MULTI).  Ring unit t of it (kUnitTokens tokens) starts t * 16 * kUnitTokens
  // bytes into each K row of 8 dims and t * 2 * kUnitTokens bytes into each V row.
  const int head_bytes = HALF ? kTileBytes / 2 : kTileBytes << lsb;
  const int64_t blk_stride = static_cast<int64_t>(hkv) * head_bytes;
  // Per-lane byte offsets: K chunk c = grp of the lane's token (K half h in PAIR), and V dim col
  // at the lane's first token.
  int k_off[PAIR ? 2 : 1];
  if constexpr (PAIR) {
#pragma unroll
    for (int h = 0; h < 2; ++h) k_off[h] = ((grp << (4 + lsb)) + 16 * h + col) * 16;
  } else {
    k_off[0] = MULTI ? ((grp << (4 + lsb)) + col) * 16 : lane * 16;
  }
  const int v_off = ((col * 32) << lsb) + grp * (PAIR ? 16 : 8);
  // A V row of a block of several units spans them all: its cache lines are left to the default
  // policy, so that the units after the first find them in L2.
  constexpr int kLoadV = MULTI ? 0 : kLoadNT;
  using Regs = std::conditional_t<PAIR, KVPairRegs<D>, KVRegs<D>>;
  // phys = the block id of ring position i of a partition with my_n positions for this wave;
  // t = the unit of that block.
  auto load_tile = [&](Regs& r, int32_t phys, int t, int i, int my_n, int h) {
    const bool ok = i < my_n && phys >= 0 && phys < a.num_blocks;
    const int64_t off = ok ? static_cast<int64_t>(phys) * blk_stride + static_cast<int64_t>(h) * head_bytes : 0;
    const int tk = ok ? t * 16 * kUnitTokens : 0, tv = ok ? t * 2 * kUnitTokens : 0;
    const int nrec = ok ? head_bytes : 0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kc + off + tk), 0,
                                                                        nrec - tk, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vc + off + tv), 0,
                                                                        nrec - tv, kRsrcWord3);
    if constexpr (PAIR) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          r.k[hh][kk] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[hh], (kk * 1024) << lsb, kLoadNT));
#pragma unroll
      for (int nn = 0; nn < NV; ++nn)
        r.v[nn] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off, (nn * 512) << lsb, kLoadV));
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        r.k[kk] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[0], (kk * 1024) << lsb, kLoadNT));
#pragma unroll
      for (int nn = 0; nn < NV; ++nn)
        r.v[nn] = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off, (nn * 512) << lsb, kLoadV));
    }
  };
  // kBkHalf: the tile of ring position i is cache blocks p0 (tokens 0-7) and p1 (tokens 8-15), each
  // [D/8][8][8] for K and [D][8] for V.  A lane's K row (token col) and its V tokens (4 grp .. 4 grp + 3)
  // lie in one of the two, so every lane reads through its own address: one load per K chunk and V
  // group as with 16-token blocks.  A block outside the pool or past the partition reads the first
  // tile of the cache instead (in bounds); its tokens are masked where they are used.
  auto load_half = [&](KVRegs<D>& r, int32_t p0, int32_t p1, int i, int my_n, int h) {
    const bool ok0 = i < my_n && p0 >= 0 && p0 < a.num_blocks;
    const bool ok1 = i < my_n && p1 >= 0 && p1 < a.num_blocks;
    const int64_t hb = static_cast<int64_t>(h) * head_bytes;
    const int64_t o0 = ok0 ? static_cast<int64_t>(p0) * blk_stride + hb : 0;
    const int64_t o1 = ok1 ? static_cast<int64_t>(p1) * blk_stride + hb : 0;
    const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(kc + (col < 8 ? o0 : o1) + grp * 128 + (col & 7) * 16);
    const u32x2_t* vp = reinterpret_cast<const u32x2_t*>(vc + (grp < 2 ? o0 : o1) + col * 16 + (grp & 1) * 8);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) r.k[kk] = __builtin_nontemporal_load(kp + kk * 32);
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) r.v[nn] = __builtin_nontemporal_load(vp + nn * 32);
  };
  // Ring position i's loads: ids0 / ids1 hold the tile's (first, second) cache block (kBkHalf) or ids0
  // the block and t its tile or unit (the other kinds).
  auto load_pos = [&](Regs& r, int32_t ids0, int32_t ids1, int t, int i, int my_n, int h) {
    if constexpr (HALF) load_half(r, ids0, ids1, i, my_n, h);
    else load_tile(r, ids0, t, i, my_n, h);
  };
  // Ring positions per partition: a multiple of NBUF, at least NBUF; those past my_n are empty.
  auto steps_of = [&](const Item& it) { return max(NBUF, (it.my_n + NBUF - 1) / NBUF * NBUF); };

  Regs ring[NBUF];
  f32x4_t o[NT][NV];
  float m[NT], l[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
  }
  int seg_p0 = 0;     // first partition of the current (sequence, KV head) segment
  int wave_turn = 0;  // which wave writes the next segment's results
  int npend = 0;      // partial segments written (at most 2: the run's first and last)
  int pend0_s = 0, pend0_h = 0, pend0_c = 0, pend0_np = 0;
  int pend1_s = 0, pend1_h = 0, pend1_c = 0, pend1_np = 0;

  // Merge the partials of all runs of (sequence s, KV head h) and write its g outputs, with
  // the whole workgroup: the runs' first partitions go to LDS (the partial of a run sits at
  // the slot of its first partition), then each thread takes 4 dims of one query head and
  // loads the runs' partials 16 at a time.  Partials are read with device-scope loads: runs on
  // other XCDs wrote them through to memory.  Called by every thread, after the stream.
  int32_t* const run_p0 = reinterpret_cast<int32_t*>(&sm_o[0][0][0]);
  // Query columns of context s (first = its group's first sequence in group mode), and the
  // q / out row of column cc with KV head h.
  auto ncols = [&](int s, int first) {
    if constexpr (MODE == kGroup) return group_members(s, first) * g;
    else return g;
  };
  auto out_row = [&](int s, int h, int cc, int first) -> int64_t {
    if constexpr (MODE == kGroup) return static_cast<int64_t>(first + cc / g) * a.hq + h * g + cc % g;
    else return static_cast<int64_t>(s) * a.hq + h * g + cc;
  };
  auto merge_ctx = [&](int s, int h, int np, int nb) {
    const int64_t A = static_cast<int64_t>(blkpre[s]) + static_cast<int64_t>(h) * wnb_of(nb);
    const int64_t k0 = chunk_owner(A, W, R, NR);
    const int64_t k1 = chunk_owner(A + static_cast<int64_t>(np - 1) * PW, W, R, NR);
    const int nr = static_cast<int>(k1 - k0 + 1);
    // Runs k0 .. k1 - 1 end inside this context: it is their last segment (slot 0).  Run k1 starts inside it
    // and holds it as its first segment, in slot 1 when the next context's first partition (at weighted offset
    // A + wnb_of(nb)) also starts in run k1, else in slot 0.
    const int last_slot = A + wnb_of(nb) < chunk_lo(k1 + 1, W, R, NR) ? 1 : 0;
    for (int i = tid; i <= nr; i += kThreads)
      run_p0[i] = i == 0 ? 0 : i == nr ? np : static_cast<int>((chunk_lo(k0 + i, W, R, NR) - A + PW - 1) / PW);
    __syncthreads();
    constexpr int kChunks = D / 4;
    constexpr int kBatch = 16;
    const int first = MODE == kGroup ? group_first(s) : s;
    for (int c4 = tid; c4 < ncols(s, first) * kChunks; c4 += kThreads) {
      const int cc = c4 / kChunks, d0 = (c4 % kChunks) * 4;
      const int64_t row = out_row(s, h, cc, first);
      float M = -INFINITY, Lsum = 0.f;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int r0 = 0; r0 < nr; r0 += kBatch) {
        float pm[kBatch], pl[kBatch];
        f32x4_t po[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int r = r0 + j;
          const int p0 = r < nr ? run_p0[r] : 0;
          const bool ok = r < nr && p0 < run_p0[r + 1];  // a run may hold no partition start
          pm[j] = -INFINITY;
          pl[j] = 0.f;
          po[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (ok) {
            const int64_t prow = ((k0 + r) * 2 + (r == nr - 1 ? last_slot : 0)) * a.part_cols + cc;
            pm[j] = __hip_atomic_load(a.part_ml + prow * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pl[j] = __hip_atomic_load(a.part_ml + prow * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              po[j][e] = __hip_atomic_load(a.part_o + prow * D + d0 + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (pl[j] > 0.f) {
            const float Mn = fmaxf(M, pm[j]);
            const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
            const float wr = __builtin_amdgcn_exp2f(pm[j] - Mn) * pl[j];
            acc = acc * sc + po[j] * wr;
            Lsum = Lsum * sc + wr;
            M = Mn;
          }
        }
      }
      f32x4_t res;
#pragma unroll
      for (int e = 0; e < 4; ++e) res[e] = Lsum > 0.f ? acc[e] / Lsum : 0.f;
      store_out4<DT>(a, row * D + d0, res);
    }
    __syncthreads();  // run_p0 is reused by the next merge
  };

  // Stream one partition's blocks (looking ahead into the next one).  At the end of a
  // segment, merge the four waves and write the output or the run's partial.
  auto run = [&](const Item cur, const int32_t cur_ids, const int32_t cur_meta, const u32x4_t (&qc)[NT][KK],
                 const Item nxi, const bool nx_ok, const int32_t nx_ids, const int32_t nx_meta) {
    // m is a reference point, not the running maximum: the weights exp2(x - m) of any m give the
    // same softmax once divided by their sum.  It moves (and l and O are rescaled) only when a score
    // of some column of the wave exceeds it by more than kLazyLog2, so weights stay below
    // 2^kLazyLog2 and most tiles leave O alone.  A column that has seen no token has m = -inf and
    // moves at its first visible token.
    auto lazy_rescale = [&](int t, float bm) {
      if (__builtin_amdgcn_ballot_w64(bm > m[t] + kLazyLog2) != 0) {
        const float m_new = fmaxf(m[t], bm);
        const float alpha = (m[t] == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m[t] - m_new);
        l[t] *= alpha;
#pragma unroll
        for (int nn = 0; nn < NV; ++nn) o[t][nn] *= alpha;
        m[t] = m_new;
      }
    };
    // PAIR: one 32-token unit.  Scores of the two K halves, one softmax update over the 32
    // tokens, and O^T += V^T P^T as 16x16x32 MFMAs (lane group j holds tokens 8 j .. 8 j + 7 of
    // both V and P).
    auto compute_pair = [&](KVPairRegs<D>& r, int i) {
      const int32_t phys = __builtin_amdgcn_readlane(cur_ids, i < 63 ? i : 63);
      int nv = cur.n - ((cur.b0 >> 1) + unit_of(i)) * kUnitTokens;  // tokens of the unit
      nv = nv > kUnitTokens ? kUnitTokens : nv;
      if (i >= cur.my_n || phys < 0 || phys >= a.num_blocks) nv = 0;
      f32x4_t sacc[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        sacc[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sacc[hh] = mfma_qk<DT>(r.k[hh][kk], qc[0][kk], sacc[hh]);
      }
      // Half h's score tile holds token 16 h + 4 grp + e of the unit in lane (col, grp), element e; the PV
      // operand wants tokens 8 grp .. 8 grp + 7 in lane group grp.  Two permlane swaps move them there:
      // lane groups 2, 3 of half 0 with groups 0, 1 of half 1, then the odd groups' first four with
      // the even groups' last four.
      float x[8];  // token 8 grp + j of the unit
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sacc[0][e]), __float_as_uint(sacc[1][e]),
                                                          false, false);
        const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
        x[e] = __uint_as_float(s16[0]);
        x[4 + e] = __uint_as_float(s16[1]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (grp * 8 + j < nv) ? x[j] * a.scale_log2 : -INFINITY;
      const float bm = rows4_max(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
      lazy_rescale(0, bm);
      float pr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pr[j] = (x[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[j] - m[0]);
      l[0] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      u32x2_t h0, l0, h1, l1;
      PSplit<DT>::split(pr, h0, l0);
      PSplit<DT>::split(pr + 4, h1, l1);
      const u32x4_t p_hi = {h0[0], h0[1], h1[0], h1[1]}, p_lo = {l0[0], l0[1], l1[0], l1[1]};
      if (nv < kUnitTokens) {  // tokens past the context: selected out of V in place
        uint32_t keep[4];
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const int t0 = grp * 8 + 2 * wd;
          keep[wd] = (t0 < nv ? 0x0000ffffu : 0u) | (t0 + 1 < nv ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int nn = 0; nn < NV; ++nn)
          r.v[nn] = u32x4_t{r.v[nn][0] & keep[0], r.v[nn][1] & keep[1], r.v[nn][2] & keep[2], r.v[nn][3] & keep[3]};
      }
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
        o[0][nn] = mfma_qk<DT>(r.v[nn], p_hi, o[0][nn]);
        o[0][nn] = mfma_qk<DT>(r.v[nn], p_lo, o[0][nn]);
      }
    };
    auto compute_tile = [&](KVRegs<D>& r, int i) {
      constexpr int kLastPos = HALF ? 31 : 63;  // lanes of cur_ids holding a position's (first) block
      const int32_t phys = __builtin_amdgcn_readlane(cur_ids, i < kLastPos ? i : kLastPos);
      int nv;          // tokens of the tile in the context (0: nothing to add)
      int owner = 0;   // kGroup: 0 for a shared tile, else 1 + the member whose own tile it is
      if constexpr (MODE == kGroup) {
        const int meta = __builtin_amdgcn_readlane(cur_meta, i < kLastPos ? i : kLastPos);
        nv = meta & 0xff;
        owner = MULTI ? (meta >> 8) & 0xff : meta >> 8;
      } else {
        const int bl = cur.b0 + unit_of(i);
        nv = cur.n - bl * kBlockTokens;
        nv = nv > kBlockTokens ? kBlockTokens : nv;
      }
      if (i >= cur.my_n) nv = 0;
      // The tokens this lane's K row and V tokens see: an id outside the pool leaves its block's
      // tokens out (kBkHalf: this lane's tokens lie in block grp >> 1 of the tile).  vmask: some lane
      // has tokens to clear from its V registers (uniform).
      int nv_lane = nv;
      bool vmask = nv < kBlockTokens;
      if constexpr (HALF) {
        const int32_t p1 = __builtin_amdgcn_readlane(cur_ids, (i < 31 ? i : 31) + 32);
        const bool ok0 = phys >= 0 && phys < a.num_blocks, ok1 = p1 >= 0 && p1 < a.num_blocks;
        nv_lane = (grp < 2 ? ok0 : ok1) ? nv : 0;
        vmask = vmask || !ok0 || !ok1;
      } else {
        if (phys < 0 || phys >= a.num_blocks) nv_lane = nv = 0;
        vmask = nv < kBlockTokens;
      }
      int nv_col[NT];  // tokens of the tile this lane's query column sees, per column tile
      int t_lo = 0, t_hi = NT - 1;  // column tiles to compute (wave-uniform)
      if constexpr (MODE == kGroup) {
#pragma unroll
        for (int t = 0; t < NT; ++t) nv_col[t] = (owner == 0 || owner - 1 == (t * 16 + col) / g) ? nv_lane : 0;
        // Column tiles with no column that sees the tile (a member's own tile is seen by its g
        // columns only; tiles past the group's columns hold none) would add exact zeros: skipped.
        t_lo = owner == 0 ? 0 : ((owner - 1) * g) / 16;
        t_hi = owner == 0 ? cur.nt - 1 : ((owner - 1) * g + g - 1) / 16;
      } else {
        nv_col[0] = nv_lane;
      }

      u32x2_t p_hi[NT], p_lo[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (NT > 1 && (t < t_lo || t > t_hi)) continue;
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sacc = mfma_qk<DT>(r.k[kk], qc[t][kk], sacc);

        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (grp * 4 + e < nv_col[t]) ? sacc[e] * a.scale_log2 : -INFINITY;
        const float bm = rows4_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        lazy_rescale(t, bm);
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = (x[e] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[e] - m[t]);
        l[t] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        PSplit<DT>::split(pr, p_hi[t], p_lo[t]);
      }
      // O^T += V^T P^T.  Tokens past the context may hold anything, even NaN: a block that is
      // not full has them selected out of its V registers (in place: the ring reloads them next);
      // a full block (all but a context's last) needs no mask.
      if (vmask) {
        const int nvl = nv_lane;
        uint32_t keep[2];
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
          const int t0 = grp * 4 + 2 * wd;
          keep[wd] = (t0 < nvl ? 0x0000ffffu : 0u) | (t0 + 1 < nvl ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int nn = 0; nn < NV; ++nn) r.v[nn] = u32x2_t{r.v[nn][0] & keep[0], r.v[nn][1] & keep[1]};
      }
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (NT > 1 && (t < t_lo || t > t_hi)) continue;
          o[t][nn] = mfma_pv_split<DT>(r.v[nn], p_hi[t], p_lo[t], o[t][nn]);
        }
      }
    };
    auto compute = [&](Regs& r, int i) {
      if constexpr (PAIR) compute_pair(r, i);
      else compute_tile(r, i);
    };

    const int steps = steps_of(cur);
    const int nx_my_n = nx_ok ? nxi.my_n : 0;
    for (int i = 0; i < steps; i += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        // Ring lookahead position; past this partition's last step it is the next one's.
        int la = i + j + NBUF - 1;
        int32_t phys, phys1 = 0;
        int tile = 0;
        int mn = cur.my_n, hh = cur.h;
        if (la >= steps) {
          // The next partition's ids were loaded after this one's first blocks.  Reading
          // them only here (the empty asm keeps the read inside the branch) keeps every
          // other wait of the loop counting only ring loads.
          int32_t t = nx_ids;
          asm volatile("" : "+v"(t));
          la -= steps;
          if constexpr (HALF) {
            phys = __builtin_amdgcn_readlane(t, la < 31 ? la : 31);
            phys1 = __builtin_amdgcn_readlane(t, (la < 31 ? la : 31) + 32);
          } else {
            phys = __builtin_amdgcn_readlane(t, la < 63 ? la : 63);
          }
          if constexpr (MULTI) {
            int32_t tm = nx_meta;
            asm volatile("" : "+v"(tm));
            tile = __builtin_amdgcn_readlane(tm, la < 63 ? la : 63) >> 16;
          }
          mn = nx_my_n;
          hh = nxi.h;
        } else if constexpr (HALF) {
          phys = __builtin_amdgcn_readlane(cur_ids, la < 31 ? la : 31);
          phys1 = __builtin_amdgcn_readlane(cur_ids, (la < 31 ? la : 31) + 32);
        } else {
          phys = __builtin_amdgcn_readlane(cur_ids, la < 63 ? la : 63);
          if constexpr (MULTI) tile = __builtin_amdgcn_readlane(cur_meta, la < 63 ? la : 63) >> 16;
        }
        load_pos(ring[(j + NBUF - 1) % NBUF], phys, phys1, tile, la, mn, hh);
        if (i + j < cur.my_n) compute(ring[j], i + j);  // positions past my_n only pad the ring
      }
    }

    if (nx_ok && nxi.s == cur.s && nxi.h == cur.h) return;  // the segment goes on

    // ---- end of segment: merge the four waves through LDS, one column tile at a time
    const bool final = seg_p0 == 0 && cur.p == cur.np - 1;  // the segment is the whole context
    const int first = MODE == kGroup ? __builtin_amdgcn_readfirstlane(group_first(cur.s)) : cur.s;
    const int ncol = ncols(cur.s, first);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t > 0) __syncthreads();  // the previous tile's merge has read the LDS
      const float lt = rows4_sum(l[t]);
      if (grp == 0) {
        sm_m[w][col] = m[t];
        sm_l[w][col] = lt;
      }
#pragma unroll
      for (int nn = 0; nn < NV; ++nn)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm_o[w][col][nn * 16 + grp * 4 + e] = o[t][nn][e];
      __syncthreads();
      // One wave, rotating per segment, merges and writes; the others go straight on.  The
      // counter of outstanding vector-memory operations also counts stores, so a wave that
      // stores cannot use its later loads before the stores complete.
      if (w == (wave_turn & (WV - 1))) {
        constexpr int kChunks = D / 4;  // 4 consecutive dims per lane and store
        const int tcols = min(16, ncol - t * 16);
        for (int c4 = lane; c4 < tcols * kChunks; c4 += kWave) {
          const int cc = c4 / kChunks, d0 = (c4 % kChunks) * 4;
          float mx = sm_m[0][cc];
#pragma unroll
          for (int ww = 1; ww < WV; ++ww) mx = fmaxf(mx, sm_m[ww][cc]);
          float L = 0.f;
          f32x4_t O = {0.f, 0.f, 0.f, 0.f};
          if (mx != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < WV; ++ww) {
              const float e = __builtin_amdgcn_exp2f(sm_m[ww][cc] - mx);
              L += e * sm_l[ww][cc];
              O += e * *reinterpret_cast<const f32x4_t*>(&sm_o[ww][cc][d0]);
            }
          }
          f32x4_t res;
#pragma unroll
          for (int e = 0; e < 4; ++e) res[e] = L > 0.f ? O[e] / L : 0.f;
          const int64_t row = out_row(cur.s, cur.h, t * 16 + cc, first);
          if (final) {
            store_out4<DT>(a, row * D + d0, res);
          } else {
            // This run's partial of the context: slot 0 if the segment is the run's last, else (the run's
            // first segment, another context following it) slot 1.
            const int64_t prow = (static_cast<int64_t>(k) * 2 + (nx_ok ? 1 : 0)) * a.part_cols + t * 16 + cc;
            // Device-scope stores: the run that merges this context may sit on another XCD.
#pragma unroll
            for (int e = 0; e < 4; ++e)
              __hip_atomic_store(a.part_o + prow * D + d0 + e, res[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d0 == 0) {
              __hip_atomic_store(a.part_ml + prow * 2, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(a.part_ml + prow * 2 + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
    // Only a run's first and last segments can be part of a context; their partials are
    // published once the run is done.
    if (!(seg_p0 == 0 && cur.p == cur.np - 1)) {
      if (npend == 0) {
        pend0_s = cur.s, pend0_h = cur.h, pend0_c = cur.p - seg_p0 + 1, pend0_np = cur.np;
      } else {
        pend1_s = cur.s, pend1_h = cur.h, pend1_c = cur.p - seg_p0 + 1, pend1_np = cur.np;
      }
      ++npend;
    }
    ++wave_turn;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) o[t][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[t] = -INFINITY;
      l[t] = 0.f;
    }
    seg_p0 = nxi.p;
  };

  // First partition: the first one that starts at or after lo (in weighted offsets).
  int64_t off;
  {
    const int s = seq_of(lo);
    const int nb = __builtin_amdgcn_readfirstlane(nb_s[s]);
    const int wn = wnb_of(nb);
    const int r = static_cast<int>(lo - __builtin_amdgcn_readfirstlane(blkpre[s]));
    int h = r / wn, p = (r % wn + PW - 1) / PW;
    if (p >= (nb + PB - 1) / PB) {
      p = 0;
      ++h;
    }
    off = __builtin_amdgcn_readfirstlane(blkpre[s]) + static_cast<int64_t>(h) * wn + static_cast<int64_t>(p) * PW;
  }
  Slot A, B;
  {
    const bool ok = off < hi;
    int s0 = 0, h0 = 0, p0 = 0;
    if (ok) {
      s0 = seq_of(off);
      const int wn = wnb_of(__builtin_amdgcn_readfirstlane(nb_s[s0]));
      const int r = static_cast<int>(off - __builtin_amdgcn_readfirstlane(blkpre[s0]));
      h0 = r / wn;
      p0 = (r % wn) / PW;
    }
    fill(A, ok, s0, h0, p0);
  }
  if (!A.ok) return;  // the run holds no partition start
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) o[t][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  seg_p0 = A.it.p;
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    load_pos(ring[j], __builtin_amdgcn_readlane(A.ids, j), HALF ? __builtin_amdgcn_readlane(A.ids, j + 32) : 0,
             MULTI ? __builtin_amdgcn_readlane(A.meta, j) >> 16 : 0, j, A.it.my_n, A.it.h);
  // Weighted length of a partition: its blocks, C, and CE if it ends its context.
  auto wlen = [&](const Item& it) { return it.len + C + (it.p == it.np - 1 ? CE : 0); };
  off += wlen(A.it);
  prepare_next(A.it, off, B);
  while (true) {
    run(A.it, A.ids, A.meta, A.q, B.it, B.ok, B.ids, B.meta);
    if (!B.ok) break;
    off += wlen(B.it);
    prepare_next(B.it, off, A);
    run(B.it, B.ids, B.meta, B.q, A.it, A.ok, A.ids, A.meta);
    if (!A.ok) break;
    off += wlen(A.it);
    prepare_next(A.it, off, B);
  }

  // Publish the run's partial segments: each adds its partitions to the count of its
  // (sequence, KV head); the run that completes a context merges the partials of all its
  // runs (its own included) and writes the output.  Every wave first waits until its
  // device-scope partial stores are complete, so they are visible to any later device-scope
  // load once the barrier has passed and thread 0 has counted them.
  if (npend == 0) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t b0 = arrive(a.run_done + static_cast<int64_t>(pend0_s) * hkv + pend0_h, a.launch_tag, pend0_c);
    merge_flag[0] = b0 + pend0_c == static_cast<uint32_t>(pend0_np);
    merge_flag[1] = 0;
    if (npend > 1) {
      const uint32_t b1 = arrive(a.run_done + static_cast<int64_t>(pend1_s) * hkv + pend1_h, a.launch_tag, pend1_c);
      merge_flag[1] = b1 + pend1_c == static_cast<uint32_t>(pend1_np);
    }
  }
  __syncthreads();
  if (merge_flag[0]) merge_ctx(pend0_s, pend0_h, pend0_np, nb_s[pend0_s]);
  if (merge_flag[1]) merge_ctx(pend1_s, pend1_h, pend1_np, nb_s[pend1_s]);
}

// ------------------------------------------------------------------ generic VALU path

constexpr int kMaxPartTokens = 1024;
constexpr int kMaxGenericD = 256;
constexpr int kMaxGenericHeads = 8;  // query heads of one KV head that a generic workgroup serves at once

// One wavefront per (partition, KV head, sequence, chunk of at most GH of the KV head's query heads),
// so that every K/V element it reads serves all GH heads of the chunk.  Scores: a lane per token,
// its K row read 16 bytes at a time and dotted with the chunk's queries.  Softmax over the
// partition per head.  Output: a lane per dim, its V row read 16 bytes (several tokens) at a time.
// Blocks whose id is outside the pool count as empty.  LDS (dynamic): scores [GH][partition
// tokens], block ids [partition blocks].
template <int DT, int GH>
__global__ __launch_bounds__(kWave) void decode_generic_kernel(DecodeArgs a) {
  using st = typename Elem<DT>::storage;
  constexpr int X = 16 / sizeof(st);  // elements per 16 bytes
  extern __shared__ float gen_lds[];
  const int D = a.head_dim;
  const int B = a.block_tokens;
  const int g = a.group;
  const int pt = a.part_blocks * B;
  float* sc = gen_lds;
  int32_t* ids = reinterpret_cast<int32_t*>(sc + GH * pt);

  const int nch = (g + GH - 1) / GH;
  int rest = blockIdx.x;
  const int p = rest % a.max_parts;
  rest /= a.max_parts;
  const int hc = rest % nch;
  rest /= nch;
  const int h = rest % a.hkv;
  const int s = rest / a.hkv;
  const int n = clamp_ctx(a, s);
  const int nparts = num_parts(n, a.part_blocks, B);
  if (p >= nparts) return;
  const int lane = threadIdx.x;
  const int j0 = h * g + hc * GH;       // first query head of the chunk
  const int gh = min(GH, g - hc * GH);  // heads in the chunk
  const int64_t row0 = static_cast<int64_t>(s) * a.hq + j0;

  if (n == 0) {
    for (int i = lane; i < gh * D; i += kWave) store_out<DT>(a, (row0 + i / D) * D + i % D, 0.0f);
    return;
  }
  const int t0 = p * pt;
  const int t1 = min(n, t0 + pt);
  const int bl0 = t0 / B;
  const int nb = (t1 - t0 + B - 1) / B;
  for (int b = lane; b < nb; b += kWave) {
    const int32_t id = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + bl0 + b];
    ids[b] = (id >= 0 && id < a.num_blocks) ? id : -1;
  }
  __syncthreads();

  const st* kc = static_cast<const st*>(a.k);
  const st* vc = static_cast<const st*>(a.v);
  const int64_t head_elems = static_cast<int64_t>(D) * B;  // one (block, KV head) tile of K or V
  auto unpack = [](const u32x4_t& raw, float (&f)[X]) {
    if constexpr (X == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(raw[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = Elem<DT>::to_float(static_cast<st>(raw[e] & 0xffffu));
        f[2 * e + 1] = Elem<DT>::to_float(static_cast<st>(raw[e] >> 16));
      }
    }
  };

  // Scores, a lane per token, TPL tokens a lane at a time: K is [D / X][B][X] per tile, so a lane's
  // 16-byte read is X dims of one token.  The queries are the same for every lane: they are read
  // from memory at uniform addresses (scalar loads) chunk by chunk, and each chunk serves the lane's
  // TPL tokens.
  constexpr int TPL = 4;
  const st* __restrict__ qg = static_cast<const st*>(a.q);
  float mx[GH];
#pragma unroll
  for (int jj = 0; jj < GH; ++jj) mx[jj] = -INFINITY;
  for (int tb = t0; tb < t1; tb += kWave * TPL) {
    const st* kb[TPL];
    bool ok[TPL];
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      const int t = tb + u * kWave + lane;
      const int id = t < t1 ? ids[(t - t0) / B] : -1;
      ok[u] = id >= 0;
      // A token outside the partition, or of a block outside the pool, reads the cache's first tile
      // (in bounds) and scores -inf.
      kb[u] = kc + (ok[u] ? (static_cast<int64_t>(id) * a.hkv + h) * head_elems + static_cast<int64_t>(t % B) * X : 0);
    }
    float acc[TPL][GH];
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int jj = 0; jj < GH; ++jj) acc[u][jj] = 0.f;
#pragma unroll 4
    for (int c = 0; c < D / X; ++c) {
      float qf[GH][X];
#pragma unroll
      for (int jj = 0; jj < GH; ++jj)
#pragma unroll
        for (int e = 0; e < X; ++e)
          qf[jj][e] = jj < gh ? Elem<DT>::to_float(qg[(row0 + jj) * D + c * X + e]) : 0.f;
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        float kf[X];
        unpack(*reinterpret_cast<const u32x4_t*>(kb[u] + static_cast<int64_t>(c) * B * X), kf);
#pragma unroll
        for (int jj = 0; jj < GH; ++jj)
#pragma unroll
          for (int e = 0; e < X; ++e) acc[u][jj] = fmaf(qf[jj][e], kf[e], acc[u][jj]);
      }
    }
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      const int t = tb + u * kWave + lane;
      if (t >= t1) continue;
#pragma unroll
      for (int jj = 0; jj < GH; ++jj) {
        const float x = ok[u] ? acc[u][jj] * a.scale_log2 : -INFINITY;
        sc[jj * pt + (t - t0)] = x;
        mx[jj] = fmaxf(mx[jj], x);
      }
    }
  }
  float L[GH];
#pragma unroll
  for (int jj = 0; jj < GH; ++jj) {
    mx[jj] = wave_max(mx[jj]);
    float lsum = 0.f;
    for (int t = t0 + lane; t < t1; t += kWave) {
      const float e = (mx[jj] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[jj * pt + (t - t0)] - mx[jj]);
      sc[jj * pt + (t - t0)] = e;
      lsum += e;
    }
    L[jj] = wave_sum(lsum);
  }
  __syncthreads();

  // Output, a lane per dim: V is [D][B] per tile, so a lane's 16-byte read is X tokens of its dim.
  constexpr int ND = kMaxGenericD / kWave;  // dims per lane, at most
  float acc[GH][ND];
#pragma unroll
  for (int jj = 0; jj < GH; ++jj)
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) acc[jj][dd] = 0.f;
  const bool vec = B % X == 0;
  for (int b = 0; b < nb; ++b) {
    const int id = ids[b];
    if (id < 0) continue;  // uniform: every lane takes the same block
    const st* vb = vc + (static_cast<int64_t>(id) * a.hkv + h) * head_elems;
    const int tb = t0 + b * B;              // first token of the block
    const int tn = min(B, t1 - tb);         // its tokens in the partition
    if (vec) {
#pragma unroll 4
      for (int e0 = 0; e0 < tn; e0 += X) {
#pragma unroll
        for (int dd = 0; dd < ND; ++dd) {
          const int d = lane + dd * kWave;
          if (d >= D) break;
          float vf[X];
          unpack(*reinterpret_cast<const u32x4_t*>(vb + static_cast<int64_t>(d) * B + e0), vf);
#pragma unroll
          for (int e = 0; e < X; ++e) {
            if (e0 + e >= tn) break;  // tokens past the context may hold anything
#pragma unroll
            for (int jj = 0; jj < GH; ++jj) acc[jj][dd] = fmaf(sc[jj * pt + (tb - t0) + e0 + e], vf[e], acc[jj][dd]);
          }
        }
      }
    } else {
      for (int e = 0; e < tn; ++e) {
#pragma unroll
        for (int dd = 0; dd < ND; ++dd) {
          const int d = lane + dd * kWave;
          if (d >= D) break;
          const float v = Elem<DT>::to_float(vb[static_cast<int64_t>(d) * B + e]);
#pragma unroll
          for (int jj = 0; jj < GH; ++jj) acc[jj][dd] = fmaf(sc[jj * pt + (tb - t0) + e], v, acc[jj][dd]);
        }
      }
    }
  }

  const bool single = nparts == 1;
#pragma unroll
  for (int jj = 0; jj < GH; ++jj) {
    if (jj >= gh) break;
    const int64_t row = row0 + jj;
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
      const int d = lane + dd * kWave;
      if (d >= D) break;
      const float res = L[jj] > 0.f ? acc[jj][dd] / L[jj] : 0.f;
      if (single) {
        store_out<DT>(a, row * D + d, res);
      } else {
        const int64_t prow = row * a.max_parts + p;
        a.part_o[prow * D + d] = res;
        if (d == 0) {
          a.part_ml[prow * 2] = mx[jj];
          a.part_ml[prow * 2 + 1] = L[jj];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ partition merge

// One workgroup per (sequence, KV head, column slice) with more than one partition merges
// the partials of that sequence's partitions for its slice of the g query heads x D outputs
// (the per-partition kernels; the split kernel merges its runs itself):
//   M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p * O_p / sum_p w_p
// where O_p is partition p's normalised output.  Threads form RG groups that take every
// RG-th partition, merge online, then combine in a fixed order: deterministic.  Zero-length
// and single-partition sequences were written by the main kernel.
template <int DT>
__global__ __launch_bounds__(256) void reduce_partitions_kernel(DecodeArgs a) {
  __shared__ float red_m[256];
  __shared__ float red_l[256];
  __shared__ __attribute__((aligned(16))) f32x4_t red_o[256];
  const int s = blockIdx.x / a.hkv;
  const int kvh = blockIdx.x % a.hkv;
  const int n = clamp_ctx(a, s);
  if (n == 0) return;
  const int PB = a.part_blocks;
  const int nb = (n + a.block_tokens - 1) / a.block_tokens;
  const int np = (nb + PB - 1) / PB;
  if (np <= 1) return;
  const int D = a.head_dim;
  const int g = a.group;
  const int tid = threadIdx.x;

  const int nout4 = g * D / 4;
  const int C = (nout4 + gridDim.y - 1) / gridDim.y;  // columns per slice, <= 256
  const int c_begin = blockIdx.y * C;
  const int RG = 256 / C;  // run groups
  const int rg = tid / C;
  const int c4 = c_begin + tid % C;
  const bool active = rg < RG && c4 < nout4;
  const int cc = active ? c4 / (D / 4) : 0, d0 = active ? (c4 % (D / 4)) * 4 : 0;
  const int64_t row = static_cast<int64_t>(s) * a.hq + kvh * g + cc;
  float M = -INFINITY, L = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int p = rg; p < np; p += RG) {
      const int64_t prow = row * a.max_parts + p;
      const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(a.part_ml + prow * 2);
      const f32x4_t O = *reinterpret_cast<const f32x4_t*>(a.part_o + prow * D + d0);
      if (!(ml[1] > 0.f)) continue;
      const float Mn = fmaxf(M, ml[0]);
      const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float wr = __builtin_amdgcn_exp2f(ml[0] - Mn) * ml[1];
      acc = acc * sc + O * wr;
      L = L * sc + wr;
      M = Mn;
    }
  }
  if (RG > 1) {
    red_m[tid] = M;
    red_l[tid] = L;
    red_o[tid] = acc;
    __syncthreads();
    if (active && rg == 0) {
      for (int r = 1; r < RG; ++r) {
        const int t = r * C + tid;
        if (!(red_l[t] > 0.f)) continue;
        const float mr = red_m[t];
        const float Mn = fmaxf(M, mr);
        const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        const float sr = __builtin_amdgcn_exp2f(mr - Mn);
        acc = acc * sc + red_o[t] * sr;
        L = L * sc + red_l[t] * sr;
        M = Mn;
      }
    }
  }
  if (active && rg == 0) {
    f32x4_t res;
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = L > 0.f ? acc[e] / L : 0.f;
    store_out4<DT>(a, row * D + d0, res);
  }
}

}  // namespace pa

using namespace pa;

namespace {

// Balance weights beyond the blocks, in blocks of streaming time: per partition its query and
// table loads and the ring's minimum depth; per context the merge through LDS and the output
// stores at its end.  Without them, a workgroup whose chunk holds many short contexts
// finishes last by tens of microseconds.
constexpr int kPartCost = 5;
constexpr int kCtxCost = 5;

// Which kernel serves a call.  kSplit: decode_split_kernel (bf16/fp16, head_dim 64/96/128/256 on blocks of
// 8 or 16 << j tokens, at most 32 query heads per KV head (16 at head_dim 256), one launch per kMaxScanSeqs
// sequences); it merges split contexts itself.  kMfma: decode_mfma_kernel, one workgroup per (partition, KV
// head, sequence), for batches beyond kMaxScanSeqs sequences on 16-token blocks whose contexts each fit one
// partition, and for block tables too wide for the split kernel's int32 tile index.  kGeneric:
// decode_generic_kernel (VALU) for every other shape.  The last two write per-partition partials that
// reduce_partitions_kernel merges.
enum Route : int32_t { kRouteSplit = 0, kRouteMfma = 1, kRouteGeneric = 2 };

struct Plan {
  int32_t part_tokens;
  int32_t part_blocks;
  int32_t ctx_limit;
  int32_t max_parts;      // partitions of the longest context
  Route route;
  int32_t sub_log2;       // kSplit: log2 of the 16-token tiles per cache block; -1: two 8-token blocks per tile
  bool group;             // kSplit: over groups of sequences sharing leading blocks
  int32_t part_cols;      // kSplit: query columns per partial slot
  size_t ml_offset;       // floats from the workspace start to the (max, sum) pairs
  size_t counter_offset;  // bytes from the workspace start to the arrival counters
  size_t workspace;
};

int32_t make_plan(const pa_decode_params* p, Plan* out) {
  if (!p) return PA_ERR_INVALID_ARG;
  const pa_cache_desc& c = p->cache;
  if (p->num_seqs < 0 || p->num_q_heads <= 0 || p->max_blocks_per_seq <= 0 || p->max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (c.num_blocks <= 0 || c.num_kv_heads <= 0 || c.head_dim <= 0 || c.block_size <= 0) return PA_ERR_INVALID_ARG;
  if (p->num_q_heads % c.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!valid_dtype(c.dtype)) return PA_ERR_INVALID_ARG;
  if (p->out_dtype != PA_F32 && p->out_dtype != c.dtype) return PA_ERR_INVALID_ARG;
  if (c.head_dim % (16 / elem_bytes(c.dtype)) != 0) return PA_ERR_INVALID_ARG;
  if (c.head_dim > kMaxGenericD || c.block_size > kMaxPartTokens) return PA_ERR_UNSUPPORTED;
  const int32_t B = c.block_size;
  // 0: 512 tokens, rounded down to whole blocks (at least one block)
  const int32_t pt = p->partition_size == 0 ? std::max(B, 512 / B * B) : p->partition_size;
  if (pt < B || pt > kMaxPartTokens || pt % B != 0) return PA_ERR_INVALID_ARG;
  const int64_t limit64 = std::min<int64_t>(p->max_context_len, int64_t{p->max_blocks_per_seq} * B);
  const int32_t limit = static_cast<int32_t>(std::min<int64_t>(limit64, INT32_MAX));
  const int32_t parts = std::max<int32_t>(1, static_cast<int32_t>((int64_t{limit} + pt - 1) / pt));
  if (parts > 8192) return PA_ERR_UNSUPPORTED;
  out->part_tokens = pt;
  out->part_blocks = pt / B;
  out->ctx_limit = limit;
  out->max_parts = parts;
  // A group's context holds at most 32 / g members' blocks (each at most ceil(limit / B)).
  int64_t gparts = parts;
  if (p->shared) {
    const pa_shared_prefix& sh = *p->shared;
    if (sh.num_groups < 0 || sh.num_groups > p->num_seqs) return PA_ERR_INVALID_ARG;
    if (sh.num_groups > 0 && !sh.groups) return PA_ERR_INVALID_ARG;
    const int64_t members = std::max(1, std::min(kMaxCols / (p->num_q_heads / c.num_kv_heads), std::max(1, p->num_seqs)));
    // Counted in the units the kernel streams: 8-token blocks go two to a tile, and each member's
    // last tile may hold a single block.
    const int32_t unit = (2 * B == kBlockTokens && pt % kBlockTokens == 0) ? kBlockTokens : B;
    const int64_t gblocks = members * ((int64_t{limit} + unit - 1) / unit);
    gparts = std::max<int64_t>(1, (gblocks + pt / unit - 1) / (pt / unit));
    if (gparts > 8192) return PA_ERR_UNSUPPORTED;
  }

  // The route.
  const int32_t D = c.head_dim, g = p->num_q_heads / c.num_kv_heads;
  int32_t lsb = 0;
  while (lsb < 6 && (kBlockTokens << lsb) < B) ++lsb;
  const bool tiles = (kBlockTokens << lsb) == B;
  // 8-token blocks, two to a tile; partitions must hold whole tiles.
  const bool half_blocks = 2 * B == kBlockTokens && pt % kBlockTokens == 0;
  const bool half = c.dtype != PA_F32 && g <= 16;
  // 17 to 32 query heads per KV head fill both 16-column tiles of the split kernel's group mode: every
  // sequence runs as a group of its own.
  const bool wide_g = c.dtype != PA_F32 && g > 16 && g <= kMaxCols;
  const bool shape = (half || wide_g) && (D == 64 || D == 96 || D == 128);
  const bool wide = half && D == 256 && (tiles || half_blocks);
  // Beyond kMaxScanSeqs sequences the split kernel runs once per slice of kMaxScanSeqs (its in-LDS index
  // covers that many).  There, when every context fits one partition, 16-token blocks at head_dim 64 or 128
  // with up to 16 query heads per KV head take the per-partition MFMA kernel instead: one workgroup per
  // (sequence, KV head) and no merge.  Measured on MI355X, 4096 sequences of 512 tokens, 32 query heads on
  // 8 KV heads, bf16: 1430 us against 1494 us in two split launches; with contexts over one partition the
  // split kernel wins (lognormal lengths, median 512: 2354 against 5647 us).  The split kernel indexes
  // the weighted tiles of a launch's (sequence, KV head) pairs with int32.
  const bool big = p->num_seqs > kMaxScanSeqs;
  const bool mfma_fits = half && (D == 64 || D == 128) && B == kBlockTokens;
  const int64_t launch_seqs = std::min<int64_t>(p->num_seqs, kMaxScanSeqs);
  const bool split = ((shape && (tiles || half_blocks)) || wide) && !(big && mfma_fits && parts == 1) &&
                     launch_seqs * c.num_kv_heads *
                             ((int64_t{p->max_blocks_per_seq} << lsb) + int64_t{kPartCost} * (parts + 1) + kCtxCost) <
                         0x7fffffffLL;
  out->route = split ? kRouteSplit : mfma_fits ? kRouteMfma : kRouteGeneric;
  out->sub_log2 = split ? (half_blocks ? -1 : lsb) : 0;
  // A batch cut into slices runs sequence by sequence (a description's groups index the whole batch).
  out->group = split && ((p->shared && p->shared->num_groups > 0 && !big) || wide_g);

  if (split) {
    // Partials per run (see DecodeArgs::part_cols); a context of one partition never spans runs.  A
    // description of shared prefixes sizes for whole groups' columns, with or without groups.
    out->part_cols = (p->shared || wide_g) ? kMaxCols : g;
    const bool partials = p->shared ? gparts > 1 : parts > 1;
    const size_t slots = size_t{kMaxRuns} * 2 * out->part_cols;
    out->ml_offset = slots * D;
    out->counter_offset = slots * (size_t{static_cast<uint32_t>(D)} + 2) * sizeof(float);
    out->workspace =
        partials ? out->counter_offset + static_cast<size_t>(p->num_seqs) * c.num_kv_heads * sizeof(uint64_t) : 0;
  } else {
    // Partials [S][H_q][max_parts][D] and [S][H_q][max_parts][2] (fp32).
    out->part_cols = 0;
    const size_t rows = static_cast<size_t>(p->num_seqs) * p->num_q_heads * parts;
    out->ml_offset = rows * D;
    out->counter_offset = rows * (size_t{static_cast<uint32_t>(D)} + 2) * sizeof(float);
    out->workspace = parts > 1 ? out->counter_offset : 0;
  }
  return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int DT>
void launch_reduce(const DecodeArgs& args, hipStream_t st, hipEvent_t stop) {
  // Output columns (4 dims each) of one (sequence, KV head) are cut into slices so that each
  // workgroup has at most 256 columns and, for few sequences, enough workgroups overall.
  const int nout4 = args.group * args.head_dim / 4;
  const int lo = (nout4 + 255) / 256;
  const int hi = std::max(lo, nout4 / 32);
  const int want = std::max(1, 2048 / std::max(1, args.num_seqs * args.hkv));
  const int nsl = std::min(hi, std::max(lo, want));
  hipExtLaunchKernelGGL(reduce_partitions_kernel<DT>, dim3(static_cast<uint32_t>(args.num_seqs) * args.hkv, nsl),
                        dim3(256), 0, st, nullptr, stop, 0, args);
}

// Workgroups of a kernel that fit on the current device at once
// (compute units x resident workgroups per CU), looked up once per (device, kernel).
int32_t resident_workgroups(const void* kernel, int threads, int* out) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode: hipGetDevice", e);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, kernel});
  if (it != cache.end()) {
    *out = it->second;
    return PA_OK;
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode: CU count", e);
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode: occupancy", e);
  *out = std::max(1, cus) * std::max(1, per_cu);
  cache[{dev, kernel}] = *out;
  return PA_OK;
}

// Rounds of the split kernel's chunk schedule, each cut into one chunk per resident
// workgroup.  One round (equal chunks) measured best on MI355X: later, smaller rounds even
// out the finish times but add partials and workgroup start-up costs that outweigh that.
constexpr int kSplitRounds = 1;

// Compute units of the current device, looked up once per device.
int32_t device_cus(int* out) {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode: hipGetDevice", e);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode: CU count", e);
    it = cache.emplace(dev, std::max(1, cus)).first;
  }
  *out = it->second;
  return PA_OK;
}

// Launch the split kernel with WV wavefronts per workgroup over `contexts` (sequence or group, KV
// head) contexts on `cus` compute units; sets args->run_grid / run_rounds.
template <int DT, int D, int MODE, int WV, int BK>
int32_t launch_split_waves(DecodeArgs* args, int64_t contexts, int cus, hipStream_t st, hipEvent_t start,
                           hipEvent_t stop) {
  const void* fn = reinterpret_cast<const void*>(&decode_split_kernel<DT, D, kPersistRing, MODE, WV, BK>);
  int resident = 0;
  const int32_t rc = resident_workgroups(fn, WV * kWave, &resident);
  if (rc != PA_OK) return rc;
  // With at least two contexts per CU but fewer than the resident workgroups, a grid of one
  // workgroup per context keeps every context whole: filling every slot instead cuts contexts into
  // runs, each cut a partial write and a merge (in group mode 32 columns of head_dim + 2 floats).
  // Measured on MI355X, sampling workload at head_dim 64 (512 contexts, 768 resident workgroups):
  // 64 -> 46 us.
  if (contexts >= 2 * int64_t{cus} && contexts < resident) resident = static_cast<int>(contexts);
  args->run_rounds = kSplitRounds;
  args->run_grid = std::min(kSplitRounds * resident, kMaxRuns / kSplitRounds * kSplitRounds);
  hipExtLaunchKernelGGL((decode_split_kernel<DT, D, kPersistRing, MODE, WV, BK>),
                        dim3(static_cast<uint32_t>(args->run_grid)), dim3(WV * kWave), 0, st, start, stop, 0, *args);
  return PA_OK;
}

// Workgroups of 4 wavefronts, two per CU, by default.  With fewer (sequence or group, KV head)
// contexts than CUs, every context is cut into runs for several workgroups anyway; one workgroup
// of 8 wavefronts per CU then halves the runs, partials and merges of each context.  Measured on
// MI355X: 4 sequences of 131072 tokens, 8 KV heads: 356 -> 339 us; with 512 to 2048 contexts the
// 8-wavefront form was 2-21% slower.
template <int DT, int D, int MODE, int BK>
int32_t launch_split(DecodeArgs* args, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  int cus = 0;
  const int32_t rc = device_cus(&cus);
  if (rc != PA_OK) return rc;
  const int64_t contexts = int64_t{MODE == kGroup ? args->num_groups : args->num_seqs} * args->hkv;
  if (contexts < cus) return launch_split_waves<DT, D, MODE, 8, BK>(args, contexts, cus, st, start, stop);
  return launch_split_waves<DT, D, MODE, 4, BK>(args, contexts, cus, st, start, stop);
}

// One launch: over groups when the batch comes with shared prefixes, else over sequences.
template <int DT, int D, int BK>
int32_t launch_split_all(DecodeArgs* args, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  if (args->num_groups > 0) return launch_split<DT, D, kGroup, BK>(args, st, start, stop);
  return launch_split<DT, D, kPlain, BK>(args, st, start, stop);
}

template <int DT, int D>
int32_t launch_split_blocks(DecodeArgs* args, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  if constexpr (D == 256) {
    // Workgroups of 4 wavefronts, one wave per SIMD.  The group mode spills about 60 VGPRs of its 512
    // registers and still reads a shared prefix once per group: on the sampling workload at head_dim 256
    // (MI355X) 518 us sequence by sequence against 225 us in groups.
    int cus = 0;
    const int32_t rc = device_cus(&cus);
    if (rc != PA_OK) return rc;
    if (args->num_groups > 0) {
      const int64_t contexts = int64_t{args->num_groups} * args->hkv;
      if (args->sub_log2 > 0) return launch_split_waves<DT, 256, kGroup, 4, kBkMulti>(args, contexts, cus, st, start, stop);
      if (args->sub_log2 < 0) return launch_split_waves<DT, 256, kGroup, 4, kBkHalf>(args, contexts, cus, st, start, stop);
      return launch_split_waves<DT, 256, kGroup, 4, kBk16>(args, contexts, cus, st, start, stop);
    }
    const int64_t contexts = int64_t{args->num_seqs} * args->hkv;
    if (args->sub_log2 > 0) return launch_split_waves<DT, 256, kPlain, 4, kBkMulti>(args, contexts, cus, st, start, stop);
    if (args->sub_log2 < 0) return launch_split_waves<DT, 256, kPlain, 4, kBkHalf>(args, contexts, cus, st, start, stop);
    return launch_split_waves<DT, 256, kPlain, 4, kBk16>(args, contexts, cus, st, start, stop);
  } else {
    if (args->sub_log2 > 0) return launch_split_all<DT, D, kBkMulti>(args, st, start, stop);
    if (args->sub_log2 < 0) return launch_split_all<DT, D, kBkHalf>(args, st, start, stop);
    return launch_split_all<DT, D, kBk16>(args, st, start, stop);
  }
}

// Launches of the split kernel for a batch of S sequences: one per slice of kMaxScanSeqs.
int split_slices(int S) { return std::max(1, (S + kMaxScanSeqs - 1) / kMaxScanSeqs); }

template <int DT>
int32_t launch_decode(DecodeArgs args, const Plan& plan, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  const int64_t D = args.head_dim;
  args.part_cost = kPartCost;
  args.ctx_cost = kCtxCost;
  args.run_grid = 0;
  args.run_rounds = 0;
  if (!plan.group) args.num_groups = 0;  // every sequence on its own
  if (plan.route == kRouteSplit) {
    // One launch per slice of at most kMaxScanSeqs sequences (one for all but the largest batches): the
    // split kernel merges its runs in place; it counts in 16-token tiles.  Slices run one after another
    // on the stream, each with its own counter tag; they share the workspace.
    args.sub_log2 = plan.sub_log2;
    args.part_blocks = plan.sub_log2 >= 0 ? args.part_blocks << plan.sub_log2 : args.part_blocks >> 1;
    if constexpr (DT != PA_F32) {
      const int S = args.num_seqs;
      const int slices = split_slices(S);
      const int64_t q_row = int64_t{args.hq} * D * elem_bytes(DT);
      const int64_t out_row = int64_t{args.hq} * D * (args.out_f32 ? 4 : elem_bytes(DT));
      for (int c = 0; c < slices; ++c) {
        DecodeArgs sa = args;
        const int s0 = c * kMaxScanSeqs;
        sa.num_seqs = std::min(kMaxScanSeqs, S - s0);
        if (!sa.share_groups && sa.num_groups > 0) sa.num_groups = sa.num_seqs;  // groups of one sequence
        sa.q = static_cast<const uint8_t*>(args.q) + s0 * q_row;
        sa.out = static_cast<uint8_t*>(args.out) + s0 * out_row;
        sa.block_tables = args.block_tables + int64_t{s0} * args.max_blocks;
        sa.context_lens = args.context_lens + s0;
        sa.launch_tag = args.launch_tag + static_cast<uint32_t>(c);
        hipEvent_t e0 = c == 0 ? start : nullptr, e1 = c == slices - 1 ? stop : nullptr;
        int32_t rc;
        if (D == 64) rc = launch_split_blocks<DT, 64>(&sa, st, e0, e1);
        else if (D == 96) rc = launch_split_blocks<DT, 96>(&sa, st, e0, e1);
        else if (D == 256) rc = launch_split_blocks<DT, 256>(&sa, st, e0, e1);
        else rc = launch_split_blocks<DT, 128>(&sa, st, e0, e1);
        if (rc != PA_OK) return rc;
      }
      return PA_OK;
    }
    return PA_ERR_UNSUPPORTED;
  }
  // The per-partition kernels need the merge kernel when a context spans several partitions.
  const bool merge = args.max_parts > 1;
  hipEvent_t main_stop = merge ? nullptr : stop;
  if (plan.route == kRouteMfma) {
    const int64_t nwg = int64_t{args.max_parts} * args.hkv * args.num_seqs;
    if (nwg > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    if constexpr (DT != PA_F32) {
      if (D == 64)
        hipExtLaunchKernelGGL((decode_mfma_kernel<DT, 64, kRing>), dim3(static_cast<uint32_t>(nwg)),
                              dim3(kWaves * kWave), 0, st, start, main_stop, 0, args);
      else
        hipExtLaunchKernelGGL((decode_mfma_kernel<DT, 128, kRing>), dim3(static_cast<uint32_t>(nwg)),
                              dim3(kWaves * kWave), 0, st, start, main_stop, 0, args);
    }
  } else {
    // Chunks of up to kMaxGenericHeads query heads per KV head: GH = the smallest power of two
    // that holds the group (or a chunk of it).
    const int g = args.group;
    const int gh = g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : kMaxGenericHeads;
    const int64_t chunks = (g + gh - 1) / gh;
    const int64_t nwg = int64_t{args.max_parts} * args.hkv * args.num_seqs * chunks;
    if (nwg > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    const int64_t pt = int64_t{args.part_blocks} * args.block_tokens;
    const size_t lds = static_cast<size_t>(gh * pt + args.part_blocks) * 4;
    const dim3 grid(static_cast<uint32_t>(nwg)), block(kWave);
    switch (gh) {
      case 1: hipExtLaunchKernelGGL((decode_generic_kernel<DT, 1>), grid, block, lds, st, start, main_stop, 0, args); break;
      case 2: hipExtLaunchKernelGGL((decode_generic_kernel<DT, 2>), grid, block, lds, st, start, main_stop, 0, args); break;
      case 4: hipExtLaunchKernelGGL((decode_generic_kernel<DT, 4>), grid, block, lds, st, start, main_stop, 0, args); break;
      default:
        hipExtLaunchKernelGGL((decode_generic_kernel<DT, kMaxGenericHeads>), grid, block, lds, st, start, main_stop, 0,
                              args);
    }
  }
  if (merge) launch_reduce<DT>(args, st, stop);
  return PA_OK;
}

}  // namespace

// ------------------------------------------------------------------ the entry point that allocates nothing

// Scratch of paged_attention_decode_noalloc: a file-scope device array, one copy per GPU for the life of
// the process.  Host code never passes `scratch` itself to a kernel (its host-side name is a stand-in, not
// a device address): each device's address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t{72} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

int32_t scratch_address(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> address of its copy of scratch
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode_noalloc: hipGetDevice", e);
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return PA_HIP_STATUS("paged_attention_decode_noalloc: scratch address", e);
    it = addr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return PA_OK;
}

}  // namespace

extern "C" size_t paged_attention_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int32_t paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                  const int32_t* block_tables, const int32_t* context_lens,
                                                  float scale, void* out, const pa_decode_params* p);

extern "C" size_t paged_attention_workspace_bytes(const pa_decode_params* p) {
  Plan plan;
  return make_plan(p, &plan) == PA_OK ? plan.workspace : 0;
}

extern "C" const char* paged_attention_decode_kernel(const pa_decode_params* p) {
  Plan plan;
  if (make_plan(p, &plan) != PA_OK || p->num_seqs == 0) return "";
  switch (plan.route) {
    case kRouteSplit: return "decode_split_kernel";
    case kRouteMfma: return "decode_mfma_kernel";
    default: return "decode_generic_kernel";
  }
}

extern "C" int32_t paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                                          void* out, const pa_decode_params* p) {
  Plan plan;
  const int32_t st = make_plan(p, &plan);
  if (st != PA_OK) return st;
  if (p->num_seqs == 0) {  // nothing to launch: the events are recorded on the stream directly
    hipStream_t st = static_cast<hipStream_t>(p->stream);
    for (void* ev : {p->start_event, p->stop_event}) {
      if (!ev) continue;
      const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(ev), st);
      if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode: event", e);
    }
    return PA_OK;
  }
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (plan.workspace > 0 && (!p->workspace || p->workspace_bytes < plan.workspace)) return PA_ERR_WORKSPACE;

  DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.part_o = plan.workspace > 0 ? static_cast<float*>(p->workspace) : nullptr;
  a.part_ml = a.part_o ? a.part_o + plan.ml_offset : nullptr;
  a.scale_log2 = scale * kLog2e;
  a.num_seqs = p->num_seqs;
  a.hq = p->num_q_heads;
  a.hkv = p->cache.num_kv_heads;
  a.group = p->num_q_heads / p->cache.num_kv_heads;
  a.head_dim = p->cache.head_dim;
  a.max_blocks = p->max_blocks_per_seq;
  a.ctx_limit = plan.ctx_limit;
  a.part_blocks = plan.part_blocks;
  a.block_tokens = p->cache.block_size;
  a.max_parts = plan.max_parts;
  a.part_cols = plan.part_cols;
  a.out_f32 = p->out_dtype == PA_F32 ? 1 : 0;
  a.num_blocks = p->cache.num_blocks;
  a.run_done = (plan.route == kRouteSplit && plan.workspace > 0)
                   ? reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(p->workspace) + plan.counter_offset)
                   : nullptr;
  if (plan.group) {
    if (p->shared && p->shared->num_groups > 0) {
      a.share_groups = p->shared->groups;
      a.num_groups = p->shared->num_groups;
    } else {  // more than 16 query heads per KV head: one group per sequence
      a.share_groups = nullptr;
      a.num_groups = p->num_seqs;
    }
  }
  // A tag no earlier call of this process used, seeded per process (a workspace may hold
  // counters another process left): the arrival counters need no clearing.
  static std::atomic<uint32_t> next_tag{static_cast<uint32_t>(
      std::chrono::steady_clock::now().time_since_epoch().count() * 0x9e3779b97f4a7c15ull >> 32) ^
      static_cast<uint32_t>(getpid())};
  a.launch_tag = next_tag.fetch_add(
      plan.route == kRouteSplit ? static_cast<uint32_t>(split_slices(p->num_seqs)) : 1u, std::memory_order_relaxed);

  hipStream_t stream = static_cast<hipStream_t>(p->stream);
  (void)hipGetLastError();  // drop an error some earlier, unrelated HIP call left behind
  int32_t rc;
  hipEvent_t start = static_cast<hipEvent_t>(p->start_event), stop = static_cast<hipEvent_t>(p->stop_event);
  switch (p->cache.dtype) {
    case PA_F32: rc = launch_decode<PA_F32>(a, plan, stream, start, stop); break;
    case PA_BF16: rc = launch_decode<PA_BF16>(a, plan, stream, start, stop); break;
    default: rc = launch_decode<PA_F16>(a, plan, stream, start, stop); break;
  }
  if (rc != PA_OK) return rc;
  return PA_HIP_STATUS("paged_attention_decode", hipGetLastError());
}

extern "C" int32_t paged_attention_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                  const int32_t* block_tables, const int32_t* context_lens,
                                                  float scale, void* out, const pa_decode_params* p) {
  Plan plan;
  const int32_t st = make_plan(p, &plan);
  if (st != PA_OK) return st;
  if (plan.workspace > kScratchBytes) return PA_ERR_WORKSPACE;
  pa_decode_params local = *p;
  local.workspace = nullptr;
  local.workspace_bytes = 0;
  if (plan.workspace > 0 && p->num_seqs > 0) {
    const int32_t rc = scratch_address(&local.workspace);
    if (rc != PA_OK) return rc;
    local.workspace_bytes = kScratchBytes;
  }
  return paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, &local);
}

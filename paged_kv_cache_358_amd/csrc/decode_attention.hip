// Paged single-query decode attention for gfx950 (MI355X).
//
// What is computed: per sequence, query head and its KV head, softmax attention of
// the one decode query over the sequence's cached tokens.  Paging does not change
// this math (zhichai.net page, Key points, "Engineering insight"); the kernel only
// follows each sequence's block table to find the scattered 16-token blocks
// (zhichai.net page, "Why it matters"; "Stop Wasting GPU Memory" page, Technical
// Details, "Core Architecture").  Softmax is taken online, block by block, as in the
// FlashAttention kernels the ml-canon page's "Connections" section says vLLM uses.
//
// Work decomposition.  A context is split into partitions of P tokens.  One
// workgroup (4 wavefronts) handles one (partition, KV head, sequence); its waves
// take the partition's blocks round-robin.  Each wave keeps a running max, sum and
// unnormalised output per query head; the four waves merge through LDS.  A sequence
// with one partition writes its output directly; otherwise each partition writes
// (max, sum, normalised output) to the workspace and a second kernel merges them
// with the log-sum-exp rule.
//
// bf16/fp16 fast path (MFMA).  All g = H_q / H_kv query heads of a KV head share
// each K/V block, so a block is one dense contraction, done on the matrix cores with
// v_mfma_f32_16x16x32_{bf16,f16}:
//   S^T[16 tokens x 16 heads] = K_blk[16 x D] . Q^T[D x 16]     (D/32 MFMAs)
//   O^T[D x 16 heads]        += V_blk^T[D x 16] . P^T[16 x 16]  (D/16 MFMAs)
// Query heads beyond g are zero columns.  The lane that holds S for (head, 4 tokens)
// after the first product is exactly the lane that must supply P for them in the
// second, so scores never leave registers.  P is split as P_hi + P_lo, both in the
// input's 16-bit type, and the 32-wide contraction slot of the second MFMA carries
// (token, hi) and (token, lo) pairs against a duplicated V, so the probabilities enter
// with ~16 significant bits instead of 8 while V and the accumulation stay exact fp32.
// The cache layout makes every load a contiguous run per instruction: K is stored in
// 16-byte chunks [D/8][16 tokens][8], so the 64 lanes of one MFMA operand load read
// 1 KiB contiguously; V is stored transposed [D][16 tokens], so a PV operand load reads
// 512 contiguous bytes (16 dims x 16 tokens).
//
// fp32 (and any shape outside the fast path): a plain VALU kernel, one wavefront per
// (partition, query head, sequence).
#include <math.h>

#include <algorithm>
#include <cmath>

#include "pa_device.h"
#include "pa_status.h"

namespace pa {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* part_o;   // [S][H_q][max_parts][D], normalised partition outputs
  float* part_ml;  // [S][H_q][max_parts][2], (max in log2 units, sum)
  float scale_log2;
  int32_t num_seqs;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t head_dim;
  int32_t max_blocks;   // block-table row stride
  int32_t ctx_limit;    // min(max_context_len, max_blocks * 16)
  int32_t part_blocks;  // blocks per partition
  int32_t max_parts;
  int32_t out_f32;
  int64_t num_blocks;
};

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int s) {
  const int n = a.context_lens[s];
  return n < 0 ? 0 : (n > a.ctx_limit ? a.ctx_limit : n);
}

__device__ __forceinline__ int num_parts(int n, int part_blocks) {
  const int pt = part_blocks * kBlockTokens;
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

// ------------------------------------------------------------------ MFMA fast path

// P (4 probabilities of one head for tokens 4j..4j+3) -> B operand of the PV MFMA:
// slots 0..3 hold the high parts, slots 4..7 the low parts (p - high).
template <int DT> struct PSplit;
template <> struct PSplit<PA_BF16> {
  __device__ static u32x4_t split(const float p[4]) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t u = __float_as_uint(p[r]) & 0xffff0000u;  // truncation: exact bf16
      const float rest = p[r] - __uint_as_float(u);               // exact in fp32
      const uint32_t ru = __float_as_uint(rest);
      hi[r] = u;
      lo[r] = (ru + 0x7fffu + ((ru >> 16) & 1u)) & 0xffff0000u;    // bf16, round to nearest even
    }
    u32x4_t out;
    out[0] = (hi[0] >> 16) | hi[1];
    out[1] = (hi[2] >> 16) | hi[3];
    out[2] = (lo[0] >> 16) | lo[1];
    out[3] = (lo[2] >> 16) | lo[3];
    return out;
  }
};
template <> struct PSplit<PA_F16> {
  __device__ static u32x4_t split(const float p[4]) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const _Float16 h = static_cast<_Float16>(p[r]);
      const _Float16 l = static_cast<_Float16>(p[r] - static_cast<float>(h));
      hi[r] = __builtin_bit_cast(uint16_t, h);
      lo[r] = __builtin_bit_cast(uint16_t, l);
    }
    u32x4_t out;
    out[0] = hi[0] | (hi[1] << 16);
    out[1] = hi[2] | (hi[3] << 16);
    out[2] = lo[0] | (lo[1] << 16);
    out[3] = lo[2] | (lo[3] << 16);
    return out;
  }
};

template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  if constexpr (DT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
}

template <int D>
struct KVRegs {
  u32x4_t k[D / 32];  // K operand, one 16-byte chunk per QK MFMA
  u32x2_t v[D / 16];  // V^T operand, 4 tokens of one dim per PV MFMA
};

constexpr int kWaves = 4;

template <int DT, int D>
__global__ __launch_bounds__(kWaves * kWave) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int KK = D / 32;
  constexpr int NV = D / 16;
  __shared__ float sm_o[kWaves][16][D];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];

  const int wg = blockIdx.x;
  const int p = wg % a.max_parts;
  const int rest = wg / a.max_parts;
  const int h = rest % a.hkv;
  const int s = rest / a.hkv;
  const int n = clamp_ctx(a, s);
  const int nparts = num_parts(n, a.part_blocks);
  if (p >= nparts) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
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
  const int my_n = (b1 - b0 > w) ? (b1 - b0 - w + kWaves - 1) / kWaves : 0;

  // Physical ids of this wave's blocks b0 + w + 4 i, one per lane (my_n <= 64).
  int32_t my_id = 0;
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

  const st* kc = static_cast<const st*>(a.k);
  const st* vc = static_cast<const st*>(a.v);
  const int64_t head_stride = static_cast<int64_t>(D) * kBlockTokens;  // elements per (block, kv head)

  auto load = [&](KVRegs<D>& r, int i) {
    int32_t phys = __builtin_amdgcn_readlane(my_id, i);
    if (phys < 0 || phys >= a.num_blocks) phys = 0;  // masked below; never dereference a bad id
    const int64_t base = (static_cast<int64_t>(phys) * a.hkv + h) * head_stride;
    const st* kb = kc + base;
    const st* vb = vc + base;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      r.k[kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + ((kk * 4 + grp) * kBlockTokens + col) * 8));
#pragma unroll
    for (int nn = 0; nn < NV; ++nn)
      r.v[nn] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(vb + (nn * 16 + col) * kBlockTokens + grp * 4));
  };

  f32x4_t o[NV];
#pragma unroll
  for (int nn = 0; nn < NV; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float l = 0.f;

  // Branch-free: a block whose id is out of range counts as empty (nv = 0), and the
  // masking below then leaves m, l and o unchanged, so no path skips a wait.
  auto compute = [&](KVRegs<D>& r, int i) {
    const int bl = b0 + w + kWaves * i;
    const int32_t phys = __builtin_amdgcn_readlane(my_id, i);
    int nv = n - bl * kBlockTokens;
    nv = nv > kBlockTokens ? kBlockTokens : nv;
    if (phys < 0 || phys >= a.num_blocks) nv = 0;

    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sacc = mfma16x16x32<DT>(r.k[kk], qop[kk], sacc);

    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (grp * 4 + e < nv) ? sacc[e] * a.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m, bm);
    const float alpha = (m == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = (x[e] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[e] - m_new);
    l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = m_new;
    const u32x4_t pop = PSplit<DT>::split(pr);

    // Absent tokens' V may hold anything, even NaN: select them out (P is 0 there too).
    uint32_t keep[2];
#pragma unroll
    for (int wd = 0; wd < 2; ++wd) {
      const int t0 = grp * 4 + 2 * wd;
      keep[wd] = (t0 < nv ? 0x0000ffffu : 0u) | (t0 + 1 < nv ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) {
      const uint32_t v0 = r.v[nn][0] & keep[0];
      const uint32_t v1 = r.v[nn][1] & keep[1];
      o[nn] *= alpha;
      const u32x4_t vop = {v0, v1, v0, v1};
      o[nn] = mfma16x16x32<DT>(vop, pop, o[nn]);
    }
  };

  // Two register sets: block i+1's loads are in flight while block i computes.  The
  // steady-state loop issues its loads unconditionally so that each wait covers only
  // the block about to be used; the last one or two blocks are peeled off.
  KVRegs<D> ra, rb;
  if (my_n > 0) {
    load(ra, 0);
    int i = 0;
    for (; i + 2 < my_n; i += 2) {
      load(rb, i + 1);
      compute(ra, i);
      load(ra, i + 2);
      compute(rb, i + 1);
    }
    if (i + 1 < my_n) {
      load(rb, i + 1);
      compute(ra, i);
      compute(rb, i + 1);
    } else {
      compute(ra, i);
    }
  }

  // Per-wave totals: the sum over the four k-groups of this head column.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
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

// ------------------------------------------------------------------ generic VALU path

constexpr int kMaxPartTokens = 1024;
constexpr int kMaxGenericD = 256;

template <int DT>
__global__ __launch_bounds__(kWave) void decode_generic_kernel(DecodeArgs a) {
  using st = typename Elem<DT>::storage;
  constexpr int X = 16 / sizeof(st);
  __shared__ float q_s[kMaxGenericD];
  __shared__ float sc[kMaxPartTokens];
  __shared__ int32_t ids[kMaxPartTokens / kBlockTokens];

  const int wg = blockIdx.x;
  const int p = wg % a.max_parts;
  const int rest = wg / a.max_parts;
  const int j = rest % a.hq;
  const int s = rest / a.hq;
  const int n = clamp_ctx(a, s);
  const int nparts = num_parts(n, a.part_blocks);
  if (p >= nparts) return;
  const int lane = threadIdx.x;
  const int D = a.head_dim;
  const int h = j / a.group;
  const int64_t row = static_cast<int64_t>(s) * a.hq + j;

  if (n == 0) {
    for (int d = lane; d < D; d += kWave) store_out<DT>(a, row * D + d, 0.0f);
    return;
  }
  const st* q = static_cast<const st*>(a.q);
  for (int d = lane; d < D; d += kWave) q_s[d] = Elem<DT>::to_float(q[row * D + d]);
  const int pt = a.part_blocks * kBlockTokens;
  const int t0 = p * pt;
  const int t1 = min(n, t0 + pt);
  const int bl0 = t0 / kBlockTokens;
  const int nb = (t1 - t0 + kBlockTokens - 1) / kBlockTokens;
  for (int b = lane; b < nb; b += kWave) {
    const int32_t id = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + bl0 + b];
    ids[b] = (id >= 0 && id < a.num_blocks) ? id : -1;
  }
  __syncthreads();

  const st* kc = static_cast<const st*>(a.k);
  const st* vc = static_cast<const st*>(a.v);
  const int64_t head_stride = static_cast<int64_t>(D) * kBlockTokens;
  float mx = -INFINITY;
  for (int t = t0 + lane; t < t1; t += kWave) {
    const int id = ids[(t - t0) / kBlockTokens];
    float x = -INFINITY;
    if (id >= 0) {
      const st* kb = kc + (static_cast<int64_t>(id) * a.hkv + h) * head_stride;
      const int off = t % kBlockTokens;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(q_s[d], Elem<DT>::to_float(kb[((d / X) * kBlockTokens + off) * X + d % X]), dot);
      x = dot * a.scale_log2;
    }
    sc[t - t0] = x;
    mx = fmaxf(mx, x);
  }
  mx = wave_max(mx);
  float lsum = 0.f;
  for (int t = t0 + lane; t < t1; t += kWave) {
    const float e = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[t - t0] - mx);
    sc[t - t0] = e;
    lsum += e;
  }
  const float L = wave_sum(lsum);
  __syncthreads();

  const bool single = nparts == 1;
  for (int d = lane; d < D; d += kWave) {
    float acc = 0.f;
    for (int t = t0; t < t1; ++t) {
      const int id = ids[(t - t0) / kBlockTokens];
      if (id < 0) continue;
      const st* vb = vc + (static_cast<int64_t>(id) * a.hkv + h) * head_stride;
      acc = fmaf(sc[t - t0], Elem<DT>::to_float(vb[d * kBlockTokens + t % kBlockTokens]), acc);
    }
    const float res = L > 0.f ? acc / L : 0.f;
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

// ------------------------------------------------------------------ partition merge

// One workgroup per (sequence, query head) with more than one partition:
//   M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p * O_p / sum_p w_p
// where O_p is partition p's normalised output.  Fixed summation order: deterministic.
template <int DT>
__global__ __launch_bounds__(256) void reduce_partitions_kernel(DecodeArgs a) {
  extern __shared__ float wts[];  // [max_parts]
  __shared__ float red[256];
  __shared__ float acc_s[256];
  const int s = blockIdx.x / a.hq;
  const int j = blockIdx.x % a.hq;
  const int n = clamp_ctx(a, s);
  const int np = num_parts(n, a.part_blocks);
  if (np <= 1) return;
  const int tid = threadIdx.x;
  const int D = a.head_dim;
  const int64_t row = static_cast<int64_t>(s) * a.hq + j;
  const float* ml = a.part_ml + row * a.max_parts * 2;
  const float* po = a.part_o + row * a.max_parts * D;

  float mx = -INFINITY;
  for (int p = tid; p < np; p += 256) mx = fmaxf(mx, ml[2 * p]);
  red[tid] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float ls = 0.f;
  for (int p = tid; p < np; p += 256) {
    const float w = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[2 * p] - mx) * ml[2 * p + 1];
    wts[p] = w;
    ls += w;
  }
  red[tid] = ls;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float L = red[0];

  // Threads split as (lane group g over partitions) x (dims): D <= 256.
  const int groups = 256 / D;
  const int gi = tid / D;
  const int d = tid % D;
  float acc = 0.f;
  if (gi < groups) {
    for (int p = gi; p < np; p += groups) acc = fmaf(wts[p], po[static_cast<int64_t>(p) * D + d], acc);
  }
  acc_s[tid] = acc;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int q = 0; q < groups; ++q) t += acc_s[q * D + tid];
    store_out<DT>(a, row * D + tid, L > 0.f ? t / L : 0.f);
  }
}

}  // namespace pa

using namespace pa;

namespace {

struct Plan {
  int32_t part_tokens;
  int32_t part_blocks;
  int32_t ctx_limit;
  int32_t max_parts;
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
  if (c.block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (c.head_dim > kMaxGenericD) return PA_ERR_UNSUPPORTED;
  const int32_t pt = p->partition_size == 0 ? 512 : p->partition_size;
  if (pt < kBlockTokens || pt > kMaxPartTokens || pt % kBlockTokens != 0) return PA_ERR_INVALID_ARG;
  const int64_t limit64 = std::min<int64_t>(p->max_context_len, int64_t{p->max_blocks_per_seq} * kBlockTokens);
  const int32_t limit = static_cast<int32_t>(std::min<int64_t>(limit64, INT32_MAX));
  const int32_t parts = std::max<int32_t>(1, static_cast<int32_t>((int64_t{limit} + pt - 1) / pt));
  if (parts > 8192) return PA_ERR_UNSUPPORTED;  // reduce kernel keeps one weight per partition in LDS
  out->part_tokens = pt;
  out->part_blocks = pt / kBlockTokens;
  out->ctx_limit = limit;
  out->max_parts = parts;
  out->workspace = parts > 1 ? static_cast<size_t>(p->num_seqs) * p->num_q_heads * parts *
                                   (static_cast<size_t>(c.head_dim) + 2) * sizeof(float)
                             : 0;
  return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int DT>
void launch_reduce(const DecodeArgs& args, hipStream_t st) {
  const size_t lds = static_cast<size_t>(args.max_parts) * sizeof(float);
  hipLaunchKernelGGL(reduce_partitions_kernel<DT>, dim3(static_cast<uint32_t>(args.num_seqs) * args.hq), dim3(256),
                     lds, st, args);
}

template <int DT>
int32_t launch_decode(const DecodeArgs& args, hipStream_t st, void* timing_event) {
  const int64_t D = args.head_dim;
  const bool fast = DT != PA_F32 && (D == 64 || D == 128) && args.group <= 16;
  if (fast) {
    const int64_t nwg = int64_t{args.max_parts} * args.hkv * args.num_seqs;
    if (nwg > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    if constexpr (DT != PA_F32) {
      if (D == 64)
        hipLaunchKernelGGL((decode_mfma_kernel<DT, 64>), dim3(static_cast<uint32_t>(nwg)), dim3(kWaves * kWave), 0,
                           st, args);
      else
        hipLaunchKernelGGL((decode_mfma_kernel<DT, 128>), dim3(static_cast<uint32_t>(nwg)), dim3(kWaves * kWave), 0,
                           st, args);
    }
  } else {
    const int64_t nwg = int64_t{args.max_parts} * args.hq * args.num_seqs;
    if (nwg > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(decode_generic_kernel<DT>, dim3(static_cast<uint32_t>(nwg)), dim3(kWave), 0, st, args);
  }
  if (timing_event) {
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(timing_event), st);
    if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_decode: timing event", e);
  }
  if (args.max_parts > 1) launch_reduce<DT>(args, st);
  return PA_OK;
}

}  // namespace

extern "C" size_t paged_attention_workspace_bytes(const pa_decode_params* p) {
  Plan plan;
  return make_plan(p, &plan) == PA_OK ? plan.workspace : 0;
}

extern "C" int32_t paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                                          void* out, const pa_decode_params* p) {
  Plan plan;
  const int32_t st = make_plan(p, &plan);
  if (st != PA_OK) return st;
  if (p->num_seqs == 0) return PA_OK;
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
  a.part_o = static_cast<float*>(p->workspace);
  a.part_ml = a.part_o ? a.part_o + static_cast<size_t>(p->num_seqs) * p->num_q_heads * plan.max_parts *
                                        p->cache.head_dim
                       : nullptr;
  a.scale_log2 = scale * kLog2e;
  a.num_seqs = p->num_seqs;
  a.hq = p->num_q_heads;
  a.hkv = p->cache.num_kv_heads;
  a.group = p->num_q_heads / p->cache.num_kv_heads;
  a.head_dim = p->cache.head_dim;
  a.max_blocks = p->max_blocks_per_seq;
  a.ctx_limit = plan.ctx_limit;
  a.part_blocks = plan.part_blocks;
  a.max_parts = plan.max_parts;
  a.out_f32 = p->out_dtype == PA_F32 ? 1 : 0;
  a.num_blocks = p->cache.num_blocks;

  hipStream_t stream = static_cast<hipStream_t>(p->stream);
  (void)hipGetLastError();  // drop an error some earlier, unrelated HIP call left behind
  int32_t rc;
  switch (p->cache.dtype) {
    case PA_F32: rc = launch_decode<PA_F32>(a, stream, p->timing_event); break;
    case PA_BF16: rc = launch_decode<PA_BF16>(a, stream, p->timing_event); break;
    default: rc = launch_decode<PA_F16>(a, stream, p->timing_event); break;
  }
  if (rc != PA_OK) return rc;
  return PA_HIP_STATUS("paged_attention_decode", hipGetLastError());
}

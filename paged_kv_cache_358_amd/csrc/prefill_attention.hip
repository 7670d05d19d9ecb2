// Paged prefill attention (gfx950): the newest tokens of each sequence, a chunk already
// written into its blocks, attend causally to the sequence's cached tokens.
//
// The prefill phase writes a sequence's tokens into blocks ("Stop Wasting GPU Memory" page,
// Technical Details, "Single Sequence Generation"); the attention itself is the unchanged
// transformer math ("PagedAttention: How Virtual Memory Paging Solved LLM KV Cache Waste"
// page, Key points), gathered through the block table.  Chunk row i of a sequence with n
// cached tokens, c of them in the chunk, is position p = n - c + i and sees tokens 0..p.
//
// One workgroup per (128-row tile of a chunk, query head, sequence), the tiles of one
// (sequence, query head) placed on one XCD so they share its L2; each wave owns 32 chunk
// rows, the columns of two 16-column MFMA tiles that share every K/V block's registers, and
// streams the K/V blocks its last row can see through a ring of register sets (the next
// blocks load while one computes).  The four
// waves of a workgroup read the same blocks, so the caches serve the repeats.  Per block:
// S^T = K Q^T with v_mfma_f32_16x16x32, an online softmax per column (query row) with the
// causal bound applied per (token, column), and O^T += V^T (P_hi + P_lo) with two
// v_mfma_f32_16x16x16 as in the decode kernels.  Each wave writes its own rows.
#include <hip/hip_ext.h>

#include <cmath>

#include "pa_device.h"
#include "pa_mfma.h"
#include "pa_status.h"

namespace pa {

struct PrefillArgs {
  const void* q;  // [T][H_q][D]
  const void* k;
  const void* v;
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* context_lens;  // [S], tokens including the chunk
  const int32_t* query_start;   // [S + 1], first row of each sequence's chunk in q / out
  void* out;                    // [T][H_q][D]
  float scale_log2;
  int32_t num_tokens;  // T
  int32_t hq;
  int32_t hkv;
  int32_t max_blocks;
  int32_t out_f32;
  int32_t tiles;      // row tiles per chunk (ceil(max_query_len / rows per workgroup))
  int32_t per_xcd;    // workgroups per XCD
  int64_t items;      // sequences x query heads x tiles
  int64_t num_blocks;
};

constexpr int kPrefillWaves = 4;
constexpr int kPrefillTiles = 2;                                 // 16-row MFMA column tiles per wave
constexpr int kPrefillWaveRows = 16 * kPrefillTiles;             // chunk rows per wave
constexpr int kPrefillRows = kPrefillWaves * kPrefillWaveRows;  // chunk rows per workgroup
constexpr int kXcdCount = 8;  // accelerator complex dies of an MI355X, one L2 each
constexpr int kPrefillRing = 3;  // K/V register sets per wave: block i computing, i+1 and i+2 loading

template <int DT>
__device__ __forceinline__ void prefill_store4(const PrefillArgs& a, int64_t idx, const f32x4_t& v) {
  if (a.out_f32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + idx) = v;
  } else {
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = Elem<DT>::from_float(v[e]);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + idx) = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
}

template <int DT, int D, int NBUF>
__global__ __launch_bounds__(kPrefillWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(
    PrefillArgs a) {
  constexpr int KK = D / 32;
  constexpr int NV = D / 16;
  constexpr int NT = kPrefillTiles;
  constexpr int kTileBytes = D * kBlockTokens * 2;

  // Workgroups go to the 8 XCDs round-robin (workgroup i on XCD i % 8).  The (sequence,
  // query head) groups are dealt to the XCDs round-robin too, and the k-th workgroup of XCD x
  // takes tile k % tiles of its (k / tiles)-th group: the tiles of one group run back to back
  // on one XCD and read the sequence's blocks through its L2 instead of fetching them from HBM
  // once per tile, while every XCD gets an even share of long and short sequences.
  const int64_t kx = blockIdx.x / kXcdCount;
  const int64_t sj = static_cast<int64_t>(blockIdx.x % kXcdCount) + kXcdCount * (kx / a.tiles);
  if (sj >= a.items / a.tiles) return;
  const int tile = static_cast<int>(kx % a.tiles);
  const int j = static_cast<int>(sj % a.hq);
  const int s = static_cast<int>(sj / a.hq);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int g = a.hq / a.hkv;
  const int h = j / g;

  const int q0 = a.query_start[s];
  const int c = a.query_start[s + 1] - q0;                  // chunk rows of this sequence
  int n = a.context_lens[s];
  n = n < 0 ? 0 : (n > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : n);
  const int r0 = tile * kPrefillRows + w * kPrefillWaveRows;  // this wave's first chunk row
  if (c <= 0 || r0 >= c) return;
  const int r_last = min(c, r0 + kPrefillWaveRows) - 1;
  const int p_last = n - c + r_last;                       // position of the wave's last row
  if (p_last < 0) return;                                  // n < c: no row of this wave has a position

  // This lane's columns: chunk row r0 + 16 t + col of tile t at position p[t] (-1 = no row /
  // no position).
  int64_t row[NT];
  bool real[NT];
  int p[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = r0 + 16 * t + col;
    row[t] = static_cast<int64_t>(q0) + r;
    real[t] = r < c && n - c + r >= 0 && row[t] >= 0 && row[t] < a.num_tokens;
    p[t] = real[t] ? n - c + r : -1;
  }

  // Q^T operands: lane (column col, k-group grp) holds dims (kk*4 + grp)*8 .. +8 of its rows.
  using st = uint16_t;
  const st* qp = static_cast<const st*>(a.q);
  u32x4_t qop[NT][KK];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t qrow = ((real[t] ? row[t] : 0) * a.hq + j) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp + qrow + (kk * 4 + grp) * 8);
      qop[t][kk] = real[t] ? x : u32x4_t{0, 0, 0, 0};
    }
  }

  const int nblk = p_last / kBlockTokens + 1;  // blocks holding tokens 0 .. p_last
  const int32_t* tab = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  // Block ids, 64 per register: lane i holds block base + i (clamped into the row).
  auto load_ids = [&](int base) { return tab[min(base + lane, a.max_blocks - 1)]; };

  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + static_cast<int64_t>(h) * kTileBytes;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + static_cast<int64_t>(h) * kTileBytes;
  const int64_t blk_stride = static_cast<int64_t>(a.hkv) * kTileBytes;
  const int k_off = lane * 16;
  const int v_off = col * 32 + grp * 8;
  // A block past the wave's last one, or an id outside the pool, gets an empty resource:
  // its loads return zeros and touch no memory.
  auto load = [&](KVRegs<D>& rg, int32_t phys, bool ok) {
    ok = ok && phys >= 0 && phys < a.num_blocks;
    const int64_t off = ok ? static_cast<int64_t>(phys) * blk_stride : 0;
    const int nrec = ok ? kTileBytes : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kbase + off), 0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vbase + off), 0, nrec, kRsrcWord3);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      rg.k[kk] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off, kk * 1024, 0));
#pragma unroll
    for (int nn = 0; nn < NV; ++nn)
      rg.v[nn] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off, nn * 512, 0));
  };

  f32x4_t o[NT][NV];
  float m[NT], l[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) o[t][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[t] = -INFINITY;
    l[t] = 0.f;
  }

  // A block whose 16 tokens all lie in the context and before the wave's first row is seen
  // whole by every row: no token needs masking (rows past the chunk are never written).
  const int p_first = n - c + r0;
  // S^T tiles of a block: the matrix-core half of a block's work, issued one block ahead.
  auto qk = [&](const KVRegs<D>& rg, f32x4_t (&s)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) s[t] = mfma_qk<DT>(rg.k[kk], qop[t][kk], s[t]);
    }
  };
  // The rest of block b's work: online softmax over its scores and O^T += V^T P^T.
  auto finish = [&](KVRegs<D>& rg, int b, int32_t phys, const f32x4_t (&s)[NT]) {
    int nv = n - b * kBlockTokens;  // tokens of the block in the context
    nv = nv > kBlockTokens ? kBlockTokens : nv;
    if (phys < 0 || phys >= a.num_blocks) nv = 0;
    const bool whole = nv == kBlockTokens && b * kBlockTokens + kBlockTokens - 1 <= p_first;
    u32x2_t p_hi[NT], p_lo[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4_t sacc = s[t];
      float x[4];
      if (whole) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = sacc[e] * a.scale_log2;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = grp * 4 + e;
          x[e] = (tok < nv && b * kBlockTokens + tok <= p[t]) ? sacc[e] * a.scale_log2 : -INFINITY;
        }
      }
      const float bm = rows4_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      const float m_new = fmaxf(m[t], bm);
      // Once the rows' running maxima settle, most blocks raise none of them: then every
      // correction factor is 1 and the rescale of the tile's O (32 accumulators a lane) is
      // skipped for the whole wave.
      const bool rescale = __builtin_amdgcn_ballot_w64(m_new != m[t]) != 0;
      const float alpha = (m[t] == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m[t] - m_new);
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pr[e] = (x[e] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[e] - m_new);
      l[t] = l[t] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m[t] = m_new;
      if (rescale) {
#pragma unroll
        for (int nn = 0; nn < NV; ++nn) o[t][nn] *= alpha;
      }
      PSplit<DT>::split(pr, p_hi[t], p_lo[t]);
    }
    // Tokens past the context may hold anything, even NaN: a block that is not full has them
    // selected out of its V registers (in place: the ring reloads them next); a full block needs
    // no mask.
    if (nv < kBlockTokens) {
      uint32_t keep[2];
#pragma unroll
      for (int wd = 0; wd < 2; ++wd) {
        const int t0 = grp * 4 + 2 * wd;
        keep[wd] = (t0 < nv ? 0x0000ffffu : 0u) | (t0 + 1 < nv ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) rg.v[nn] = u32x2_t{rg.v[nn][0] & keep[0], rg.v[nn][1] & keep[1]};
    }
    // Both tiles use each V register of the block.
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        o[t][nn] = mfma_pv<DT>(rg.v[nn], p_hi[t], o[t][nn]);
        o[t][nn] = mfma_pv<DT>(rg.v[nn], p_lo[t], o[t][nn]);
      }
    }
  };

  // A ring of NBUF register sets: blocks b+1 .. b+NBUF-1 are loading while block b computes.
  // The scores of block b+1 are computed before block b's softmax and PV, so the matrix cores
  // work on the next block while the vector units take this one's softmax.  Block ids come 64
  // to a register; ids_next holds the 64 after, loaded 64 blocks ahead of its first use, and
  // the pair advances once the blocks reach past the first register.
  int base = 0;
  int32_t ids = load_ids(0);
  int32_t ids_next = load_ids(64);
  auto phys_at = [&](int pos) {
    return pos < base + 64 ? __builtin_amdgcn_readlane(ids, pos - base) : __builtin_amdgcn_readlane(ids_next, pos - base - 64);
  };
  KVRegs<D> ring[NBUF];
#pragma unroll
  for (int jj = 0; jj < NBUF - 1; ++jj) load(ring[jj], phys_at(jj), jj < nblk);
  f32x4_t s_next[NT];
  qk(ring[0], s_next);
  for (int b = 0; b < nblk; b += NBUF) {
    if (b - base >= 64) {
      base += 64;
      ids = ids_next;
      ids_next = load_ids(base + 64);
    }
#pragma unroll
    for (int jj = 0; jj < NBUF; ++jj) {
      const int i = b + jj;
      const int la = i + NBUF - 1;
      load(ring[(jj + NBUF - 1) % NBUF], phys_at(la), la < nblk);
      if (i < nblk) {
        f32x4_t s_cur[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) s_cur[t] = s_next[t];
        if (i + 1 < nblk) qk(ring[(jj + 1) % NBUF], s_next);
        finish(ring[jj], i, phys_at(i), s_cur);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = rows4_sum(l[t]);
    if (!real[t]) continue;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int64_t orow = (row[t] * a.hq + j) * D;
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) prefill_store4<DT>(a, orow + nn * 16 + grp * 4, o[t][nn] * inv);
  }
}

}  // namespace pa

using namespace pa;

extern "C" int32_t paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                           const int32_t* block_tables, const int32_t* context_lens,
                                           const int32_t* query_start, float scale, void* out,
                                           const pa_prefill_params* p) {
  if (!p) return PA_ERR_INVALID_ARG;
  const pa_cache_desc& c = p->cache;
  if (p->num_seqs < 0 || p->num_tokens < 0 || p->num_q_heads <= 0 || p->max_blocks_per_seq <= 0 ||
      p->max_query_len < 0 || c.num_blocks <= 0 || c.num_kv_heads <= 0 || c.head_dim <= 0)
    return PA_ERR_INVALID_ARG;
  if (p->num_q_heads % c.num_kv_heads != 0 || !valid_dtype(c.dtype)) return PA_ERR_INVALID_ARG;
  if (p->out_dtype != PA_F32 && p->out_dtype != c.dtype) return PA_ERR_INVALID_ARG;
  if (c.block_size != kBlockTokens || c.dtype == PA_F32 || (c.head_dim != 64 && c.head_dim != 128))
    return PA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  hipEvent_t start = static_cast<hipEvent_t>(p->start_event), stop = static_cast<hipEvent_t>(p->stop_event);
  (void)hipGetLastError();  // drop an error some earlier, unrelated HIP call left behind
  if (p->num_seqs == 0 || p->num_tokens == 0 || p->max_query_len == 0) {
    for (hipEvent_t ev : {start, stop}) {
      if (!ev) continue;
      const hipError_t e = hipEventRecord(ev, st);
      if (e != hipSuccess) return PA_HIP_STATUS("paged_attention_prefill: event", e);
    }
    return PA_OK;
  }
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out) return PA_ERR_INVALID_ARG;
  auto a16 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; };
  if (!a16(q) || !a16(k_cache) || !a16(v_cache) || !a16(out)) return PA_ERR_INVALID_ARG;

  PrefillArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.out = out;
  a.scale_log2 = scale * kLog2e;
  a.num_tokens = p->num_tokens;
  a.hq = p->num_q_heads;
  a.hkv = c.num_kv_heads;
  a.max_blocks = p->max_blocks_per_seq;
  a.out_f32 = p->out_dtype == PA_F32 ? 1 : 0;
  a.num_blocks = c.num_blocks;
  a.tiles = (p->max_query_len + kPrefillRows - 1) / kPrefillRows;
  a.items = static_cast<int64_t>(p->num_seqs) * p->num_q_heads * a.tiles;
  const int64_t groups = static_cast<int64_t>(p->num_seqs) * p->num_q_heads;
  const int64_t per_xcd = (groups + kXcdCount - 1) / kXcdCount * a.tiles;
  if (per_xcd * kXcdCount > 0x7fffffffLL || per_xcd > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  a.per_xcd = static_cast<int32_t>(per_xcd);
  const dim3 grid(static_cast<uint32_t>(per_xcd * kXcdCount));
  const dim3 block(kPrefillWaves * kWave);
  if (c.dtype == PA_BF16) {
    if (c.head_dim == 64)
      hipExtLaunchKernelGGL((prefill_mfma_kernel<PA_BF16, 64, kPrefillRing>), grid, block, 0, st, start, stop, 0, a);
    else
      hipExtLaunchKernelGGL((prefill_mfma_kernel<PA_BF16, 128, kPrefillRing>), grid, block, 0, st, start, stop, 0, a);
  } else {
    if (c.head_dim == 64)
      hipExtLaunchKernelGGL((prefill_mfma_kernel<PA_F16, 64, kPrefillRing>), grid, block, 0, st, start, stop, 0, a);
    else
      hipExtLaunchKernelGGL((prefill_mfma_kernel<PA_F16, 128, kPrefillRing>), grid, block, 0, st, start, stop, 0, a);
  }
  return PA_HIP_STATUS("paged_attention_prefill", hipGetLastError());
}

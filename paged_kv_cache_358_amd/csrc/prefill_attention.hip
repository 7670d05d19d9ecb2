// Paged prefill attention (gfx950): the newest tokens of each sequence, a chunk already
// written into its blocks, attend causally to the sequence's cached tokens.
//
// The prefill phase writes a sequence's tokens into blocks ("Stop Wasting GPU Memory" page,
// Technical Details, "Single Sequence Generation"); the attention itself is the unchanged
// transformer math ("PagedAttention: How Virtual Memory Paging Solved LLM KV Cache Waste"
// page, Key points), gathered through the block table.  Chunk row i of a sequence with n
// cached tokens, c of them in the chunk, is position p = n - c + i and sees tokens 0..p.
//
// One workgroup of four waves per (128-row tile of a chunk, query head, sequence), the tiles of
// one (sequence, query head) placed on one XCD so that they share its L2.  Each wave owns 32 chunk
// rows, two 16-column MFMA tiles.  The K/V blocks the tile's last row can see are streamed in
// stages of four 16-token blocks: each wave loads one block of the next stage into registers and
// writes it to LDS while the current stage computes, one barrier per stage.  Per stage and row
// tile: S^T = K Q^T with v_mfma_f32_16x16x32 (K read from LDS), one online-softmax update over the
// stage's 64 tokens with the causal bound applied only on the stages that need it, and
// O^T += V^T (P_hi + P_lo) with v_mfma_f32_16x16x32 over block pairs.  Each wave writes its own rows.
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
  const int32_t* seq_order;  // [S]: the sequence of each scheduling rank, or null (batch order)
  int32_t num_seqs;
  int32_t block_tokens;  // B: 8 or 16 << sub_log2
  int32_t sub_log2;      // log2 of the 16-token tiles per block (B >= 16), -1 for 8-token blocks
};

constexpr int kPrefillWaves = 4;
constexpr int kPrefillTiles = 2;                                 // 16-row MFMA column tiles per wave
constexpr int kPrefillWaveRows = 16 * kPrefillTiles;             // chunk rows per wave
constexpr int kPrefillRows = kPrefillWaves * kPrefillWaveRows;  // chunk rows per workgroup
constexpr int kXcdCount = 8;  // accelerator complex dies of an MI355X, one L2 each

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

// Each wave loads one 16-token block of a stage (K and V tiles as stored, V with the tokens past the
// context zeroed) and writes it to one of two LDS buffers; every wave then computes its 32 rows
// against all four blocks.  The PV product's 32-wide contraction takes tokens 4 grp .. 4 grp + 3 of
// both blocks of a pair, the order in which the score tiles leave them in a lane; P is split into
// hi + lo in the cache's 16-bit type, so that it enters the product with about 16 significant bits.
constexpr int kStageBlocks = kPrefillWaves;  // 16-token blocks per stage: one per wave
constexpr float kLazyLog2 = 8.0f;  // how far (log2 units) a score may exceed the softmax reference point m

// Block kinds: kPb16, 16-token blocks; kPbMulti, blocks of 16 << sub_log2 tokens (32, 64, ...);
// kPbHalf, 8-token blocks.
constexpr int kPb16 = 0, kPbMulti = 1, kPbHalf = 2;

// Head_dim 256 doubles the output tiles and K/V registers (256 VGPRs and about 230 AGPRs, no scratch) and
// its LDS stages take 128 KiB: one workgroup per CU, one wave per SIMD.  One 16-row tile per wave instead
// (half the registers) measured slower on MI355X: 3.12 against 2.63 ms on the MHA workload's chunks.
template <int DT, int D, int BK>
__global__ __launch_bounds__(kPrefillWaves * kWave) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2))) void
prefill_tiled_kernel(PrefillArgs a) {
  constexpr int KK = D / 32;
  constexpr int NV = D / 16;
  constexpr int NT = kPrefillTiles;
  constexpr int kTileBytes = D * kBlockTokens * 2;
  // K: [buffer][block of the stage][tile as stored].  V: [buffer][block pair][16-dim group][lane][block of
  // the pair][4 tokens]: a lane's PV operand (4 tokens of both blocks) is one 16-byte read, and the 64
  // lanes of a read cover 1 KiB without gaps.
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][kStageBlocks][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][kStageBlocks / 2][NV][kWave * 16];

  // Workgroups go to the 8 XCDs round-robin (workgroup i on XCD i % 8).  The (sequence, query head)
  // groups are dealt to the XCDs round-robin too, and the k-th workgroup of XCD x takes tile
  // k % tiles of its (k / tiles)-th group: the tiles of one group run back to back on one XCD and
  // read the sequence's blocks through its L2 instead of fetching them from HBM once per tile,
  // while every XCD gets an even share of long and short sequences.
  const int64_t kx = blockIdx.x / kXcdCount;
  const int64_t sj = static_cast<int64_t>(blockIdx.x % kXcdCount) + kXcdCount * (kx / a.tiles);
  if (sj >= a.items / a.tiles) return;
  const int tile = static_cast<int>(kx % a.tiles);
  const int j = static_cast<int>(sj % a.hq);
  // Groups go out in rank order: rank r is sequence seq_order[r] when an order is given.
  int s = static_cast<int>(sj / a.hq);
  if (a.seq_order) {
    s = a.seq_order[s];
    if (s < 0 || s >= a.num_seqs) return;
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int g = a.hq / a.hkv;
  const int h = j / g;

  const int q0 = a.query_start[s];
  const int c = a.query_start[s + 1] - q0;  // chunk rows of this sequence
  int n = a.context_lens[s];
  n = n < 0 ? 0 : (n > a.max_blocks * a.block_tokens ? a.max_blocks * a.block_tokens : n);
  // Workgroup-uniform exits (before any barrier): no row of the tile, or no row with a position.
  const int R0 = tile * kPrefillRows;
  if (c <= 0 || R0 >= c) return;
  const int p_wg_last = n - c + min(c, R0 + kPrefillRows) - 1;
  if (p_wg_last < 0) return;
  const int nblk = p_wg_last / kBlockTokens + 1;  // blocks holding tokens 0 .. p_wg_last
  const int nstage = (nblk + kStageBlocks - 1) / kStageBlocks;

  // This wave's rows: r0 .. r0 + 31; the last stage it needs (-1: none).
  const int r0 = R0 + w * kPrefillWaveRows;
  const int p_w_last = r0 < c ? n - c + min(c, r0 + kPrefillWaveRows) - 1 : -1;
  const int w_last_stage = p_w_last >= 0 ? p_w_last / (kBlockTokens * kStageBlocks) : -1;
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
  const int p_first = n - c + r0;  // position of the wave's first row (rows before it see every earlier token)

  // The exponent is taken as exp2(kscale * s - m) with one FMA per score and the maximum over raw
  // scores, which needs kscale > 0: a negative scale negates Q instead (exact: a sign flip of every
  // element), and a zero scale (every visible token weighs the same) zeroes Q with kscale = 1.
  const float scl = a.scale_log2;
  const bool qzero = scl == 0.f;
  const uint32_t qflip = scl < 0.f ? 0x80008000u : 0u;
  const float kscale = qzero ? 1.f : fabsf(scl);
  using st = uint16_t;
  const st* qp = static_cast<const st*>(a.q);
  u32x4_t qop[NT][KK];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t qrow = ((real[t] ? row[t] : 0) * a.hq + j) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp + qrow + (kk * 4 + grp) * 8);
      qop[t][kk] = real[t] && !qzero ? (x ^ qflip) : u32x4_t{0, 0, 0, 0};
    }
  }

  // Everything counts in 16-token tiles: stage st holds tiles st * 4 .. st * 4 + 3, and this wave loads
  // tile st * 4 + w.  Tile u is tile u % SB of cache block u / SB for blocks of 16 << sub_log2 tokens
  // (SB = 1 << sub_log2), and cache blocks 2u and 2u + 1 for 8-token blocks.  Block ids of this wave's
  // tiles: lane i of ids (and of ids2, the second block of an 8-token pair) holds stage base + i's.
  const int lsb = BK == kPbMulti ? a.sub_log2 : 0;
  constexpr bool half = BK == kPbHalf;
  const int32_t* tab = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  auto tile_block = [&](int base, int second) {
    const int u = (base + lane) * kStageBlocks + w;
    return tab[min(half ? 2 * u + second : u >> lsb, a.max_blocks - 1)];
  };
  auto load_ids = [&](int base) { return tile_block(base, 0); };
  int ids_base = 0;
  int32_t ids = load_ids(0);
  int32_t ids2 = half ? tile_block(0, 1) : 0;

  // A (cache block, KV head) holds K as [D/8][B][8] and V as [D][B].
  const int head_bytes = half ? kTileBytes / 2 : kTileBytes << lsb;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + static_cast<int64_t>(h) * head_bytes;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + static_cast<int64_t>(h) * head_bytes;
  const int64_t blk_stride = static_cast<int64_t>(a.hkv) * head_bytes;
  // Lane (col, grp): K token col of chunk kk * 4 + grp, V dim col (of each 16-dim group) at the
  // tile's tokens 4 grp .. 4 grp + 3.  Offsets into a block of 16 << lsb tokens, tile 0 (k_goff,
  // v_off), and into the tile's K in LDS, which is kept as a 16-token block's (k_off).
  const int k_goff = ((grp << (4 + lsb)) + col) * 16;
  const int k_off = lane * 16;
  const int v_off = ((col * 32) << lsb) + grp * 8;
  // Load tile b (this wave's tile of a stage) into registers.  A tile past the workgroup's last one, or
  // a block id outside the pool, loads zeros: an empty resource (no memory touched) or, for 8-token
  // blocks, whose lanes each read through their own address, a select after reading the cache's first
  // tile (in bounds).
  auto gload = [&](KVRegs<D>& rg, int b, int32_t phys, int32_t phys2) {
    const bool in = b < nblk;
    if constexpr (half) {
      const bool ok0 = in && phys >= 0 && phys < a.num_blocks;
      const bool ok1 = in && phys2 >= 0 && phys2 < a.num_blocks;
      const int64_t o0 = ok0 ? static_cast<int64_t>(phys) * blk_stride : 0;
      const int64_t o1 = ok1 ? static_cast<int64_t>(phys2) * blk_stride : 0;
      const bool kok = col < 8 ? ok0 : ok1, vok = grp < 2 ? ok0 : ok1;
      const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(kbase + (col < 8 ? o0 : o1) + grp * 128 + (col & 7) * 16);
      const u32x2_t* vp = reinterpret_cast<const u32x2_t*>(vbase + (grp < 2 ? o0 : o1) + col * 16 + (grp & 1) * 8);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4_t x = __builtin_nontemporal_load(kp + kk * 32);
        rg.k[kk] = kok ? x : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
        const u32x2_t x = __builtin_nontemporal_load(vp + nn * 32);
        rg.v[nn] = vok ? x : u32x2_t{0, 0};
      }
      return;
    }
    const bool ok = in && phys >= 0 && phys < a.num_blocks;
    const int sub = b & ((1 << lsb) - 1);  // tile of its cache block
    const int64_t off = ok ? static_cast<int64_t>(phys) * blk_stride : 0;
    const int tk = ok ? sub * 256 : 0, tv = ok ? sub * 32 : 0;
    const int nrec = ok ? head_bytes : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kbase + off + tk), 0, nrec - tk, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vbase + off + tv), 0, nrec - tv, kRsrcWord3);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      rg.k[kk] =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, k_goff, (kk * 1024) << lsb, 0));
#pragma unroll
    for (int nn = 0; nn < NV; ++nn)
      rg.v[nn] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off, (nn * 512) << lsb, 0));
  };
  // Block b's tiles into buffer buf, in the layout they have in the cache; V tokens past the context
  // (which may hold anything, even NaN) are zeroed so that no product reads them.
  auto lwrite = [&](KVRegs<D>& rg, int buf, int b, int32_t phys) {
    int nv = n - b * kBlockTokens;
    nv = nv > kBlockTokens ? kBlockTokens : (nv < 0 ? 0 : nv);
    if (b >= nblk || (!half && (phys < 0 || phys >= a.num_blocks))) nv = 0;
    uint8_t* kt = k_lds[buf][w];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) *reinterpret_cast<u32x4_t*>(kt + k_off + kk * 1024) = rg.k[kk];
    uint32_t keep[2];
#pragma unroll
    for (int wd = 0; wd < 2; ++wd) {
      const int t0 = grp * 4 + 2 * wd;
      keep[wd] = (t0 < nv ? 0x0000ffffu : 0u) | (t0 + 1 < nv ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int nn = 0; nn < NV; ++nn)
      *reinterpret_cast<u32x2_t*>(&v_lds[buf][w >> 1][nn][lane * 16 + (w & 1) * 8]) =
          u32x2_t{rg.v[nn][0] & keep[0], rg.v[nn][1] & keep[1]};
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

  // One stage (buffer buf, blocks b0 .. b0 + 3) for this wave's rows.
  auto compute = [&](int buf, int b0) {
    // Scores: lane (row col of tile t, k-group grp) gets tokens 4 grp .. 4 grp + 3 of each block.
    f32x4_t sc[NT][kStageBlocks];
#pragma unroll
    for (int bb = 0; bb < kStageBlocks; ++bb) {
      u32x4_t kop[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kop[kk] = *reinterpret_cast<const u32x4_t*>(k_lds[buf][bb] + k_off + kk * 1024);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sc[t][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) sc[t][bb] = mfma_qk<DT>(kop[kk], qop[t][kk], sc[t][bb]);
      }
    }
    // Stage tokens b0 * 16 .. b0 * 16 + 63: those past the context or after a row's position count
    // nothing for that row.  A stage every row of the wave sees whole (all but the last one or two
    // of a wave) needs no mask: the branch is uniform across the wave.
    const int t_end = min(n, (b0 + kStageBlocks) * kBlockTokens) - 1;  // last token of the stage in the context
    const bool whole = t_end == (b0 + kStageBlocks) * kBlockTokens - 1 && t_end <= p_first;
    // Raw scores, those a row does not see set to -inf (kscale * -inf = -inf, exp2 of it 0).
    if (!whole) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // Token tok counts for row t of this lane when tok <= lim (p = -1 for a row past the chunk).
        const int lim = min(t_end, p[t]) - (b0 * kBlockTokens + grp * 4);
#pragma unroll
        for (int bb = 0; bb < kStageBlocks; ++bb)
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[t][bb][e] = bb * kBlockTokens + e <= lim ? sc[t][bb][e] : -INFINITY;
      }
    }
    u32x4_t p_hi[NT][kStageBlocks / 2], p_lo[NT][kStageBlocks / 2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float bm = fmaxf(fmaxf(sc[t][0][0], sc[t][0][1]), fmaxf(sc[t][0][2], sc[t][0][3]));
#pragma unroll
      for (int bb = 1; bb < kStageBlocks; ++bb)
        bm = fmaxf(bm, fmaxf(fmaxf(sc[t][bb][0], sc[t][bb][1]), fmaxf(sc[t][bb][2], sc[t][bb][3])));
      bm = rows4_max(bm) * kscale;
      // m is a reference point, not the running maximum: the weights exp2(k s - m) of any m give the
      // same softmax once divided by their sum.  It moves (and l and O are rescaled) only when some
      // row of the wave sees a score more than kLazyLog2 above it, so weights stay below
      // 2^kLazyLog2 and most stages skip the rescale.  A row that has seen no token has m = -inf and
      // moves at its first visible token.
      if (__builtin_amdgcn_ballot_w64(bm > m[t] + kLazyLog2) != 0) {
        const float m_new = fmaxf(m[t], bm);
        const float alpha = (m[t] == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m[t] - m_new);
        l[t] *= alpha;
#pragma unroll
        for (int nn = 0; nn < NV; ++nn) o[t][nn] *= alpha;
        m[t] = m_new;
      }
      // Exponents of a row still at m = -inf (no visible token yet) are taken against 0: exp2(-inf) = 0
      // weighs its masked tokens without a select.
      const float m_use = m[t] == -INFINITY ? 0.0f : m[t];
      float pr[kStageBlocks][4];
      float sum = 0.f;
#pragma unroll
      for (int bb = 0; bb < kStageBlocks; ++bb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[bb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][bb][e], kscale, -m_use));
          sum += pr[bb][e];
        }
      l[t] += sum;
#pragma unroll
      for (int pp = 0; pp < kStageBlocks / 2; ++pp) {
        u32x2_t ha, la, hb, lb;
        PSplit<DT>::split(pr[2 * pp], ha, la);
        PSplit<DT>::split(pr[2 * pp + 1], hb, lb);
        p_hi[t][pp] = u32x4_t{ha[0], ha[1], hb[0], hb[1]};
        p_lo[t][pp] = u32x4_t{la[0], la[1], lb[0], lb[1]};
      }
    }
    // O^T += V^T P^T over block pairs: the V operand of lane (dim col, k-group grp) is tokens
    // 4 grp .. 4 grp + 3 of both blocks of the pair.
#pragma unroll
    for (int pp = 0; pp < kStageBlocks / 2; ++pp) {
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
        const u32x4_t vop = *reinterpret_cast<const u32x4_t*>(&v_lds[buf][pp][nn][lane * 16]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          o[t][nn] = mfma_qk<DT>(vop, p_hi[t][pp], o[t][nn]);
          o[t][nn] = mfma_qk<DT>(vop, p_lo[t][pp], o[t][nn]);
        }
      }
    }
  };

  KVRegs<D> rg;
  {
    const int32_t phys = __builtin_amdgcn_readlane(ids, 0);
    gload(rg, w, phys, half ? __builtin_amdgcn_readlane(ids2, 0) : 0);
    lwrite(rg, 0, w, phys);
  }
  __syncthreads();
  for (int stg = 0; stg < nstage; ++stg) {
    const int nxt = stg + 1;
    int32_t phys_n = -1;
    if (nxt < nstage) {
      if (nxt - ids_base >= 64) {
        ids_base += 64;
        ids = load_ids(ids_base);
        if (half) ids2 = tile_block(ids_base, 1);
      }
      phys_n = __builtin_amdgcn_readlane(ids, nxt - ids_base);
      gload(rg, nxt * kStageBlocks + w, phys_n, half ? __builtin_amdgcn_readlane(ids2, nxt - ids_base) : 0);
    }
    if (stg <= w_last_stage) compute(stg & 1, stg * kStageBlocks);
    if (nxt < nstage) lwrite(rg, nxt & 1, nxt * kStageBlocks + w, phys_n);
    __syncthreads();
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

// The VALU kernel: fp32 caches, and 16-bit caches of the shapes the MFMA kernel does not take (head_dim
// other than 64, 96, 128, 256; blocks other than 8 and 16 << j tokens).  One wavefront per (chunk row,
// query head), four to a workgroup (consecutive rows of one (sequence, head)).  The row's visible tokens go
// in passes of 64, a lane per token: the lane scores its token against the row's query (K in 16-byte
// chunks of X dims), the pass updates the row's online softmax (max and sum over the wave), then every
// lane accumulates output dims lane, lane + 64, ... over the pass's tokens, each token's weight and block
// id broadcast from its lane.  Any head_dim that is a multiple of X up to 256 and any block size up to
// 1024.  A block id outside the pool leaves its tokens out.
constexpr int kPrefillValuWaves = 4;
constexpr int kPrefillValuMaxD = 256;

// Dot product of 16 bytes of K and of the query (X elements each).
template <int DT>
__device__ __forceinline__ float dot16(const void* k, const void* q) {
  if constexpr (DT == PA_F32) {
    const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(k);
    const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(q);
    return kv[0] * qv[0] + kv[1] * qv[1] + kv[2] * qv[2] + kv[3] * qv[3];
  } else {
    const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(k);
    const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(q);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += Elem<DT>::to_float(static_cast<uint16_t>(kv[e] & 0xffffu)) *
             Elem<DT>::to_float(static_cast<uint16_t>(qv[e] & 0xffffu));
      acc += Elem<DT>::to_float(static_cast<uint16_t>(kv[e] >> 16)) * Elem<DT>::to_float(static_cast<uint16_t>(qv[e] >> 16));
    }
    return acc;
  }
}

template <int DT>
__global__ __launch_bounds__(kPrefillValuWaves * kWave) void prefill_valu_kernel(PrefillArgs a, int32_t D) {
  using T = typename Elem<DT>::storage;
  constexpr int X = 16 / static_cast<int>(sizeof(T));  // dims per 16-byte K chunk
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows_pad = a.tiles * kPrefillValuWaves;  // row slots per (sequence rank, query head)
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kPrefillValuWaves + w;
  const int i = static_cast<int>(item % rows_pad);
  const int64_t sj = item / rows_pad;
  if (sj >= static_cast<int64_t>(a.num_seqs) * a.hq) return;
  const int j = static_cast<int>(sj % a.hq);
  int s = static_cast<int>(sj / a.hq);
  if (a.seq_order) {
    s = a.seq_order[s];
    if (s < 0 || s >= a.num_seqs) return;
  }
  const int q0 = a.query_start[s];
  const int c = a.query_start[s + 1] - q0;
  int n = a.context_lens[s];
  const int B = a.block_tokens;
  n = n < 0 ? 0 : (n > a.max_blocks * B ? a.max_blocks * B : n);
  const int64_t row = static_cast<int64_t>(q0) + i;
  const int pos = n - c + i;  // this row's position: it sees tokens 0 .. pos
  if (i >= c || pos < 0 || row < 0 || row >= a.num_tokens) return;
  const int h = j / (a.hq / a.hkv);

  const T* qrow = static_cast<const T*>(a.q) + (row * a.hq + j) * D;
  const int64_t head_elems = static_cast<int64_t>(D) * B;  // elements of one (block, KV head) tile of K or V
  const T* kbase = static_cast<const T*>(a.k) + h * head_elems;
  const T* vbase = static_cast<const T*>(a.v) + h * head_elems;
  const int64_t blk_elems = static_cast<int64_t>(a.hkv) * head_elems;
  const int32_t* tab = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;

  float m = -INFINITY, l = 0.f;
  float o[kPrefillValuMaxD / kWave];
#pragma unroll
  for (int k = 0; k < kPrefillValuMaxD / kWave; ++k) o[k] = 0.f;
  for (int t0 = 0; t0 <= pos; t0 += kWave) {
    const int t = t0 + lane;
    int32_t phys = -1;
    float x = -INFINITY;  // log2-scaled score of token t
    if (t <= pos) {
      const int32_t id = tab[t / B];
      if (id >= 0 && id < a.num_blocks) {
        phys = id;
        const T* kp = kbase + id * blk_elems + (t % B) * X;  // chunk dc at + dc * B * X
        float acc = 0.f;
        for (int dc = 0; dc < D / X; ++dc) acc += dot16<DT>(kp + static_cast<int64_t>(dc) * B * X, qrow + dc * X);
        x = acc * a.scale_log2;
      }
    }
    const float m_new = fmaxf(m, wave_max(x));
    if (m_new == -INFINITY) continue;  // no visible token in the pass yet (wave-uniform)
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
    const float pw = x == -INFINITY ? 0.f : exp2f(x - m_new);
    l = l * alpha + wave_sum(pw);
#pragma unroll
    for (int k = 0; k < kPrefillValuMaxD / kWave; ++k) o[k] *= alpha;
    m = m_new;
    const int ntok = min(kWave, pos + 1 - t0);
    for (int tt = 0; tt < ntok; ++tt) {
      const float p_t = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pw), tt));
      const int32_t ph = __builtin_amdgcn_readlane(phys, tt);
      if (ph < 0 || p_t == 0.f) continue;  // wave-uniform
      const T* vp = vbase + ph * blk_elems + (t0 + tt) % B;
#pragma unroll
      for (int k = 0; k < kPrefillValuMaxD / kWave; ++k) {
        const int d = lane + k * kWave;
        if (d < D) o[k] += p_t * Elem<DT>::to_float(vp[static_cast<int64_t>(d) * B]);
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t obase = (row * a.hq + j) * D;
#pragma unroll
  for (int k = 0; k < kPrefillValuMaxD / kWave; ++k) {
    const int d = lane + k * kWave;
    if (d >= D) continue;
    if (a.out_f32)
      static_cast<float*>(a.out)[obase + d] = o[k] * inv;
    else
      static_cast<T*>(a.out)[obase + d] = static_cast<T>(Elem<DT>::from_float(o[k] * inv));
  }
}

template <int DT, int D>
void launch_prefill(int bk, dim3 grid, dim3 block, hipStream_t st, hipEvent_t start, hipEvent_t stop,
                    const PrefillArgs& a) {
  if (bk == kPbHalf)
    hipExtLaunchKernelGGL((prefill_tiled_kernel<DT, D, kPbHalf>), grid, block, 0, st, start, stop, 0, a);
  else if (bk == kPbMulti)
    hipExtLaunchKernelGGL((prefill_tiled_kernel<DT, D, kPbMulti>), grid, block, 0, st, start, stop, 0, a);
  else
    hipExtLaunchKernelGGL((prefill_tiled_kernel<DT, D, kPb16>), grid, block, 0, st, start, stop, 0, a);
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
      p->max_query_len < 0 || c.num_blocks <= 0 || c.num_kv_heads <= 0 || c.head_dim <= 0 || c.block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (p->num_q_heads % c.num_kv_heads != 0 || !valid_dtype(c.dtype)) return PA_ERR_INVALID_ARG;
  if (p->out_dtype != PA_F32 && p->out_dtype != c.dtype) return PA_ERR_INVALID_ARG;
  // The MFMA kernel: bf16/fp16, head_dim 64, 96, 128 or 256, blocks of 8 or 16 << j tokens.  Everything else
  // within head_dim <= 256 (a multiple of 16 bytes of elements) and blocks of up to 1024 tokens: the VALU kernel.
  int32_t sub_log2 = -1;  // 8-token blocks
  if (c.block_size != kBlockTokens / 2) {
    sub_log2 = 0;
    while (sub_log2 < 6 && (kBlockTokens << sub_log2) < c.block_size) ++sub_log2;
  }
  const bool mfma_blocks = c.block_size == kBlockTokens / 2 || (kBlockTokens << sub_log2) == c.block_size;
  const bool mfma = c.dtype != PA_F32 && mfma_blocks &&
                    (c.head_dim == 64 || c.head_dim == 96 || c.head_dim == 128 || c.head_dim == 256);
  if (!mfma && (c.block_size > 1024 || c.head_dim % (16 / elem_bytes(c.dtype)) != 0 ||
                c.head_dim > kPrefillValuMaxD))
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
  a.seq_order = p->seq_order;
  a.num_seqs = p->num_seqs;
  a.block_tokens = c.block_size;
  a.sub_log2 = sub_log2;
  if (!mfma) {
    // four rows of one (sequence, query head) per workgroup
    a.tiles = (p->max_query_len + kPrefillValuWaves - 1) / kPrefillValuWaves;
    a.items = static_cast<int64_t>(p->num_seqs) * p->num_q_heads * a.tiles;
    if (a.items > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    const dim3 vgrid(static_cast<uint32_t>(a.items)), vblock(kPrefillValuWaves * kWave);
    if (c.dtype == PA_F32)
      hipExtLaunchKernelGGL(prefill_valu_kernel<PA_F32>, vgrid, vblock, 0, st, start, stop, 0, a, c.head_dim);
    else if (c.dtype == PA_BF16)
      hipExtLaunchKernelGGL(prefill_valu_kernel<PA_BF16>, vgrid, vblock, 0, st, start, stop, 0, a, c.head_dim);
    else
      hipExtLaunchKernelGGL(prefill_valu_kernel<PA_F16>, vgrid, vblock, 0, st, start, stop, 0, a, c.head_dim);
    return PA_HIP_STATUS("paged_attention_prefill", hipGetLastError());
  }
  a.tiles = (p->max_query_len + kPrefillRows - 1) / kPrefillRows;
  a.items = static_cast<int64_t>(p->num_seqs) * p->num_q_heads * a.tiles;
  const int64_t groups = static_cast<int64_t>(p->num_seqs) * p->num_q_heads;
  const int64_t per_xcd = (groups + kXcdCount - 1) / kXcdCount * a.tiles;
  if (per_xcd * kXcdCount > 0x7fffffffLL || per_xcd > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  a.per_xcd = static_cast<int32_t>(per_xcd);
  const dim3 grid(static_cast<uint32_t>(per_xcd * kXcdCount));
  const dim3 block(kPrefillWaves * kWave);
  const int bk = sub_log2 < 0 ? kPbHalf : sub_log2 > 0 ? kPbMulti : kPb16;
  if (c.dtype == PA_BF16) {
    if (c.head_dim == 64)
      launch_prefill<PA_BF16, 64>(bk, grid, block, st, start, stop, a);
    else if (c.head_dim == 96)
      launch_prefill<PA_BF16, 96>(bk, grid, block, st, start, stop, a);
    else if (c.head_dim == 256)
      launch_prefill<PA_BF16, 256>(bk, grid, block, st, start, stop, a);
    else
      launch_prefill<PA_BF16, 128>(bk, grid, block, st, start, stop, a);
  } else {
    if (c.head_dim == 64)
      launch_prefill<PA_F16, 64>(bk, grid, block, st, start, stop, a);
    else if (c.head_dim == 96)
      launch_prefill<PA_F16, 96>(bk, grid, block, st, start, stop, a);
    else if (c.head_dim == 256)
      launch_prefill<PA_F16, 256>(bk, grid, block, st, start, stop, a);
    else
      launch_prefill<PA_F16, 128>(bk, grid, block, st, start, stop, a);
  }
  return PA_HIP_STATUS("paged_attention_prefill", hipGetLastError());
}

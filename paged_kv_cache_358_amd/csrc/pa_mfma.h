// MFMA building blocks shared by the gfx950 attention kernels: the S^T = K Q^T and
// O^T += V^T P^T tiles over one 16-token block, and the buffer loads that feed them.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kRsrcWord3 = 0x00020000;  // raw (unstructured) buffer, 32-bit data format
constexpr int kLoadNT = 2;              // buffer-load cache policy: non-temporal (streamed once)

// P (4 probabilities of one head for tokens 4j..4j+3) split as P = hi + lo, both in the
// cache's 16-bit type; each half is the B operand of one PV MFMA, so the probabilities
// enter the product with ~16 significant bits while the accumulation stays fp32.
template <int DT> struct PSplit;
template <> struct PSplit<PA_BF16> {
  // Two probabilities to a packed bf16 pair, rounded to nearest even (v_cvt_pk_bf16_f32).
  __device__ static uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
  }
  __device__ static void split(const float p[4], u32x2_t& hi_out, u32x2_t& lo_out) {
    // hi = bf16(p); the remainder p - hi is exact in fp32; lo = bf16(remainder).
    const uint32_t h01 = pack(p[0], p[1]), h23 = pack(p[2], p[3]);
    const float r0 = p[0] - __uint_as_float(h01 << 16), r1 = p[1] - __uint_as_float(h01 & 0xffff0000u);
    const float r2 = p[2] - __uint_as_float(h23 << 16), r3 = p[3] - __uint_as_float(h23 & 0xffff0000u);
    hi_out = u32x2_t{h01, h23};
    lo_out = u32x2_t{pack(r0, r1), pack(r2, r3)};
  }
};
template <> struct PSplit<PA_F16> {
  __device__ static void split(const float p[4], u32x2_t& hi_out, u32x2_t& lo_out) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const _Float16 h = static_cast<_Float16>(p[r]);
      const _Float16 l = static_cast<_Float16>(p[r] - static_cast<float>(h));
      hi[r] = __builtin_bit_cast(uint16_t, h);
      lo[r] = __builtin_bit_cast(uint16_t, l);
    }
    hi_out = u32x2_t{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
    lo_out = u32x2_t{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
  }
};

// S^T tile: v_mfma_f32_16x16x32 (8 elements of the contraction per lane).
template <int DT>
__device__ __forceinline__ f32x4_t mfma_qk(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  if constexpr (DT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
}

// O^T tile: v_mfma_f32_16x16x16 (4 tokens per lane), V straight from its load registers.
template <int DT>
__device__ __forceinline__ f32x4_t mfma_pv(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  if constexpr (DT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b),
                                                     c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                                 0, 0);
  }
}

// O^T tile over 16 tokens with split probabilities in one v_mfma_f32_16x16x32: the contraction
// runs over (token, half) pairs.  Lane group kg holds its tokens 4 kg .. 4 kg + 3 twice on the V
// side and the hi then the lo halves of their probabilities on the P side, so one instruction adds
// V^T (P_hi + P_lo)^T; it takes the issue time of one 16x16x16 product, not two.
template <int DT>
__device__ __forceinline__ f32x4_t mfma_pv_split(const u32x2_t& v, const u32x2_t& hi, const u32x2_t& lo,
                                                 const f32x4_t& c) {
  return mfma_qk<DT>(u32x4_t{v[0], v[1], v[0], v[1]}, u32x4_t{hi[0], hi[1], lo[0], lo[1]}, c);
}

// Max and sum over the four 16-lane rows of a wavefront (lanes l, l^16, l^32, l^48: one MFMA
// output column's four k-groups), with the gfx950 permlane swaps, which stay in the vector ALU,
// instead of shuffles routed through LDS.  Swapping a register with itself leaves x at lane l and
// x at lane l^16 (or l^32) in the two results, in some order; max and + do not depend on it.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
struct KVRegs {
  u32x4_t k[D / 32];  // K operand, one 16-byte chunk per QK MFMA
  u32x2_t v[D / 16];  // V^T operand, 4 tokens of one dim per PV MFMA
};

// 32 tokens of one cache block: K as two 16-row operands (row r of half h is token 16 h + r, so
// that every K load reads whole 256-byte runs of a chunk), V^T with 8 consecutive tokens of one
// dim per lane, the operand of a 16x16x32 PV MFMA.  Two permlane swaps bring the probabilities of
// tokens 8 j .. 8 j + 7 to lane group j, in the order the PV operand needs.
template <int D>
struct KVPairRegs {
  u32x4_t k[2][D / 32];
  u32x4_t v[D / 16];
};

}  // namespace pa

// MXFP4 (OCP MX v1.0: e2m1 codes, one e8m0 scale per 32 elements) to bf16
// MFMA fragments, exactly, for the grouped GEMMs with MXFP4 weights.
// "DeepSeek-V4.1-Flash fine-grained MoE (5A)" sec. 1: routed experts in FP4.
#pragma once

#include "gemm_tile.h"

namespace moe {
namespace {

// e2m1 code -> binary32 bits (OCP MX v1.0: bit 3 sign, 2 exponent bits with
// bias 1, 1 mantissa bit; exponent 0 encodes 0 and 0.5).
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t c) {
  const uint32_t mag = c & 7u;
  uint32_t b = (mag == 0u) ? 0u
             : (mag == 1u) ? 0x3F000000u
                           : ((((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22));
  return b | ((c & 8u) << 28);
}

// Two codes of one byte, times 2^(s-127), as a bf16 pair (exact).
__device__ __forceinline__ uint32_t mx_pair(uint32_t byte, float scale) {
  const float lo = __uint_as_float(e2m1_bits(byte & 15u)) * scale;
  const float hi = __uint_as_float(e2m1_bits(byte >> 4)) * scale;
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Two fragments (8 e2m1 codes each, k-consecutive, low nibble first, with
// their e8m0 scales) -> two MFMA fragments of 8 bf16. The hardware
// conversion multiplies by the fp32 scale exactly for scale codes 2..252,
// where 2^(s - 127) is the float with exponent field s; when either code is
// outside that range (tiny or huge blocks) both fragments are formed from
// fp32 products instead. One range test serves both fragments.
template <int I>
__device__ __forceinline__ uint32_t mx_cvt(uint32_t codes, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, I));
}
__device__ __forceinline__ void mx_fragments(uint32_t c0, uint32_t s0, uint32_t c1, uint32_t s1,
                                             bf16x8_t& f0, bf16x8_t& f1) {
  u32x4_t o0, o1;
  if (max(s0 - 2u, s1 - 2u) < 251u) {
    const float a0 = __uint_as_float(s0 << 23), a1 = __uint_as_float(s1 << 23);
    o0.x = mx_cvt<0>(c0, a0);
    o0.y = mx_cvt<1>(c0, a0);
    o0.z = mx_cvt<2>(c0, a0);
    o0.w = mx_cvt<3>(c0, a0);
    o1.x = mx_cvt<0>(c1, a1);
    o1.y = mx_cvt<1>(c1, a1);
    o1.z = mx_cvt<2>(c1, a1);
    o1.w = mx_cvt<3>(c1, a1);
  } else {
    const float a0 = e8m0_scale(s0), a1 = e8m0_scale(s1);
    o0.x = mx_pair(c0 & 0xFFu, a0);
    o0.y = mx_pair((c0 >> 8) & 0xFFu, a0);
    o0.z = mx_pair((c0 >> 16) & 0xFFu, a0);
    o0.w = mx_pair(c0 >> 24, a0);
    o1.x = mx_pair(c1 & 0xFFu, a1);
    o1.y = mx_pair((c1 >> 8) & 0xFFu, a1);
    o1.z = mx_pair((c1 >> 16) & 0xFFu, a1);
    o1.w = mx_pair(c1 >> 24, a1);
  }
  f0 = __builtin_bit_cast(bf16x8_t, o0);
  f1 = __builtin_bit_cast(bf16x8_t, o1);
}

}  // namespace
}  // namespace moe

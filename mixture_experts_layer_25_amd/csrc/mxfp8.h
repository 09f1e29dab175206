// MXFP8 (OCP MX v1.0: e4m3 elements, one e8m0 scale per 32 values)
// quantisation of fp32 blocks, and the grouped scale layout the A8 GEMM
// reads. Shared by the quantiser (gemm_a8.hip), the GEMM's SwiGLU epilogue
// and the quantising dispatch copy (dispatch.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Byte offset of the e8m0 scale of (row, 32-element block kb) in the
// grouped scale layout the GEMM reads: [ceil(K/512)][rows][16], i.e. for
// each run of 16 blocks (8 GEMM steps) every row's 16 scales are one
// 16-byte piece, copied by one lane.
__device__ __forceinline__ size_t grouped_scale(long long row, int kb, long long rows) {
  return ((size_t)(kb / 16) * rows + row) * 16 + kb % 16;
}

// Two floats -> two e4m3 codes in the low (HI = false) or high 16 bits of
// `old`, saturated to +-448, rounded to nearest even.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// MXFP8 block of 32 fp32 values: returns the e8m0 scale code and writes the
// 32 e4m3 codes (8 dwords, element 4i + b in byte b of dword i).
__device__ __forceinline__ uint32_t mxfp8_block(const float (&v)[32], uint32_t (&q)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // floor(log2 amax) = biased exponent field - 127 for normal amax; zero
  // and subnormal amax take the lowest scale code, 0
  const int ef = (int)(__float_as_uint(amax) >> 23);
  const int s = max(ef - 8, 0);  // scale code = floor(log2 amax) - 8 + 127
  const int sh = 127 - s;        // elements are v * 2^sh
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = __builtin_amdgcn_ldexpf(v[4 * i], sh);
    const float b = __builtin_amdgcn_ldexpf(v[4 * i + 1], sh);
    const float c = __builtin_amdgcn_ldexpf(v[4 * i + 2], sh);
    const float d = __builtin_amdgcn_ldexpf(v[4 * i + 3], sh);
    q[i] = fp8x2<true>(c, d, fp8x2<false>(a, b, 0u));
  }
  return (uint32_t)s;
}

}  // namespace moe

// Combine: weighted sum of each token's expert outputs, back in token order.
//
// "moe f&b compute flow" (Echo's blog), Combine: expert outputs are summed
// with the router weights and put back per token. "ops-transformer MoE
// operator on Ascend NPU", MoEForward steps 3-4 (scatter back, weighted
// sum); "FFN, SwiGLU and MoE" sec. 3: y = sum over the selected experts of
// weight * expert output; "DeepSeek-V4.1-Flash fine-grained MoE (5A)"
// sec. 3: the shared expert's output is added once.
//
// One wave per token. Each lane owns 8 consecutive columns: it gathers the
// token's kept y_perm rows (fp32, 2 x 16-byte loads per row), accumulates
// slot by slot in ascending order with fused multiply-adds, adds the shared
// expert row, and stores 8 outputs at once. HBM-bound.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_shared, int T,
                                                      int D, int k, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int pos[kMaxK];
  float w[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    pos[j] = j < k ? slot_pos[(size_t)t * k + j] : -1;
    w[j] = j < k ? topk_w[(size_t)t * k + j] : 0.0f;
  }
  const int nv = D / 8;
  for (int v = lane; v < nv; v += 64) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (pos[j] >= 0) {
        const float4* src = reinterpret_cast<const float4*>(y_perm + (size_t)pos[j] * D) + 2 * v;
        const float4 a = src[0], b = src[1];
        acc[0] = __builtin_fmaf(w[j], a.x, acc[0]);
        acc[1] = __builtin_fmaf(w[j], a.y, acc[1]);
        acc[2] = __builtin_fmaf(w[j], a.z, acc[2]);
        acc[3] = __builtin_fmaf(w[j], a.w, acc[3]);
        acc[4] = __builtin_fmaf(w[j], b.x, acc[4]);
        acc[5] = __builtin_fmaf(w[j], b.y, acc[5]);
        acc[6] = __builtin_fmaf(w[j], b.z, acc[6]);
        acc[7] = __builtin_fmaf(w[j], b.w, acc[7]);
      }
    }
    if (y_shared) {
      const float4* src = reinterpret_cast<const float4*>(y_shared + (size_t)t * D) + 2 * v;
      const float4 a = src[0], b = src[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    if (OUT_BF16) {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + (size_t)t * D)[v] = o;
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * D) + 2 * v;
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const moe_cfg& c, const float* y_perm, const int32_t* slot_pos,
                          const float* topk_w, const float* y_shared, void* y, hipStream_t s) {
  const dim3 grid(ceil_div(c.T, 4));
  if (c.act_dtype == MOE_BF16)
    combine_kernel<true><<<grid, 256, 0, s>>>(y_perm, slot_pos, topk_w, y_shared, c.T, c.D,
                                              c.top_k, y);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(y_perm, slot_pos, topk_w, y_shared, c.T, c.D,
                                               c.top_k, y);
  return hipGetLastError();
}

}  // namespace moe

// Combine: weighted sum of each token's expert outputs, back in token order.
//
// "moe f&b compute flow" (Echo's blog), Combine: expert outputs are summed
// with the router weights and put back per token. "ops-transformer MoE
// operator on Ascend NPU", MoEForward steps 3-4 (scatter back, weighted
// sum); "FFN, SwiGLU and MoE" sec. 3: y = sum over the selected experts of
// weight * expert output; "DeepSeek-V4.1-Flash fine-grained MoE (5A)"
// sec. 3: the shared expert's output is added once.
//
// One wave per token. Each lane owns groups of 8 consecutive columns (eight
// groups in flight per iteration: a 4096-column row in one pass; four were
// 2-3 % slower, two 1 % slower): it gathers the token's kept y_perm rows
// (fp32, 2 x 16-byte loads per row and group), accumulates slot by slot in
// ascending order with fused multiply-adds, adds the shared expert row, and
// stores 8 outputs at once. HBM-bound.
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
  // eight groups of 8 columns per iteration (v, v + 64, ..., v + 448): all
  // their loads are in flight together; each column's sum keeps the order
  // slot 0, 1, ..., then the shared row
  constexpr int UN = 8;
  const int nv = D / 8;
  for (int v0 = lane; v0 < nv; v0 += 64 * UN) {
    float acc[UN][8];
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (pos[j] >= 0) {
        const float4* src = reinterpret_cast<const float4*>(y_perm + (size_t)pos[j] * D);
        float4 a[UN], b[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int v = v0 + 64 * u;
          if (v < nv) {
            a[u] = src[2 * v];
            b[u] = src[2 * v + 1];
          } else {
            a[u] = b[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          acc[u][0] = __builtin_fmaf(w[j], a[u].x, acc[u][0]);
          acc[u][1] = __builtin_fmaf(w[j], a[u].y, acc[u][1]);
          acc[u][2] = __builtin_fmaf(w[j], a[u].z, acc[u][2]);
          acc[u][3] = __builtin_fmaf(w[j], a[u].w, acc[u][3]);
          acc[u][4] = __builtin_fmaf(w[j], b[u].x, acc[u][4]);
          acc[u][5] = __builtin_fmaf(w[j], b[u].y, acc[u][5]);
          acc[u][6] = __builtin_fmaf(w[j], b[u].z, acc[u][6]);
          acc[u][7] = __builtin_fmaf(w[j], b[u].w, acc[u][7]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int v = v0 + 64 * u;
      if (v >= nv) continue;
      if (y_shared) {
        const float4* src = reinterpret_cast<const float4*>(y_shared + (size_t)t * D) + 2 * v;
        const float4 a = src[0], b = src[1];
        acc[u][0] += a.x; acc[u][1] += a.y; acc[u][2] += a.z; acc[u][3] += a.w;
        acc[u][4] += b.x; acc[u][5] += b.y; acc[u][6] += b.z; acc[u][7] += b.w;
      }
      if (OUT_BF16) {
        // y is written once and not read again here: non-temporal stores
        // (384- and 128-expert layers 2-3 % faster, the 8-expert layer
        // within 1.5 %, with the MALL flushed before each run)
        typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
        const u32x4v o = {pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3]),
                          pack_bf16x2(acc[u][4], acc[u][5]), pack_bf16x2(acc[u][6], acc[u][7])};
        __builtin_nontemporal_store(
            o, reinterpret_cast<u32x4v*>(static_cast<uint16_t*>(y) + (size_t)t * D) + v);
      } else {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * D) + 2 * v;
        dst[0] = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
        dst[1] = make_float4(acc[u][4], acc[u][5], acc[u][6], acc[u][7]);
      }
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

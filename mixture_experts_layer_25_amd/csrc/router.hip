// Router: logits, selection key, top-k in registers, gating weights.
//
// "FFN, SwiGLU and MoE" (bjdmk.com) sec. 3: r = W_r x, p = softmax(r), the
// k largest, optional renormalisation. "ops-transformer MoE operator on
// Ascend NPU": router in FP32 (pitfall 3); a new score must be strictly
// larger to displace a kept one (optimisation 2), so equal keys go to the
// lower expert index. "DeepSeek-V4.1-Flash fine-grained MoE (5A)" sec. 1, 3:
// select on score + bias, weight with the raw sqrt(softplus(score)).
// "MoE routing: Top-K, Expert-Choice and Sigmoid Gating": sigmoid weights.
//
// Each logit is one fp32 fused multiply-add chain over d = 0..D-1 from +0,
// so every logit is bit-reproducible. The chain order rules out MFMA (whose
// internal summation order is not specified); the work runs on the vector
// ALUs: a workgroup stages a D-chunk of x (transposed, fp32) and of W_r in
// LDS, and each thread keeps RT tokens x RE experts of accumulators in
// registers. A token's experts live in NE adjacent lanes, so top-k is a
// butterfly arg-max over those lanes, k times, with no sorting.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

struct RouterArgs {
  const void* x;
  const float* W_r;
  const float* bias;
  int32_t* idx;
  float* w;
  float* logits;
  int T, D, E, k, gating, renorm;
};

constexpr int kMaxK = 16;

template <int NE, int RE, int RT, int DK, bool XBF16>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  constexpr int NT = 256 / NE;  // token groups per workgroup
  constexpr int TB = NT * RT;   // tokens per workgroup
  constexpr int EP = NE * RE;   // experts, padded
  __shared__ float xs[DK][TB];
  __shared__ float wsm[DK][EP];

  const int tid = threadIdx.x;
  const int te = tid % NE;
  const int tt = tid / NE;
  const int t0 = blockIdx.x * TB;

  float acc[RT][RE];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < RE; ++j) acc[i][j] = 0.0f;

  for (int d0 = 0; d0 < a.D; d0 += DK) {
    const int dk = min(DK, a.D - d0);
    __syncthreads();
    for (int q = tid; q < TB * DK; q += 256) {
      const int tl = q / DK, dd = q % DK;
      const int t = t0 + tl;
      float v = 0.0f;
      if (t < a.T && dd < dk) {
        const size_t off = (size_t)t * a.D + d0 + dd;
        v = XBF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[off])
                  : static_cast<const float*>(a.x)[off];
      }
      xs[dd][tl] = v;
    }
    for (int q = tid; q < DK * EP; q += 256) {
      const int dd = q / EP, e = q % EP;
      float v = 0.0f;
      if (dd < dk && e < a.E) v = a.W_r[(size_t)(d0 + dd) * a.E + e];
      wsm[dd][e] = v;
    }
    __syncthreads();
    for (int dd = 0; dd < dk; ++dd) {
      float xv[RT], wv[RE];
#pragma unroll
      for (int i = 0; i < RT; ++i) xv[i] = xs[dd][tt * RT + i];
#pragma unroll
      for (int j = 0; j < RE; ++j) wv[j] = wsm[dd][te + NE * j];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < RE; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
    }
  }

  for (int i = 0; i < RT; ++i) {
    const int t = t0 + tt * RT + i;
    float key[RE];
    bool avail[RE];
#pragma unroll
    for (int j = 0; j < RE; ++j) {
      const int e = te + NE * j;
      avail[j] = e < a.E;
      key[j] = avail[j] ? acc[i][j] + (a.bias ? a.bias[e] : 0.0f) : -INFINITY;
      if (a.logits && t < a.T && avail[j]) a.logits[(size_t)t * a.E + e] = acc[i][j];
    }
    // softmax normaliser over all experts: max key, then sum of exp(key - max)
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < RE; ++j) m = fmaxf(m, key[j]);
#pragma unroll
    for (int o = NE / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, NE));
    float Z = 0.0f;
    if (a.gating == MOE_GATE_SOFTMAX) {
#pragma unroll
      for (int j = 0; j < RE; ++j)
        if (avail[j]) Z += expf(key[j] - m);
#pragma unroll
      for (int o = NE / 2; o >= 1; o >>= 1) Z += __shfl_xor(Z, o, NE);
    }

    float wsel[kMaxK];
    int isel[kMaxK];
    float wsum = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxK; ++s) {
      if (s < a.k) {
        float bk = -INFINITY, bl = 0.0f;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < RE; ++j) {
          const int e = te + NE * j;
          if (avail[j] && (key[j] > bk || (key[j] == bk && e < bi))) {
            bk = key[j];
            bi = e;
            bl = acc[i][j];
          }
        }
#pragma unroll
        for (int o = NE / 2; o >= 1; o >>= 1) {
          const float ok = __shfl_xor(bk, o, NE);
          const int oi = __shfl_xor(bi, o, NE);
          const float ol = __shfl_xor(bl, o, NE);
          if (ok > bk || (ok == bk && oi < bi)) {
            bk = ok;
            bi = oi;
            bl = ol;
          }
        }
#pragma unroll
        for (int j = 0; j < RE; ++j)
          if (te + NE * j == bi) avail[j] = false;
        float wv;
        if (a.gating == MOE_GATE_SOFTMAX) {
          wv = expf(bk - m) / Z;
        } else if (a.gating == MOE_GATE_SIGMOID) {
          wv = 1.0f / (1.0f + expf(-bl));
        } else {
          const float sp = fmaxf(bl, 0.0f) + log1pf(expf(-fabsf(bl)));
          wv = sqrtf(sp);
        }
        wsel[s] = wv;
        isel[s] = bi;
        wsum += wv;
      }
    }
    if (te == 0 && t < a.T) {
#pragma unroll
      for (int s = 0; s < kMaxK; ++s) {
        if (s < a.k) {
          a.idx[(size_t)t * a.k + s] = isel[s];
          a.w[(size_t)t * a.k + s] = a.renorm ? wsel[s] / wsum : wsel[s];
        }
      }
    }
  }
}

template <int NE, int RE, int RT, int DK>
hipError_t launch(const RouterArgs& a, bool xbf16, hipStream_t s) {
  constexpr int TB = (256 / NE) * RT;
  dim3 grid(ceil_div(a.T, TB));
  if (xbf16)
    router_kernel<NE, RE, RT, DK, true><<<grid, 256, 0, s>>>(a);
  else
    router_kernel<NE, RE, RT, DK, false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const moe_cfg& c, const void* x, const float* W_r, const float* bias,
                         int32_t* idx, float* w, float* logits, hipStream_t s) {
  RouterArgs a{x, W_r, bias, idx, w, logits, c.T, c.D, c.E, c.top_k, c.gating, c.renorm};
  const bool b = c.act_dtype == MOE_BF16;
  if (c.E <= 8) return launch<8, 1, 1, 32>(a, b, s);
  if (c.E <= 16) return launch<16, 1, 2, 32>(a, b, s);
  if (c.E <= 32) return launch<32, 1, 4, 32>(a, b, s);
  if (c.E <= 64) return launch<64, 1, 8, 32>(a, b, s);
  if (c.E <= 128) return launch<64, 2, 8, 32>(a, b, s);
  if (c.E <= 256) return launch<64, 4, 8, 32>(a, b, s);
  if (c.E <= 384) return launch<64, 6, 16, 32>(a, b, s);
  if (c.E <= 512) return launch<64, 8, 8, 16>(a, b, s);
  return launch<64, 16, 4, 16>(a, b, s);
}

}  // namespace moe

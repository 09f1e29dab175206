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
// ALUs: a workgroup stages D-chunks of x (transposed, fp32) and of W_r in a
// double-buffered LDS area (the next chunk's loads fly while the current one
// is multiplied), and each thread keeps RT tokens x RE experts of
// accumulators in registers. A token's experts live in NE adjacent lanes,
// so top-k is a butterfly arg-max over those lanes, k times, with no
// sorting.
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

// Selection and gating from the workgroup's logit tile lg ([token][EP],
// in LDS, complete): thread (tt, te) holds experts te + NE j of tokens
// tt * RT + i. Keys = logit + bias; k rounds of a butterfly arg-max over the
// token's NE lanes (a larger key wins, an equal key goes to the lower
// expert index); weights by the gating mode; lane te == 0 writes the
// token's k indices and weights.
template <int NE, int RE, int RT>
__device__ __forceinline__ void select_topk(const RouterArgs& a, const float* lg, int tt, int te,
                                            int t0) {
  constexpr int EP = NE * RE;
  for (int i = 0; i < RT; ++i) {
    const int t = t0 + tt * RT + i;
    const float* row = lg + (tt * RT + i) * EP;
    float key[RE], lgt[RE];
    bool avail[RE];
#pragma unroll
    for (int j = 0; j < RE; ++j) {
      const int e = te + NE * j;
      avail[j] = e < a.E;
      lgt[j] = row[e];
      key[j] = avail[j] ? lgt[j] + (a.bias ? a.bias[e] : 0.0f) : -INFINITY;
      if (a.logits && t < a.T && avail[j]) a.logits[(size_t)t * a.E + e] = lgt[j];
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
            bl = lgt[j];
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

template <int NE, int RE, int RT, int DK, int NTH, bool XBF16>
__global__ __launch_bounds__(NTH) void router_kernel(RouterArgs a) {
  constexpr int NT = NTH / NE;  // token groups per workgroup
  constexpr int TB = NT * RT;   // tokens per workgroup
  constexpr int EP = NE * RE;   // experts, padded
  constexpr int VX = XBF16 ? 8 : 4;                     // x values per 16-byte load
  constexpr int NXV = (TB * DK / VX + NTH - 1) / NTH;  // x loads per thread per chunk
  constexpr int NWV = (DK * EP / 4 + NTH - 1) / NTH;   // W_r loads per thread per chunk
  __shared__ float xs[2][DK][TB];
  __shared__ float wsm[2][DK][EP];

  const int tid = threadIdx.x;
  const int te = tid % NE;
  const int tt = tid / NE;
  const int t0 = blockIdx.x * TB;
  const int D = a.D, E = a.E;
  const bool wvec = (E & 3) == 0;

  float acc[RT][RE];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < RE; ++j) acc[i][j] = 0.0f;

  // Chunk c covers d = c*DK .. c*DK+DK-1. Its x rows (TB tokens) and W_r
  // rows go global -> registers -> LDS (x transposed to [d][token], fp32);
  // the next chunk's loads are in flight while this one is multiplied.
  uint4 rx[NXV];
  float4 rw[NWV];
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const int d0 = c * DK;
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + NTH * i;
      const int tl = v / (DK / VX), dg = v % (DK / VX);
      const int t = t0 + tl, d = d0 + VX * dg;
      rx[i] = make_uint4(0, 0, 0, 0);
      if (v < TB * DK / VX && t < a.T && d < D)
        rx[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) +
                                                ((size_t)t * D + d) * (XBF16 ? 2 : 4));
    }
    const int nw = min(DK, D - d0) * E;  // valid floats of this chunk
    const float* wsrc = a.W_r + (size_t)d0 * E;
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int f = 4 * (tid + NTH * i);
      float4 w4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (wvec) {
        if (f < nw) w4 = *reinterpret_cast<const float4*>(wsrc + f);
      } else {
        if (f < nw) w4.x = wsrc[f];
        if (f + 1 < nw) w4.y = wsrc[f + 1];
        if (f + 2 < nw) w4.z = wsrc[f + 2];
        if (f + 3 < nw) w4.w = wsrc[f + 3];
      }
      rw[i] = w4;
    }
  };
  auto store_chunk = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + NTH * i;
      if (v < TB * DK / VX) {
        const int tl = v / (DK / VX), dg = v % (DK / VX);
        const uint32_t w4[4] = {rx[i].x, rx[i].y, rx[i].z, rx[i].w};
#pragma unroll
        for (int q = 0; q < VX; ++q) {
          const float val = XBF16 ? __uint_as_float(((q & 1) ? (w4[q >> 1] & 0xFFFF0000u) : (w4[q >> 1] << 16)))
                                  : __uint_as_float(w4[q]);
          xs[buf][VX * dg + q][tl] = val;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int f = 4 * (tid + NTH * i);
      const float vals[4] = {rw[i].x, rw[i].y, rw[i].z, rw[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ff = f + q;
        const int dd = ff / E, e = ff % E;
        if (dd < DK) wsm[buf][dd][e] = vals[q];
      }
    }
  };

  const int nch = (D + DK - 1) / DK;
  // padded experts (E <= e < EP) read zeros: clear those LDS columns once
  for (int q = tid; q < 2 * DK * EP; q += NTH) (&wsm[0][0][0])[q] = 0.0f;
  __syncthreads();
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) load_chunk(c + 1);
    const int dk = min(DK, D - c * DK);
    for (int dd = 0; dd < dk; ++dd) {
      float xv[RT], wv[RE];
#pragma unroll
      for (int i = 0; i < RT; ++i) xv[i] = xs[buf][dd][tt * RT + i];
#pragma unroll
      for (int j = 0; j < RE; ++j) wv[j] = wsm[buf][dd][te + NE * j];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < RE; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
    }
    if (c + 1 < nch) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // Logits of the workgroup's tokens to LDS ([token][expert], reusing the
  // W_r buffers), so that the selection below can walk the tokens with a
  // loop instead of unrolled register indexing.
  static_assert(TB <= 2 * DK, "logit tile must fit in the W_r buffers");
  float* lg = &wsm[0][0][0];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < RE; ++j) lg[(tt * RT + i) * EP + te + NE * j] = acc[i][j];
  __syncthreads();

  select_topk<NE, RE, RT>(a, lg, tt, te, t0);
}

// Few experts (E <= 16): one logit chain per lane, lane (tt, te) = token
// tt, expert te. The chains are too few to need register blocking, so the
// operands are laid out d-contiguous instead: x as [token][d] and W_r
// transposed to [expert][d] (fp32, rows padded by 16 bytes so the lanes'
// rows fall in distinct LDS banks), and each lane takes 4 d per pair of
// 16-byte reads. Chunks of DK are double-buffered as above.
template <int NE, int DK, int NTH, bool XBF16>
__global__ __launch_bounds__(NTH) void router_dv_kernel(RouterArgs a) {
  constexpr int TB = NTH / NE;  // tokens per workgroup
  constexpr int XP = DK + 4;    // padded row, floats
  constexpr int VX = XBF16 ? 8 : 4;
  constexpr int NXV = (TB * DK / VX + NTH - 1) / NTH;  // 16-byte x loads per thread per chunk
  constexpr int NWV = (DK * NE + NTH - 1) / NTH;       // W_r floats per thread per chunk
  static_assert(DK % 4 == 0 && DK % VX == 0, "chunk shape");
  __shared__ __attribute__((aligned(16))) float xs[2][TB][XP];
  __shared__ __attribute__((aligned(16))) float ws[2][NE][XP];

  const int tid = threadIdx.x;
  const int te = tid % NE;
  const int tt = tid / NE;
  const int t0 = blockIdx.x * TB;
  const int D = a.D, E = a.E;

  uint4 rx[NXV];
  float rw[NWV];
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const int d0 = c * DK;
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + NTH * i;
      const int tl = v / (DK / VX), dg = v % (DK / VX);
      const int t = t0 + tl, d = d0 + VX * dg;
      rx[i] = make_uint4(0, 0, 0, 0);
      if (v < TB * DK / VX && t < a.T && d < D)
        rx[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) +
                                                ((size_t)t * D + d) * (XBF16 ? 2 : 4));
    }
    // W_r[d][e] for d in the chunk, e < NE: consecutive threads read
    // consecutive (d, e), i.e. consecutive W_r floats when E == NE
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int f = tid + NTH * i, dd = f / NE, e = f % NE;
      rw[i] = (dd < DK && d0 + dd < D && e < E) ? a.W_r[(size_t)(d0 + dd) * E + e] : 0.0f;
    }
  };
  auto store_chunk = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + NTH * i;
      if (v < TB * DK / VX) {
        const int tl = v / (DK / VX), dg = v % (DK / VX);
        float4* dst = reinterpret_cast<float4*>(&xs[buf][tl][VX * dg]);
        if (XBF16) {
          dst[0] = make_float4(__uint_as_float(rx[i].x << 16), __uint_as_float(rx[i].x & 0xFFFF0000u),
                               __uint_as_float(rx[i].y << 16), __uint_as_float(rx[i].y & 0xFFFF0000u));
          dst[1] = make_float4(__uint_as_float(rx[i].z << 16), __uint_as_float(rx[i].z & 0xFFFF0000u),
                               __uint_as_float(rx[i].w << 16), __uint_as_float(rx[i].w & 0xFFFF0000u));
        } else {
          dst[0] = make_float4(__uint_as_float(rx[i].x), __uint_as_float(rx[i].y),
                               __uint_as_float(rx[i].z), __uint_as_float(rx[i].w));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int f = tid + NTH * i, dd = f / NE, e = f % NE;
      if (dd < DK) ws[buf][e][dd] = rw[i];
    }
  };

  float acc = 0.0f;
  const int nch = (D + DK - 1) / DK;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) load_chunk(c + 1);
    const int dk = min(DK, D - c * DK);  // a multiple of 8
    const float* xr = &xs[buf][tt][0];
    const float* wr = &ws[buf][te][0];
#pragma unroll 4
    for (int dd = 0; dd < dk; dd += 4) {
      const float4 xv = *reinterpret_cast<const float4*>(xr + dd);
      const float4 wv = *reinterpret_cast<const float4*>(wr + dd);
      acc = __builtin_fmaf(xv.x, wv.x, acc);
      acc = __builtin_fmaf(xv.y, wv.y, acc);
      acc = __builtin_fmaf(xv.z, wv.z, acc);
      acc = __builtin_fmaf(xv.w, wv.w, acc);
    }
    if (c + 1 < nch) store_chunk(buf ^ 1);
    __syncthreads();
  }

  float* lg = &ws[0][0][0];  // logit tile [TB][NE]
  lg[tt * NE + te] = acc;
  __syncthreads();
  select_topk<NE, 1, 1>(a, lg, tt, te, t0);
}

template <int NE, int DK, int NTH>
hipError_t launch_dv(const RouterArgs& a, bool xbf16, hipStream_t s) {
  dim3 grid(ceil_div(a.T, NTH / NE));
  if (xbf16)
    router_dv_kernel<NE, DK, NTH, true><<<grid, NTH, 0, s>>>(a);
  else
    router_dv_kernel<NE, DK, NTH, false><<<grid, NTH, 0, s>>>(a);
  return hipGetLastError();
}

template <int NE, int RE, int RT, int DK, int NTH = 256>
hipError_t launch(const RouterArgs& a, bool xbf16, hipStream_t s) {
  constexpr int TB = (NTH / NE) * RT;
  dim3 grid(ceil_div(a.T, TB));
  if (xbf16)
    router_kernel<NE, RE, RT, DK, NTH, true><<<grid, NTH, 0, s>>>(a);
  else
    router_kernel<NE, RE, RT, DK, NTH, false><<<grid, NTH, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const moe_cfg& c, const void* x, const float* W_r, const float* bias,
                         int32_t* idx, float* w, float* logits, hipStream_t s) {
  RouterArgs a{x, W_r, bias, idx, w, logits, c.T, c.D, c.E, c.top_k, c.gating, c.renorm};
  const bool b = c.act_dtype == MOE_BF16;
  // (NE lanes per token, RE experts and RT tokens per lane, DK-deep chunks,
  // threads per workgroup): enough workgroups for every CU and at least two
  // waves per SIMD where the token count allows
  if (c.E <= 8) return launch_dv<8, 512, 128>(a, b, s);
  if (c.E <= 16) return launch_dv<16, 512, 128>(a, b, s);
  if (c.E <= 32) return launch<32, 1, 4, 64>(a, b, s);
  if (c.E <= 64) return launch<64, 1, 8, 64>(a, b, s);
  if (c.E <= 128) return launch<64, 2, 4, 32, 512>(a, b, s);
  if (c.E <= 256) return launch<64, 4, 4, 32, 1024>(a, b, s);
  if (c.E <= 384) return launch<64, 6, 4, 32, 1024>(a, b, s);
  if (c.E <= 512) return launch<64, 8, 8, 16>(a, b, s);
  return launch<64, 16, 4, 16>(a, b, s);
}

}  // namespace moe

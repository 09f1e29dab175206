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
// accumulators in registers (a lane's RE experts are adjacent, so their
// weights arrive in one or two vector LDS reads per d, and its RT tokens'
// x in one broadcast read). A token's experts live in NE adjacent lanes,
// so top-k is a butterfly arg-max over those lanes, k times, with no
// sorting.
#include <math.h>

#include "common.h"
#include "gating.h"
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
    // largest key, and (softmax without renormalisation) the normaliser over
    // all experts, the sum of exp(key - max)
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < RE; ++j) m = fmaxf(m, key[j]);
#pragma unroll
    for (int o = NE / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, NE));
    float Z = 0.0f;
    if (a.gating == MOE_GATE_SOFTMAX && !a.renorm) {
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
        const float wv = gate_weight(a.gating, a.renorm, bk, bl, m, Z);
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
  __shared__ __attribute__((aligned(16))) float xs[2][DK][TB];
  __shared__ __attribute__((aligned(16))) float wsm[2][DK][EP];

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
    if (E == EP && wvec) {
      // the chunk's [DK][E] floats are wsm's own layout: 16-byte stores
#pragma unroll
      for (int i = 0; i < NWV; ++i) {
        const int f = 4 * (tid + NTH * i);
        if (f < DK * EP) *reinterpret_cast<float4*>(&wsm[buf][0][0] + f) = rw[i];
      }
      return;
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
      // the lane's RE experts are adjacent: one or two vector LDS reads
#pragma unroll
      for (int j = 0; j < RE; ++j) wv[j] = wsm[buf][dd][te * RE + j];
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
    for (int j = 0; j < RE; ++j) lg[(tt * RT + i) * EP + te * RE + j] = acc[i][j];
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

// Exactly 8 experts and D <= 4096: the whole W_r ([D][8] fp32, 128 KB) is
// copied into LDS once, by asynchronous global->LDS copies, and x streams
// through a ring of 4 chunks of 4 KB (16 tokens x 128 d bf16, or 64 d
// fp32), also copied asynchronously, so that no register staging or
// transposition sits between the loads and the chains. One lane per chain
// (token tt, expert te); each 16 d take two (bf16) or four (fp32) 16-byte x
// reads, shared by the token's 8 lanes, and eight paired W_r reads (8 lanes
// read 8 consecutive floats), all in flight together. The x rows hold their
// 16-byte groups at slot group ^ (token mod 8), so the 8 tokens of a wave
// read 8 distinct bank groups. The ring is paced by explicit counter waits
// and barriers, and the LDS reads wait for themselves, so that copies of
// later chunks stay in flight while a chunk is summed. With bf16 x the
// reads of the next 16 d are issued before the FMAs of the current 16 d
// (one wave per SIMD cannot hide the read latency otherwise).
constexpr int kE8Tokens = 16;                     // tokens per workgroup (2 waves)
constexpr int kE8Threads = 8 * kE8Tokens;         // one lane per (token, expert)
constexpr int kE8ChunkBytes = 256 * kE8Tokens;    // one x chunk: 256 bytes per token
constexpr int kE8Ring = 4;           // x chunks in the ring
constexpr int kE8MaxD = 4096;        // W_r rows that fit beside the ring

typedef float e8_f2 __attribute__((ext_vector_type(2)));
typedef float e8_f4 __attribute__((ext_vector_type(4)));
typedef unsigned e8_u2 __attribute__((ext_vector_type(2)));
typedef unsigned e8_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t e8_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(p);
}
__device__ __forceinline__ void lds_copy16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <bool XBF16>
__global__ __launch_bounds__(kE8Threads) void router_e8_kernel(RouterArgs a) {
  constexpr int SX = XBF16 ? 2 : 4;
  constexpr int DKX = kE8ChunkBytes / (kE8Tokens * SX);  // d per chunk: 128 or 64
  static_assert(kE8Ring == 4, "the chunk loop is unrolled for 4 ring slots");
  // One array per ring slot, so that the compiler can tell a slot's reads
  // from the copies still in flight into the other slots.
  __shared__ __attribute__((aligned(16))) unsigned char wl[kE8MaxD * 32];
  __shared__ __attribute__((aligned(16))) unsigned char xl0[kE8ChunkBytes];
  __shared__ __attribute__((aligned(16))) unsigned char xl1[kE8ChunkBytes];
  __shared__ __attribute__((aligned(16))) unsigned char xl2[kE8ChunkBytes];
  __shared__ __attribute__((aligned(16))) unsigned char xl3[kE8ChunkBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int te = tid & 7;   // expert
  const int tt = tid >> 3;  // token in the workgroup
  const int t0 = blockIdx.x * kE8Tokens;
  const int D = a.D;
  const int nch = (D + DKX - 1) / DKX;

  // W_r copy: 16-byte pieces p = kE8Threads i + tid of the D * 32 bytes
  const int wpieces = D * 2;
  const int wper = (wpieces + kE8Threads - 1) / kE8Threads;  // the same for every thread
  for (int i = 0; i < wper; ++i) {
    const int p = min(kE8Threads * i + tid, wpieces - 1);
    lds_copy16(reinterpret_cast<const unsigned char*>(a.W_r) + 16 * (size_t)p,
               wl + 16 * (kE8Threads * i + 64 * wave));
  }
  // x chunk c -> its ring slot: LDS piece q = 64 (2 wave + r) + lane holds
  // token q / 16, group (q % 16) ^ (token % 8)
  auto issue_x = [&](int c, unsigned char* slot) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = 64 * (2 * wave + r) + lane;
      const int tk = q >> 4, g = (q & 15) ^ (tk & 7);
      const int t = min(t0 + tk, a.T - 1);
      const int d = min(c * DKX + g * (16 / SX), D - 16 / SX);
      lds_copy16(static_cast<const unsigned char*>(a.x) + ((size_t)t * D + d) * SX,
                 slot + 1024 * (2 * wave + r));
    }
  };
  if (0 < nch) issue_x(0, xl0);
  if (1 < nch) issue_x(1, xl1);
  if (2 < nch) issue_x(2, xl2);

  float acc = 0.0f;
  const unsigned char* wrow = wl + te * 4;
  const int sw = tt & 7;
  // one chunk from `slot`; the copies of chunk c + 3 go to `next`
  auto chunk = [&](int c, const unsigned char* slot, unsigned char* next)
      __attribute__((always_inline)) {
    // chunk c (and the W_r copy, issued first) have landed once at most the
    // later chunks' two copies per thread are in flight
    const int ahead = min(kE8Ring - 2, nch - 1 - c);
    if (ahead >= 2) wait_vm<4>();
    else if (ahead == 1) wait_vm<2>();
    else wait_vm<0>();
    // every thread's copies of chunk c landed; every wave is done with the
    // slot of chunk c - 1, which the copies of chunk c + 3 overwrite
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (c + kE8Ring - 1 < nch) issue_x(c + kE8Ring - 1, next);
    const int dk = min(DKX, D - c * DKX);  // a multiple of 8
    // The LDS reads sit in one asm block that waits for them itself: a
    // plain load would make the compiler wait for every copy in flight,
    // the ring's prefetch included.
    const uint32_t xbase = e8_lds_addr(slot) + tt * 256;
    uint32_t wa = e8_lds_addr(wrow) + (uint32_t)c * DKX * 32;
    int dd = 0;
    if (XBF16 && dk == DKX) {
      // A whole bf16 chunk (8 blocks of 16 d), software-pipelined: each asm
      // block issues the LDS reads of the next 16 d, then runs the unpacks
      // and the 16 FMAs of the current 16 d (in the same order as below:
      // d ascending, one fused multiply-add each), then waits for its
      // reads. Two register sets alternate.
      e8_f2 wA[8], wB[8];
      e8_u4 uA0, uA1, uB0, uB1;
      float tmp;
      auto xa = [&](int blk, int h) { return xbase + (((2 * blk + h) ^ sw) * 16); };
#define E8_RD8(N, ADDR)                                                              \
  "ds_read2_b32 %[" N "0], %[" ADDR "] offset1:8\n\t"                                \
  "ds_read2_b32 %[" N "1], %[" ADDR "] offset0:16 offset1:24\n\t"                    \
  "ds_read2_b32 %[" N "2], %[" ADDR "] offset0:32 offset1:40\n\t"                    \
  "ds_read2_b32 %[" N "3], %[" ADDR "] offset0:48 offset1:56\n\t"                    \
  "ds_read2_b32 %[" N "4], %[" ADDR "] offset0:64 offset1:72\n\t"                    \
  "ds_read2_b32 %[" N "5], %[" ADDR "] offset0:80 offset1:88\n\t"                    \
  "ds_read2_b32 %[" N "6], %[" ADDR "] offset0:96 offset1:104\n\t"                   \
  "ds_read2_b32 %[" N "7], %[" ADDR "] offset0:112 offset1:120\n\t"
#define E8_FMA2(U, I)                                                                \
  "v_lshlrev_b32 %[t], 16, %[" U "]\n\t"                                              \
  "v_fmac_f32 %[acc], %[t], %[w" #I "x]\n\t"                                          \
  "v_and_b32 %[t], 0xffff0000, %[" U "]\n\t"                                          \
  "v_fmac_f32 %[acc], %[t], %[w" #I "y]\n\t"
#define E8_FMAS                                                                      \
  E8_FMA2("u0", 0) E8_FMA2("u1", 1) E8_FMA2("u2", 2) E8_FMA2("u3", 3) E8_FMA2("u4", 4)  \
  E8_FMA2("u5", 5) E8_FMA2("u6", 6) E8_FMA2("u7", 7)
#define E8_CUR(W, U0, U1)                                                            \
  [u0] "v"(U0.x), [u1] "v"(U0.y), [u2] "v"(U0.z), [u3] "v"(U0.w), [u4] "v"(U1.x),      \
      [u5] "v"(U1.y), [u6] "v"(U1.z), [u7] "v"(U1.w), [w0x] "v"(W[0].x),               \
      [w0y] "v"(W[0].y), [w1x] "v"(W[1].x), [w1y] "v"(W[1].y), [w2x] "v"(W[2].x),      \
      [w2y] "v"(W[2].y), [w3x] "v"(W[3].x), [w3y] "v"(W[3].y), [w4x] "v"(W[4].x),      \
      [w4y] "v"(W[4].y), [w5x] "v"(W[5].x), [w5y] "v"(W[5].y), [w6x] "v"(W[6].x),      \
      [w6y] "v"(W[6].y), [w7x] "v"(W[7].x), [w7y] "v"(W[7].y)
#define E8_NEXT(W, U0, U1)                                                           \
  [n0] "=&v"(W[0]), [n1] "=&v"(W[1]), [n2] "=&v"(W[2]), [n3] "=&v"(W[3]),              \
      [n4] "=&v"(W[4]), [n5] "=&v"(W[5]), [n6] "=&v"(W[6]), [n7] "=&v"(W[7]),          \
      [nu0] "=&v"(U0), [nu1] "=&v"(U1)
      // reads of block BLK into (NW, NU0, NU1) while block BLK - 1 in (CW,
      // CU0, CU1) is summed
#define E8_STEP(BLK, NW, NU0, NU1, CW, CU0, CU1)                                     \
  asm volatile(E8_RD8("n", "na") "ds_read_b128 %[nu0], %[nx0]\n\t"                   \
               "ds_read_b128 %[nu1], %[nx1]\n\t" E8_FMAS "s_waitcnt lgkmcnt(0)"         \
               : E8_NEXT(NW, NU0, NU1), [acc] "+v"(acc), [t] "=&v"(tmp)               \
               : E8_CUR(CW, CU0, CU1), [na] "v"(wa + 512 * (BLK)),                    \
                 [nx0] "v"(xa(BLK, 0)), [nx1] "v"(xa(BLK, 1)))
      asm volatile(E8_RD8("n", "na") "ds_read_b128 %[nu0], %[nx0]\n\t"
                   "ds_read_b128 %[nu1], %[nx1]\n\ts_waitcnt lgkmcnt(0)"
                   : E8_NEXT(wA, uA0, uA1)
                   : [na] "v"(wa), [nx0] "v"(xa(0, 0)), [nx1] "v"(xa(0, 1)));
      E8_STEP(1, wB, uB0, uB1, wA, uA0, uA1);
      E8_STEP(2, wA, uA0, uA1, wB, uB0, uB1);
      E8_STEP(3, wB, uB0, uB1, wA, uA0, uA1);
      E8_STEP(4, wA, uA0, uA1, wB, uB0, uB1);
      E8_STEP(5, wB, uB0, uB1, wA, uA0, uA1);
      E8_STEP(6, wA, uA0, uA1, wB, uB0, uB1);
      E8_STEP(7, wB, uB0, uB1, wA, uA0, uA1);
      asm volatile(E8_FMAS : [acc] "+v"(acc), [t] "=&v"(tmp) : E8_CUR(wB, uB0, uB1));
#undef E8_STEP
#undef E8_NEXT
#undef E8_CUR
#undef E8_FMAS
#undef E8_FMA2
#undef E8_RD8
      static_assert(!XBF16 || DKX == 128, "the pipelined path covers 8 blocks of 16 d");
      dd = dk;
    }
    // 16 d per block: 8 W_r pairs and 16 x values in flight at once
    for (; dd + 16 <= dk; dd += 16, wa += 512) {
      const int g = dd / (16 / SX);
      e8_f2 w[8];
      float xv[16];
      if (XBF16) {
        e8_u4 u0, u1;
        asm volatile(
            "ds_read2_b32 %0, %10 offset1:8\n\t"
            "ds_read2_b32 %1, %10 offset0:16 offset1:24\n\t"
            "ds_read2_b32 %2, %10 offset0:32 offset1:40\n\t"
            "ds_read2_b32 %3, %10 offset0:48 offset1:56\n\t"
            "ds_read2_b32 %4, %10 offset0:64 offset1:72\n\t"
            "ds_read2_b32 %5, %10 offset0:80 offset1:88\n\t"
            "ds_read2_b32 %6, %10 offset0:96 offset1:104\n\t"
            "ds_read2_b32 %7, %10 offset0:112 offset1:120\n\t"
            "ds_read_b128 %8, %11\n\t"
            "ds_read_b128 %9, %12\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(w[0]), "=v"(w[1]), "=v"(w[2]), "=v"(w[3]), "=v"(w[4]), "=v"(w[5]),
              "=v"(w[6]), "=v"(w[7]), "=v"(u0), "=v"(u1)
            : "v"(wa), "v"(xbase + ((g ^ sw) * 16)), "v"(xbase + (((g + 1) ^ sw) * 16)));
        const unsigned uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xv[2 * i] = __uint_as_float(uu[i] << 16);
          xv[2 * i + 1] = __uint_as_float(uu[i] & 0xFFFF0000u);
        }
      } else {
        e8_f4 f0, f1, f2, f3;
        asm volatile(
            "ds_read2_b32 %0, %12 offset1:8\n\t"
            "ds_read2_b32 %1, %12 offset0:16 offset1:24\n\t"
            "ds_read2_b32 %2, %12 offset0:32 offset1:40\n\t"
            "ds_read2_b32 %3, %12 offset0:48 offset1:56\n\t"
            "ds_read2_b32 %4, %12 offset0:64 offset1:72\n\t"
            "ds_read2_b32 %5, %12 offset0:80 offset1:88\n\t"
            "ds_read2_b32 %6, %12 offset0:96 offset1:104\n\t"
            "ds_read2_b32 %7, %12 offset0:112 offset1:120\n\t"
            "ds_read_b128 %8, %13\n\t"
            "ds_read_b128 %9, %14\n\t"
            "ds_read_b128 %10, %15\n\t"
            "ds_read_b128 %11, %16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(w[0]), "=v"(w[1]), "=v"(w[2]), "=v"(w[3]), "=v"(w[4]), "=v"(w[5]),
              "=v"(w[6]), "=v"(w[7]), "=v"(f0), "=v"(f1), "=v"(f2), "=v"(f3)
            : "v"(wa), "v"(xbase + ((g ^ sw) * 16)), "v"(xbase + (((g + 1) ^ sw) * 16)),
              "v"(xbase + (((g + 2) ^ sw) * 16)), "v"(xbase + (((g + 3) ^ sw) * 16)));
        const e8_f4 ff[4] = {f0, f1, f2, f3};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[4 * i] = ff[i].x;
          xv[4 * i + 1] = ff[i].y;
          xv[4 * i + 2] = ff[i].z;
          xv[4 * i + 3] = ff[i].w;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc = __builtin_fmaf(xv[2 * i], w[i].x, acc);
        acc = __builtin_fmaf(xv[2 * i + 1], w[i].y, acc);
      }
    }
    for (; dd < dk; dd += 4, wa += 128) {
      const int g = dd / (16 / SX), within = (dd % (16 / SX)) * SX;
      const uint32_t xa = xbase + ((g ^ sw) * 16) + within;
      e8_f2 w01, w23;
      float xv[4];
      if (XBF16) {
        e8_u2 u;
        asm volatile(
            "ds_read2_b32 %0, %3 offset1:8\n\t"
            "ds_read2_b32 %1, %3 offset0:16 offset1:24\n\t"
            "ds_read_b64 %2, %4\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(w01), "=v"(w23), "=v"(u)
            : "v"(wa), "v"(xa));
        xv[0] = __uint_as_float(u.x << 16);
        xv[1] = __uint_as_float(u.x & 0xFFFF0000u);
        xv[2] = __uint_as_float(u.y << 16);
        xv[3] = __uint_as_float(u.y & 0xFFFF0000u);
      } else {
        e8_f4 f;
        asm volatile(
            "ds_read2_b32 %0, %3 offset1:8\n\t"
            "ds_read2_b32 %1, %3 offset0:16 offset1:24\n\t"
            "ds_read_b128 %2, %4\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(w01), "=v"(w23), "=v"(f)
            : "v"(wa), "v"(xa));
        xv[0] = f.x;
        xv[1] = f.y;
        xv[2] = f.z;
        xv[3] = f.w;
      }
      acc = __builtin_fmaf(xv[0], w01.x, acc);
      acc = __builtin_fmaf(xv[1], w01.y, acc);
      acc = __builtin_fmaf(xv[2], w23.x, acc);
      acc = __builtin_fmaf(xv[3], w23.y, acc);
    }
  };
  for (int c = 0; c < nch; c += 4) {
    chunk(c, xl0, xl3);
    if (c + 1 < nch) chunk(c + 1, xl1, xl0);
    if (c + 2 < nch) chunk(c + 2, xl2, xl1);
    if (c + 3 < nch) chunk(c + 3, xl3, xl2);
  }

  __syncthreads();  // every wave done with the ring
  float* lg = reinterpret_cast<float*>(xl0);  // logit tile [32][8]
  lg[tt * 8 + te] = acc;
  __syncthreads();
  select_topk<8, 1, 1>(a, lg, tt, te, t0);
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
  if (c.E == 8 && c.D <= kE8MaxD) {
    dim3 grid(ceil_div(c.T, kE8Tokens));
    if (b) router_e8_kernel<true><<<grid, kE8Threads, 0, s>>>(a);
    else router_e8_kernel<false><<<grid, kE8Threads, 0, s>>>(a);
    return hipGetLastError();
  }
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

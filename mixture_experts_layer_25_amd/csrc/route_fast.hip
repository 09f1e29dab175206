// Screened router for many experts: the same indices and weights as the
// exact router (router.hip), with most of its fp32 FMA chains skipped.
//
// "ops-transformer MoE operator on Ascend NPU", pitfall 3: the router runs
// in FP32, and its performance comparison counts routing and top-k among
// the overheads; "FFN, SwiGLU and MoE" sec. 3: r = W_r x, the k largest.
// Each logit is defined as one fp32 fused multiply-add chain over d
// ascending (the order that makes the selection bit-reproducible). With
// hundreds of experts, computing every chain costs T*E*D FMAs on the vector
// ALUs. Only the chains of experts that can reach a token's top k are
// needed, and which those are can be decided from a cheaper estimate with a
// rigorous error bound:
//
//   1. prep:   W_r [D][E] -> W_r^T [E][D] fp32 (rows for the exact chains)
//              and bf16(W_r)^T (the MFMA operand); per expert the 2-norms
//              of the weights and of the bf16 residual, their maxima N, R.
//   2. screen: a_e = x . bf16(w_e) on the bf16 MFMA (products exact in
//              fp32, fp32 accumulation), and ||x_t||^2 in double.
//   3. cand:   per token, approximate keys ka_e = a_e + bias_e, A = the
//              k-th largest; candidates = experts with ka_e >= A - 2 eps_t.
//   4. exact:  the exact chains of the candidates only.
//   5. select: top k of the candidates' exact keys, ties to the lower
//              index, and the weights, by the exact router's order and
//              gate_weight.
//
// The bound. Let c_e be the exact chain (the defined logit) and t_e the
// real dot product. For an fp32 FMA chain |c_e - t_e| <= g_D sum_d |x_d
// w_de| with g_D = D u / (1 - D u), u = 2^-24. The screen's products are
// exact; its accumulation error is bounded here by twice the same bound
// (an allowance for truncating or reordered accumulation inside the MFMA,
// whose summation order is not specified; a k-split into two halves of D
// added in fp32 is one more such order) and once more for safety, and the
// bf16 residual adds |sum_d x_d (h_de - w_de)| <= ||x_t|| ||r_e||. With
// sum |x_d w_de| <= ||x_t|| ||w_e|| and |h| <= (1 + 2^-8) |w|:
//   |a_e - c_e| <= eps_t = ||x_t|| (R + 5 g_D (1 + 2^-8) N),
// widened for the fp32 additions of the bias to the two keys. If an expert
// e is in the exact top k, its key k_e >= K_k (the k-th largest exact key);
// the k experts with the largest approximate keys have exact keys >= A -
// eps, so K_k >= A - eps, hence ka_e >= k_e - eps >= A - 2 eps: e is a
// candidate. A non-candidate has k_e <= ka_e + eps < A - eps <= K_k, below
// the k-th key even with ties, so it is never selected. The candidate
// threshold is compared in double. Inputs are assumed finite.
#include <math.h>

#include <type_traits>
#include <utility>

#include "common.h"
#include "gating.h"
#include "gemm_tile.h"
#include "launch.h"

namespace moe {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16v8_t __attribute__((ext_vector_type(8)));

constexpr int kMaxK = 16;
constexpr int kScrTM = 64;    // screen tile: tokens (experts: 64 or 128)
// exact chains: tokens x experts per workgroup (16384 tokens x 384
// experts: 64 x 4 workgroups; 8192 x 128: 128 x 4)
struct ExTile {
  int tb, er;
};
inline ExTile ex_tile(int E) { return E >= 256 ? ExTile{256, 96} : ExTile{64, 32}; }
constexpr int kExDK = 64;     // exact chains: d per staged chunk

struct ScreenWs {
  uint16_t* whi;   // bf16(W_r)^T [E][D]
  float* wt;       // W_r^T [E][D]
  unsigned long long* wmax;  // [0] = N (max ||w_e||), [1] = R (max ||r_e||), as double bits
  float* S;        // approximate logits [T][E]
  double* nx2;     // ||x_t||^2 [T]
  int16_t* cand;   // candidates of token t: cand[t][0..ncand[t]), ascending
  int32_t* ncand;  // [T]
  float* exl;      // exact logit of candidate slot i of token t: [T][E]
  float* exk;      // its key (logit + bias) [T][E]
  int32_t* gpairs; // per exact-chain workgroup: its pairs listed by expert
  size_t bytes;
};

// k-split of the screen GEMM: two halves of D (summed in order by the
// candidate kernel) when its tiles alone would give under two workgroups
// per CU
int screen_ksplit(const moe_cfg& c) {
  const long long tiles = (long long)ceil_div(c.T, kScrTM) * ceil_div(c.E, c.E <= 128 ? 64 : 128);
  return tiles < 512 && c.D >= 64 * 32 ? 2 : 1;
}

ScreenWs carve(const moe_cfg& c, void* base) {
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    off = align_up(off, 256);
    char* r = p ? p + off : nullptr;
    off += n;
    return r;
  };
  const size_t ED = (size_t)c.E * c.D, TE = (size_t)c.T * c.E;
  ScreenWs w;
  w.whi = reinterpret_cast<uint16_t*>(take(ED * 2));
  w.wt = reinterpret_cast<float*>(take(ED * 4));
  w.wmax = reinterpret_cast<unsigned long long*>(take(16));
  const int ks = screen_ksplit(c);
  w.S = reinterpret_cast<float*>(take(ks * TE * 4));
  w.nx2 = reinterpret_cast<double*>(take((size_t)ks * c.T * 8));
  w.cand = reinterpret_cast<int16_t*>(take(TE * 2));
  w.ncand = reinterpret_cast<int32_t*>(take((size_t)c.T * 4));
  w.exl = reinterpret_cast<float*>(take(TE * 4));
  w.exk = reinterpret_cast<float*>(take(TE * 4));
  w.gpairs = reinterpret_cast<int32_t*>(
      take((size_t)ceil_div(c.T, ex_tile(c.E).tb) * ex_tile(c.E).tb * ceil_div(c.E, ex_tile(c.E).er) *
           ex_tile(c.E).er * 4));
  w.bytes = align_up(off, 256);
  return w;
}

// ---- 1. prep: transpose W_r (32 x 32 tiles through LDS), bf16 copy
__global__ __launch_bounds__(256) void screen_prep_kernel(const float* __restrict__ W_r, int D,
                                                          int E, float* __restrict__ wt,
                                                          uint16_t* __restrict__ whi,
                                                          unsigned long long* __restrict__ wmax) {
  __shared__ float tile[32][33];
  const int e0 = blockIdx.x * 32, d0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 2) wmax[threadIdx.x] = 0ull;
  for (int r = ty; r < 32; r += 8) {
    const int d = d0 + r, e = e0 + tx;
    tile[r][tx] = (d < D && e < E) ? W_r[(size_t)d * E + e] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, d = d0 + tx;
    if (e < E && d < D) {
      const float v = tile[tx][r];
      wt[(size_t)e * D + d] = v;
      whi[(size_t)e * D + d] = (uint16_t)f32_to_bf16(v);
    }
  }
}

// per expert (one workgroup): ||w_e||, ||w_e - bf16(w_e)|| in double
// (squares of fp32 values and of their bf16 residuals are exact in double;
// the sums, in a fixed order, and the roots are rounded up by a relative
// 2^-40), then the maxima over experts (positive doubles order like their
// bit patterns)
__global__ __launch_bounds__(256) void screen_norms_kernel(const float* __restrict__ wt,
                                                           const uint16_t* __restrict__ whi,
                                                           int D, int E,
                                                           unsigned long long* __restrict__ wmax) {
  __shared__ double part[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  double sw = 0.0, sr = 0.0;
  for (int d = 4 * tid; d < D; d += 1024) {
    const float4 w4 = *reinterpret_cast<const float4*>(wt + (size_t)e * D + d);
    const uint2 h4 = *reinterpret_cast<const uint2*>(whi + (size_t)e * D + d);
    const float w[4] = {w4.x, w4.y, w4.z, w4.w};
    const float h[4] = {__uint_as_float(h4.x << 16), __uint_as_float(h4.x & 0xFFFF0000u),
                        __uint_as_float(h4.y << 16), __uint_as_float(h4.y & 0xFFFF0000u)};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double wd = w[q], rd = wd - (double)h[q];
      sw += wd * wd;
      sr += rd * rd;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sw += __shfl_xor(sw, o, 64);
    sr += __shfl_xor(sr, o, 64);
  }
  if (lane == 0) {
    part[0][wave] = sw;
    part[1][wave] = sr;
  }
  __syncthreads();
  if (tid == 0) {
    const double up = 1.0 + 0x1p-40;
    const double tw = (part[0][0] + part[0][1]) + (part[0][2] + part[0][3]);
    const double tr = (part[1][0] + part[1][1]) + (part[1][2] + part[1][3]);
    atomicMax(&wmax[0], (unsigned long long)__double_as_longlong(sqrt(tw) * up));
    atomicMax(&wmax[1], (unsigned long long)__double_as_longlong(sqrt(tr) * up));
  }
}

// ---- 2. screen: S = x . bf16(W_r) on v_mfma_f32_16x16x32_bf16. Tile 64
// tokens x TN experts (128, or 64 for at most 128 experts), 4 waves, wave w
// owns experts (TN/4) w .. of the tile (4 x TN/64 MFMA tiles). Operands go
// straight from global memory to LDS (global_load_lds, 16 bytes a lane) in
// steps of 32 k, NS steps in a ring with NS - 1 in flight; a step holds 64
// A rows and TN W^T rows of 64 bytes each, k-group g of row r at slot
// g ^ ((r >> 2) & 3) (the lane that copies a slot fetches that k-group), so
// that the 16 lanes of a fragment read, rows r..r+15 of one k-group, hit 16
// distinct 16-byte bank groups. Lane l supplies row l%16 of A and column
// l%16 of B with k = 8 (l/16) .. +7 and holds rows 4 (l/16) + r of column
// l%16 of the 16 x 16 result. The token tile's workgroups also sum x_t^2 in
// double: wave w of expert tile w mod (expert tiles) over rows 16 w ..
// 16 w + 15 of its A fragments, then the 4 lanes of a row.
template <int TN>
__global__ __launch_bounds__(256) void screen_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ whi,
                                                          int T, int D, int E,
                                                          float* __restrict__ S,
                                                          double* __restrict__ nx2) {
  constexpr int NS = 4;                        // ring of steps (48 or 32 KB)
  constexpr int AB = kScrTM * 64, SB = AB + TN * 64;
  constexpr int PER = 1 + TN / 64;             // 16-byte copies per thread per step
  constexpr int NJ = TN / 64;                  // 16-column MFMA tiles per wave
  __shared__ __attribute__((aligned(1024))) unsigned char sm[NS * SB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * kScrTM, e0 = blockIdx.y * TN;
  // k-split z = blockIdx.z of gridDim.z: steps [k0, k0 + nk) of the D / 32,
  // partial sums to S and nx2 slice z
  const int nkd = D / 32, per = (nkd + gridDim.z - 1) / gridDim.z;
  const int k0 = blockIdx.z * per, nk = min(nkd, k0 + per) - k0;
  S += (size_t)blockIdx.z * T * E;
  nx2 += (size_t)blockIdx.z * T;
  // the copies: this lane's row of A (and of each W^T quarter) and k-group
  const int cr = 16 * wave + (lane >> 2), cs = lane & 3;
  const uint16_t* ag =
      x + (size_t)min(t0 + cr, T - 1) * D + 32 * k0 + 8 * (cs ^ ((cr >> 2) & 3));
  const uint16_t* bg[NJ];
#pragma unroll
  for (int q = 0; q < NJ; ++q) {
    const int r = 64 * q + cr;
    bg[q] = whi + (size_t)min(e0 + r, E - 1) * D + 32 * k0 + 8 * (cs ^ ((r >> 2) & 3));
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    unsigned char* st = sm + (kt % NS) * SB;
    dma16(ag + 32 * kt, st + 1024 * wave);
#pragma unroll
    for (int q = 0; q < NJ; ++q) dma16(bg[q] + 32 * kt, st + AB + 4096 * q + 1024 * wave);
  };
  // wave w's 16 rows are summed by the expert tile w mod gridDim.y, so the
  // double-precision squares are spread over the token tile's workgroups
  const bool norm = (int)(wave % gridDim.y) == (int)blockIdx.y;
  double sq = 0.0;
  f32x4_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int l16 = lane & 15, g = lane >> 4;
  const int rs = 16 * (g ^ ((l16 >> 2) & 3));  // rows 16 i + l16 share bits 2-3 of l16
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_copy_groups<PER>(min(NS - 2, nk - 1 - kt));
    __syncthreads();  // step kt in LDS for every lane; step kt - 1 read by every wave
    if (kt + NS - 1 < nk) issue(kt + NS - 1);
    const unsigned char* st = sm + (kt % NS) * SB;
    bf16v8_t a[4], b[NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16v8_t*>(st + (16 * i + l16) * 64 + rs);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      b[j] = *reinterpret_cast<const bf16v8_t*>(st + AB + ((TN / 4) * wave + 16 * j + l16) * 64 + rs);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    if (norm) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + (16 * wave + l16) * 64 + rs);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double lo = __uint_as_float(v[q] << 16), hi = __uint_as_float(v[q] & 0xFFFF0000u);
        sq += lo * lo;
        sq += hi * hi;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * i + 4 * g + r, e = e0 + (TN / 4) * wave + 16 * j + l16;
        if (t < T && e < E) S[(size_t)t * E + e] = acc[i][j][r];
      }
  if (norm) {
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    const int t = t0 + 16 * wave + l16;
    if (g == 0 && t < T) nx2[t] = sq;
  }
}

// ---- 3. candidates: one wave per token; lane l holds experts l + 64 j
// (coalesced reads); for j ascending a ballot gives the wave's candidates
// among experts 64 j .. 64 j + 63 in lane order, so the list comes out in
// ascending expert order
template <int NJ>
__global__ __launch_bounds__(256) void screen_cand_kernel(
    const float* __restrict__ S, const double* __restrict__ nx2, const float* __restrict__ bias,
    const unsigned long long* __restrict__ wmax, double cg, int ks, int T, int E, int k,
    int16_t* __restrict__ cand, int32_t* __restrict__ ncand) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nj = (E + 63) / 64;
  float ka[NJ];
  bool avail[NJ];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    avail[j] = j < nj && e < E;
    float a = 0.0f;
    if (avail[j]) {
      a = S[(size_t)t * E + e];
      for (int z = 1; z < ks; ++z) a += S[((size_t)z * T + t) * E + e];  // k-split parts in order
    }
    ka[j] = avail[j] ? a + (bias ? bias[e] : 0.0f) : -INFINITY;
    if (avail[j]) amax = fmaxf(amax, fabsf(ka[j]));
  }
  double nxt = nx2[t];
  for (int z = 1; z < ks; ++z) nxt += nx2[(size_t)z * T + t];
  const double N = __longlong_as_double((long long)wmax[0]);
  const double R = __longlong_as_double((long long)wmax[1]);
  // the k-th largest approximate key: the largest order-preserving code U
  // of a key such that at least k keys have codes >= U, found bit by bit
  // from the top (every count is a sum of ballots, uniform across the wave)
  uint32_t code[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t b = __float_as_uint(ka[j]);
    code[j] = avail[j] ? ((b >> 31) ? ~b : (b | 0x80000000u)) : 0u;
  }
  uint32_t U = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = U | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(code[j] >= c));
    if (cnt >= k) U = c;
  }
  const float A = __uint_as_float((U >> 31) ? (U & 0x7FFFFFFFu) : ~U);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  // eps_t and the threshold, in double (cg = 5 g_D (1 + 2^-8), from the host)
  const double nx = sqrt(nxt * (1.0 + 0x1p-40)) * (1.0 + 0x1p-50);
  const double eps = nx * (R + cg * N);
  const double epsk = eps * (1.0 + 0x1p-20) + 0x1p-21 * ((double)amax + eps) + 1e-30;
  const double theta = (double)A - 2.0 * epsk;
  int16_t* out = cand + (size_t)t * E;
  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j < nj) {
      const bool c = avail[j] && (double)ka[j] >= theta;
      const unsigned long long m = __ballot(c);
      if (c) out[base + __popcll(m & below)] = (int16_t)(lane + 64 * j);
      base += __popcll(m);
    }
  }
  if (lane == 0) ncand[t] = base;
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <class F, int... S>
__device__ __forceinline__ void for_each_index_(F&& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void for_each_index(F&& f) {
  for_each_index_(f, std::make_integer_sequence<int, N>{});
}

// ---- 4. exact chains of the candidates. Workgroup = TB tokens x ERX
// experts (a tile this large lets each staged row serve several pairs;
// 256 x 96 from 256 experts, 64 x 32 below). The block's candidate pairs
// are counted per expert and listed by expert (in the workspace); a unit is
// one expert and up to UT of its candidate tokens, so a thread runs UT
// independent chains that read the expert's weights once per 8 d. The x
// rows of the block and the W_r^T rows of the expert range stream through
// LDS in chunks of 64 d; each chain runs d ascending from +0, one fused
// multiply-add per term (the definition of the logit). The logit and the
// key (logit + bias, one fp32 add) go to the pair's slot in its token's
// candidate list. More units than threads: further passes over d.
//
// The time goes to the chains themselves (a variant without them runs in
// 14-22 us of the 75-155): UT chains per lane, each an unpack and an FMA
// per term. A token keeps about 14 candidates of 128 or 384 experts, so a
// 64 x 32 tile holds about 220 pairs and a 256 x 96 tile about 940. The
// small tiles run one chain per unit (UT = 1); the large ones three, with
// the units dealt round-robin to waves 0..3 and then 4..7 (BAL). Measured
// against the other unit sizes, prefetch depths and dealings (4 chains,
// 2 chains, consecutive units per wave): these were the fastest.
template <int TB, int ERX, int UT, int PF, bool BAL>
__global__ __launch_bounds__(512) void screen_exact_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wt, const float* __restrict__ bias,
    const int16_t* __restrict__ cand, const int32_t* __restrict__ ncand, int T, int D, int E,
    int32_t* __restrict__ gpairs, float* __restrict__ exl, float* __restrict__ exk) {
  constexpr int DK = kExDK, NTH = 512;
  static_assert(TB <= 256 && TB <= NTH && ERX <= NTH, "pair encoding and list build");
  constexpr int XP = DK + 8;  // bf16 row, padded to 144 bytes
  constexpr int WP = DK + 4;  // fp32 row, padded to 272 bytes
  constexpr int NXV = TB * DK / 8 / NTH;    // 16-byte x pieces per thread per chunk
  constexpr int NWV = ERX * DK / 4 / NTH;   // 16-byte W pieces per thread per chunk
  static_assert(NXV * NTH * 8 == TB * DK && NWV * NTH * 4 == ERX * DK, "chunk shape");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][TB][XP];
  __shared__ __attribute__((aligned(16))) float ws[2][ERX][WP];
  __shared__ int cnt[ERX], seg[ERX + 1], ucum[ERX + 1];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TB, e0 = blockIdx.y * ERX;
  int32_t* pl = gpairs + (size_t)(blockIdx.y * gridDim.x + blockIdx.x) * TB * ERX;

  // ---- the block's pairs, listed by expert: pl[seg[e] ..] = token | slot << 8
  if (tid < ERX) cnt[tid] = 0;
  __syncthreads();
  const int my_t = t0 + tid;
  const bool has_t = tid < TB && my_t < T;
  const int nc = has_t ? ncand[my_t] : 0;
  const int16_t* cl = cand + (size_t)(has_t ? my_t : 0) * E;
  for (int i = 0; i < nc; ++i) {
    const int e = cl[i];
    if (e >= e0 + ERX) break;  // ascending
    if (e >= e0) atomicAdd(&cnt[e - e0], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0, b = 0;
    for (int e = 0; e < ERX; ++e) {
      const int v = cnt[e];
      seg[e] = a;
      ucum[e] = b;
      cnt[e] = a;  // the expert's cursor
      a += v;
      b += (v + UT - 1) / UT;
    }
    seg[ERX] = a;
    ucum[ERX] = b;
  }
  __syncthreads();
  for (int i = 0; i < nc; ++i) {
    const int e = cl[i];
    if (e >= e0 + ERX) break;
    if (e >= e0) pl[atomicAdd(&cnt[e - e0], 1)] = tid | (i << 8);
  }
  __syncthreads();  // orders the list's global writes before its reads in this workgroup
  const int nunits = ucum[ERX];
  if (nunits == 0) return;

  // ---- chunk staging: global -> registers -> LDS. The LDS holds two
  // chunks (the one being read and the next); the registers hold the next
  // PF chunks, whose loads are issued PF chunks ahead so that the latency
  // of a load from L2 or memory (1-2 us) spreads over PF chunks of chains.
  // Every step issues the same loads, unconditionally: chunk indices past
  // the end, d past D (the second half of a last 32-d chunk) and tokens or
  // experts past the tile's end are clamped to valid addresses and their
  // data is never read, so the compiler's wait before a chunk's LDS store
  // counts only the PF - 1 younger chunks, never all of them.
  const int nch = (D + DK - 1) / DK;
  u32x4_t rx[PF][NXV], rw[PF][NWV];  // native vectors: kept in registers
  auto load_chunk = [&](int c, u32x4_t(&qx)[NXV], u32x4_t(&qw)[NWV]) __attribute__((always_inline)) {
    const int d0 = min(c, nch - 1) * DK;
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + NTH * i, tl = v / (DK / 8), dg = v % (DK / 8);
      const int t = min(t0 + tl, T - 1), d = d0 + 8 * dg;
      qx[i] = *reinterpret_cast<const u32x4_t*>(x + (size_t)t * D + min(d, D - 8));
    }
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int v = tid + NTH * i, el = v / (DK / 4), dg = v % (DK / 4);
      const int e = min(e0 + el, E - 1), d = d0 + 4 * dg;
      qw[i] = *reinterpret_cast<const u32x4_t*>(wt + (size_t)e * D + min(d, D - 4));
    }
  };
  auto store_chunk = [&](int buf, const u32x4_t(&qx)[NXV], const u32x4_t(&qw)[NWV])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int v = tid + NTH * i, tl = v / (DK / 8), dg = v % (DK / 8);
      *reinterpret_cast<u32x4_t*>(&xs[buf][tl][8 * dg]) = qx[i];
    }
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      const int v = tid + NTH * i, el = v / (DK / 4), dg = v % (DK / 4);
      *reinterpret_cast<u32x4_t*>(&ws[buf][el][4 * dg]) = qw[i];
    }
  };

  for (int u0 = 0; u0 < nunits; u0 += NTH) {
    // units u0 .. u0 + 255 go round-robin to waves 0..3 (one per SIMD),
    // the next 256 to waves 4..7
    const int wv = tid >> 6;
    const int un = BAL ? u0 + (wv >> 2) * 256 + (tid & 63) * 4 + (wv & 3) : u0 + tid;
    const bool mine = un < nunits;
    // the unit's expert: the last el with ucum[el] <= un
    int el = 0;
    if (mine) {
      int lo = 0, hi = ERX;  // ucum[lo] <= un < ucum[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ucum[mid] <= un) lo = mid;
        else hi = mid;
      }
      el = lo;
    }
    const int first = seg[el] + UT * (un - ucum[el]);
    const int nt = mine ? min(UT, seg[el + 1] - first) : 0;
    int tl[UT], sl[UT];
#pragma unroll
    for (int i = 0; i < UT; ++i) {
      const int p = nt > 0 ? pl[first + min(i, nt - 1)] : 0;
      tl[i] = p & 0xFF;
      sl[i] = p >> 8;
    }
    float acc[UT];
#pragma unroll
    for (int i = 0; i < UT; ++i) acc[i] = 0.0f;
    // chunk c sits in register slot c % PF until it is stored to LDS; the
    // slots are named by compile-time indices (unrolled through
    // for_each_index) so that they stay in registers
    for_each_index<PF>([&](auto si) __attribute__((always_inline)) {
      constexpr int s = decltype(si)::value;
      load_chunk(s, rx[s], rw[s]);
    });
    store_chunk(0, rx[0], rw[0]);
    __syncthreads();
    for (int cb = 0; cb < nch; cb += PF) {
      for_each_index<PF>([&](auto si) __attribute__((always_inline)) {
        constexpr int s = decltype(si)::value;
        const int c = cb + s;
        // slot s (chunk c) went to LDS before this step: refill it
        load_chunk(c + PF, rx[s], rw[s]);
        if (c < nch) {
          const int buf = c & 1;
          if (mine) {
            const float* wr = &ws[buf][el][0];
            // 8 d per step: one 16-byte x read per chain, two W reads shared
            // by the unit's chains (8-byte x reads: 3-4 % slower)
            auto step = [&](int dd) __attribute__((always_inline)) {
              const float4 w0 = *reinterpret_cast<const float4*>(wr + dd);
              const float4 w1 = *reinterpret_cast<const float4*>(wr + dd + 4);
#pragma unroll
              for (int i = 0; i < UT; ++i) {
                const uint4 xv = *reinterpret_cast<const uint4*>(&xs[buf][tl[i]][dd]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.x << 16), w0.x, acc[i]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.x & 0xFFFF0000u), w0.y, acc[i]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.y << 16), w0.z, acc[i]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.y & 0xFFFF0000u), w0.w, acc[i]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.z << 16), w1.x, acc[i]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.z & 0xFFFF0000u), w1.y, acc[i]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.w << 16), w1.z, acc[i]);
                acc[i] = __builtin_fmaf(__uint_as_float(xv.w & 0xFFFF0000u), w1.w, acc[i]);
              }
            };
            const int dk = min(DK, D - c * DK);  // 64, or 32 for a last chunk
#pragma unroll 2
            for (int dd = 0; dd < dk; dd += 8) step(dd);
          }
          if (c + 1 < nch) store_chunk(buf ^ 1, rx[(s + 1) % PF], rw[(s + 1) % PF]);
          __syncthreads();
        }
      });
    }
    const float b = bias ? bias[e0 + el] : 0.0f;
#pragma unroll
    for (int i = 0; i < UT; ++i)
      if (i < nt) {
        const size_t q = (size_t)(t0 + tl[i]) * E + sl[i];
        exl[q] = acc[i];
        exk[q] = acc[i] + b;
      }
  }
}

// ---- 5. selection among the candidates (one wave per token): a larger key
// (logit + bias) ranks first, an equal key goes to the lower expert index,
// as in the exact router; the candidates of rank 0 .. k-1 are selected in
// that order, with weights by gate_weight (m = the largest key; softmax is
// always renormalised here) and their sum taken in selection order.
// Tokens with at most 64 candidates: lane i holds candidate i and counts the
// candidates ahead of it (its rank).
__global__ __launch_bounds__(256) void screen_select64_kernel(
    const int16_t* __restrict__ cand, const int32_t* __restrict__ ncand,
    const float* __restrict__ exl, const float* __restrict__ exk, int T, int E, int k,
    int gating, int renorm, int32_t* __restrict__ idx, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int n = ncand[t];
  if (n > 64) return;  // the other launch's token
  const bool avail = lane < n;
  const size_t q = (size_t)t * E + lane;
  const int ex = avail ? cand[q] : 0x7FFFFFFF;
  const float lgt = avail ? exl[q] : 0.0f;
  const float key = avail ? exk[q] : -INFINITY;
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const float kj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key), j));
    const int ej = __builtin_amdgcn_readlane(ex, j);
    rank += (kj > key || (kj == key && ej < ex)) ? 1 : 0;
  }
  const bool sel = avail && rank < k;
  // n >= k >= 1: the k largest approximate keys are always candidates
  const int l0 = __ffsll(__ballot(sel && rank == 0)) - 1;
  const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key), l0));
  const float wv = sel ? gate_weight(gating, renorm, key, lgt, m, 1.0f) : 0.0f;
  float wsum = 0.0f;
  for (int r = 0; r < k; ++r) {
    const int lr = __ffsll(__ballot(sel && rank == r)) - 1;
    wsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), lr));
  }
  if (sel) {
    idx[(size_t)t * k + rank] = ex;
    w[(size_t)t * k + rank] = renorm ? wv / wsum : wv;
  }
}

// Tokens with more than 64 candidates (NJ columns of 64): k rounds of a
// butterfly arg-max under the same order
template <int NJ>
__global__ __launch_bounds__(256) void screen_select_kernel(
    const int16_t* __restrict__ cand, const int32_t* __restrict__ ncand,
    const float* __restrict__ exl, const float* __restrict__ exk, int T, int E, int k,
    int gating, int renorm, int32_t* __restrict__ idx, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int n = ncand[t];
  if (n > 64 * NJ || n <= 64) return;  // the other launch's token
  float key[NJ], lgt[NJ];
  int ex[NJ];
  bool avail[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + 64 * j;
    avail[j] = i < n;
    const size_t q = (size_t)t * E + i;
    ex[j] = avail[j] ? cand[q] : 0x7FFFFFFF;
    lgt[j] = avail[j] ? exl[q] : 0.0f;
    key[j] = avail[j] ? exk[q] : -INFINITY;
  }
  float wsel[kMaxK];
  int isel[kMaxK];
  float wsum = 0.0f, m = 0.0f;
#pragma unroll
  for (int s = 0; s < kMaxK; ++s) {
    if (s < k) {
      float bk = -INFINITY, bl = 0.0f;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (avail[j] && (key[j] > bk || (key[j] == bk && ex[j] < bi))) {
          bk = key[j];
          bi = ex[j];
          bl = lgt[j];
        }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ok = __shfl_xor(bk, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        const float ol = __shfl_xor(bl, o, 64);
        if (ok > bk || (ok == bk && oi < bi)) {
          bk = ok;
          bi = oi;
          bl = ol;
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (ex[j] == bi) avail[j] = false;
      if (s == 0) m = bk;
      const float wv = gate_weight(gating, renorm, bk, bl, m, 1.0f);
      wsel[s] = wv;
      isel[s] = bi;
      wsum += wv;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < kMaxK; ++s)
      if (s < k) {
        idx[(size_t)t * k + s] = isel[s];
        w[(size_t)t * k + s] = renorm ? wsel[s] / wsum : wsel[s];
      }
  }
}

}  // namespace

bool router_screen_applies(const moe_cfg& c) {
  return c.act_dtype == MOE_BF16 && c.E >= kScreenMinE && c.E <= 1024 &&
         !(c.gating == MOE_GATE_SOFTMAX && !c.renorm);
}

size_t router_screen_ws_bytes(const moe_cfg& c) { return carve(c, nullptr).bytes; }

hipError_t launch_router_screened(const moe_cfg& c, const void* x, const float* W_r,
                                  const float* bias, int32_t* idx, float* w, void* ws,
                                  hipStream_t s) {
  const ScreenWs f = carve(c, ws);
  const int T = c.T, D = c.D, E = c.E;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  screen_prep_kernel<<<dim3(ceil_div(E, 32), ceil_div(D, 32)), 256, 0, s>>>(W_r, D, E, f.wt,
                                                                             f.whi, f.wmax);
  screen_norms_kernel<<<E, 256, 0, s>>>(f.wt, f.whi, D, E, f.wmax);
  const int ks = screen_ksplit(c);
  if (E <= 128)  // more workgroups for few experts
    screen_gemm_kernel<64><<<dim3(ceil_div(T, kScrTM), ceil_div(E, 64), ks), 256, 0, s>>>(
        xb, f.whi, T, D, E, f.S, f.nx2);
  else
    screen_gemm_kernel<128><<<dim3(ceil_div(T, kScrTM), ceil_div(E, 128), ks), 256, 0, s>>>(
        xb, f.whi, T, D, E, f.S, f.nx2);
  // 5 g_D (1 + 2^-8): the chain's own bound, the MFMA allowance and a
  // safety margin (see the derivation at the top)
  const double u = 0x1p-24, gD = D * u / (1.0 - D * u);
  const double cg = 5.0 * gD * (1.0 + 0x1p-8);
  const int nj = ceil_div(E, 64);
  const dim3 g4(ceil_div(T, 4));
  if (nj <= 4) screen_cand_kernel<4><<<g4, 256, 0, s>>>(f.S, f.nx2, bias, f.wmax, cg, ks, T, E, c.top_k, f.cand, f.ncand);
  else if (nj <= 6) screen_cand_kernel<6><<<g4, 256, 0, s>>>(f.S, f.nx2, bias, f.wmax, cg, ks, T, E, c.top_k, f.cand, f.ncand);
  else if (nj <= 8) screen_cand_kernel<8><<<g4, 256, 0, s>>>(f.S, f.nx2, bias, f.wmax, cg, ks, T, E, c.top_k, f.cand, f.ncand);
  else screen_cand_kernel<16><<<g4, 256, 0, s>>>(f.S, f.nx2, bias, f.wmax, cg, ks, T, E, c.top_k, f.cand, f.ncand);
  if (E >= 256)
    screen_exact_kernel<256, 96, 3, 2, true>
        <<<dim3(ceil_div(T, 256), ceil_div(E, 96)), 512, 0, s>>>(xb, f.wt, bias, f.cand, f.ncand,
                                                                  T, D, E, f.gpairs, f.exl, f.exk);
  else
    screen_exact_kernel<64, 32, 1, 2, false>
        <<<dim3(ceil_div(T, 64), ceil_div(E, 32)), 512, 0, s>>>(xb, f.wt, bias, f.cand, f.ncand,
                                                                 T, D, E, f.gpairs, f.exl, f.exk);
  screen_select64_kernel<<<g4, 256, 0, s>>>(f.cand, f.ncand, f.exl, f.exk, T, E, c.top_k,
                                            c.gating, c.renorm, idx, w);
  screen_select_kernel<16><<<g4, 256, 0, s>>>(f.cand, f.ncand, f.exl, f.exk, T, E, c.top_k,
                                                 c.gating, c.renorm, idx, w);
  return hipGetLastError();
}

}  // namespace moe

// Tile map of the grouped GEMMs, and the fp32 expert FFN.
//
// "ops-transformer MoE operator on Ascend NPU", optimisation 3: all experts'
// matmuls in one launch although each expert has a different number of
// rows. The tile map lists every (expert, first row) M-tile of BM rows over
// the kept segments (an expert's last M-tile of at most BM/2 rows, when
// wide tiles are on, in a second list); the GEMM grid is sized on the host
// for the worst case and surplus workgroups exit, so no count travels back
// to the host.
//
// The fp32 path ("FFN, SwiGLU and MoE" sec. 2: H = SiLU(x W_gate) * (x W_up),
// y = H W_down) is for fp32 activations and weights; it runs one workgroup
// per segment row with fp32 fused multiply-adds, which is ample for the
// small fp32 layers it serves.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void tilemap_kernel(const int32_t* __restrict__ offsets, int E,
                                                       int bm, int wide_rows,
                                                       int32_t* __restrict__ tilemap,
                                                       int32_t* __restrict__ flags) {
  // wide_rows > 0: an expert's last M-tile with at most wide_rows rows is a
  // wide tile, listed after all regular M-tiles
  __shared__ int wave_tot[2][16];
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
  int rows = 0, start = 0;
  if (e < E) {
    start = offsets[e];
    rows = offsets[e + 1] - start;
  }
  const int full = rows / bm, rem = rows - full * bm;
  const int nw = (wide_rows > 0 && rem > 0 && rem <= wide_rows) ? 1 : 0;
  const int nt = full + (rem > 0 ? 1 : 0) - nw;  // regular M-tiles
  const int incl = wave_inclusive_scan(nt);
  const int inclw = wave_inclusive_scan(nw);
  if (lane == 63) {
    wave_tot[0][wave] = incl;
    wave_tot[1][wave] = inclw;
  }
  __syncthreads();
  int base = incl - nt, basew = inclw - nw, total = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) {
      base += wave_tot[0][w];
      basew += wave_tot[1][w];
    }
    total += wave_tot[0][w];
  }
  for (int i = 0; i < nt; ++i) {
    tilemap[2 + 2 * (base + i)] = e;
    tilemap[3 + 2 * (base + i)] = start + i * bm;
  }
  if (nw) {
    tilemap[2 + 2 * (total + basew)] = e;
    tilemap[3 + 2 * (total + basew)] = start + full * bm;
  }
  if (e == 1023) {
    tilemap[0] = total;
    tilemap[1] = wide_rows > 0 ? basew + nw : -1;
  }
  if (flags && e < 2 * kSplitSlots) flags[e] = 0;  // both banks
}

// expert of a segment row: the last e with offsets[e] <= r
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_f32_gateup_kernel(
    const float* __restrict__ x_perm, const int32_t* __restrict__ offsets, int E, int D, int F,
    const float* __restrict__ Wg, const float* __restrict__ Wu, float clamp,
    float* __restrict__ H) {
  extern __shared__ float xrow[];
  const int r = blockIdx.x;
  if (r >= offsets[E]) return;
  const int e = expert_of_row(offsets, E, r);
  for (int d = threadIdx.x; d < D; d += 256) xrow[d] = x_perm[(size_t)r * D + d];
  __syncthreads();
  const float* g_w = Wg + (size_t)e * D * F;
  const float* u_w = Wu + (size_t)e * D * F;
  for (int f = threadIdx.x; f < F; f += 256) {
    float g = 0.0f, u = 0.0f;
    for (int d = 0; d < D; ++d) {
      g = __builtin_fmaf(xrow[d], g_w[(size_t)d * F + f], g);
      u = __builtin_fmaf(xrow[d], u_w[(size_t)d * F + f], u);
    }
    if (clamp > 0.0f) {
      g = clampf(g, clamp);
      u = clampf(u, clamp);
    }
    H[(size_t)r * F + f] = g / (1.0f + expf(-g)) * u;
  }
}

__global__ __launch_bounds__(256) void ffn_f32_down_kernel(const float* __restrict__ H,
                                                           const int32_t* __restrict__ offsets,
                                                           int E, int D, int F,
                                                           const float* __restrict__ Wd,
                                                           float* __restrict__ y_perm) {
  extern __shared__ float hrow[];
  const int r = blockIdx.x;
  if (r >= offsets[E]) return;
  const int e = expert_of_row(offsets, E, r);
  for (int f = threadIdx.x; f < F; f += 256) hrow[f] = H[(size_t)r * F + f];
  __syncthreads();
  const float* d_w = Wd + (size_t)e * F * D;
  for (int c = threadIdx.x; c < D; c += 256) {
    float acc = 0.0f;
    for (int f = 0; f < F; ++f) acc = __builtin_fmaf(hrow[f], d_w[(size_t)f * D + c], acc);
    y_perm[(size_t)r * D + c] = acc;
  }
}

}  // namespace

hipError_t launch_tilemap(const moe_cfg& c, const int32_t* offsets, int32_t* tilemap,
                          int32_t* flags, bool wide, hipStream_t s) {
  tilemap_kernel<<<1, 1024, 0, s>>>(offsets, c.E, kBM, wide ? kBM / 2 : 0, tilemap, flags);
  return hipGetLastError();
}

hipError_t launch_ffn_f32_gate_up(const moe_cfg& c, const float* x_perm, const int32_t* offsets,
                                  const float* Wg, const float* Wu, float* H, hipStream_t s) {
  const int rows = c.T * c.top_k;
  if (rows == 0) return hipSuccess;
  ffn_f32_gateup_kernel<<<rows, 256, c.D * sizeof(float), s>>>(x_perm, offsets, c.E, c.D, c.F, Wg,
                                                               Wu, c.clamp, H);
  return hipGetLastError();
}

hipError_t launch_ffn_f32_down(const moe_cfg& c, const float* H, const int32_t* offsets,
                               const float* Wd, float* y_perm, hipStream_t s) {
  const int rows = c.T * c.top_k;
  if (rows == 0) return hipSuccess;
  ffn_f32_down_kernel<<<rows, 256, c.F * sizeof(float), s>>>(H, offsets, c.E, c.D, c.F, Wd,
                                                             y_perm);
  return hipGetLastError();
}

}  // namespace moe

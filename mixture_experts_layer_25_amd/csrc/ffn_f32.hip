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
// y = H W_down) is for fp32 activations and weights: the same grouped
// structure (tiles of one expert's rows, all experts in one launch) on the
// fp32 MFMA, with LDS-staged operand tiles.
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

// ---- fp32 grouped GEMM on v_mfma_f32_16x16x4_f32. A tile is 64 rows of
// one expert's segment x 64 columns; K streams through LDS in steps of 32
// (the next step's operands are loaded into registers while the current
// one is multiplied). Workgroup = 4 waves, wave w owns rows 32 (w / 2) ..
// and columns 32 (w % 2) .. of the tile as 2 x 2 blocks of 16 x 16. M-tile
// slot m (the grid covers ceil(rows / 64) + E slots, surplus workgroups
// exit) is the m-th tile in expert order, found by a scan of the segment
// lengths. SWIGLU: two weight matrices (gate, up) share the A tile and the
// epilogue forms h = SiLU(clamp(g)) * clamp(u) in fp32; DOWN: one matrix,
// fp32 out. The MFMA's summation order is its own; fp32 products and
// accumulation keep the result within the fp32 layer's tolerance.
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 32;

typedef float f32x4v_t __attribute__((ext_vector_type(4)));

template <bool SWIGLU>
__global__ __launch_bounds__(256) void ffn_f32_gemm_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ offsets, int E, int K, int N,
    const float* __restrict__ B0, const float* __restrict__ B1, float clamp,
    float* __restrict__ out) {
  constexpr int BM = kF32BM, BN = kF32BN, BK = kF32BK, NB = SWIGLU ? 2 : 1;
  __shared__ float As[BK][BM];
  __shared__ float Bs[NB][BK][BN];
  __shared__ int s_tile[3];  // expert, first row, segment end
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.x, n0 = blockIdx.y * BN;

  // ---- the tile's expert and rows: the m-th M-tile in expert order
  if (tid == 0) s_tile[0] = -1;
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      int seg0 = 0, seg1 = 0;
      if (e < E) {
        seg0 = offsets[e];
        seg1 = offsets[e + 1];
      }
      const int nt = (seg1 - seg0 + BM - 1) / BM;
      const int incl = wave_inclusive_scan(nt);
      const int first = base + incl - nt;
      if (e < E && m >= first && m < first + nt) {
        s_tile[0] = e;
        s_tile[1] = seg0 + (m - first) * BM;
        s_tile[2] = seg1;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;
  const int row0 = s_tile[1], row_end = s_tile[2];
  const float* Bw0 = B0 + (size_t)e * K * N;
  const float* Bw1 = SWIGLU ? B1 + (size_t)e * K * N : nullptr;

  // ---- operand loads: thread -> float4 p of A (row (tid + 256 p) / 8,
  // k 4 (tid % 8)) and of each B (k (tid + 256 p) / 16, columns 4 (tid % 16)),
  // p = 0, 1; zero outside the tile's rows, N and K
  constexpr int NP = BK / 16;  // float4 pieces per thread and operand
  static_assert(BM * BK == 4 * 256 * NP && BK * BN == 4 * 256 * NP, "load shape");
  const int ak = 4 * (tid % (BK / 4)), bn = 4 * (tid & 15);
  const bool b_col_ok = n0 + bn < N;  // N % 4 == 0: a float4 is wholly in or out
  f32x4v_t ra[NP], rb[NB][NP];
  auto load = [&](int k0) __attribute__((always_inline)) {
    const f32x4v_t z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int ar = (tid + 256 * p) / (BK / 4), bk = (tid + 256 * p) >> 4;
      ra[p] = row0 + ar < row_end && k0 + ak < K
                  ? *reinterpret_cast<const f32x4v_t*>(A + (size_t)(row0 + ar) * K + k0 + ak)
                  : z;
      const bool bok = b_col_ok && k0 + bk < K;
      rb[0][p] = bok ? *reinterpret_cast<const f32x4v_t*>(Bw0 + (size_t)(k0 + bk) * N + n0 + bn) : z;
      if constexpr (SWIGLU)
        rb[1][p] = bok ? *reinterpret_cast<const f32x4v_t*>(Bw1 + (size_t)(k0 + bk) * N + n0 + bn) : z;
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int ar = (tid + 256 * p) / (BK / 4), bk = (tid + 256 * p) >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) As[ak + i][ar] = ra[p][i];
#pragma unroll
      for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4v_t*>(&Bs[b][bk][bn]) = rb[b][p];
    }
  };

  f32x4v_t acc[NB][2][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[b][i][j] = f32x4v_t{0.0f, 0.0f, 0.0f, 0.0f};

  // lane l supplies A row l % 16 and B column l % 16 at k = l / 16 of each
  // 4-deep MFMA step, and holds rows 4 (l / 16) + r of column l % 16
  const int wr = 32 * (wave >> 1), wc = 32 * (wave & 1);
  const int fi = lane & 15, fk = lane >> 4;
  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    stage();
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int s = 0; s < BK / 4; ++s) {
      const int kk = 4 * s + fk;
      float a[2], bv[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[kk][wr + 16 * i + fi];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) bv[b][j] = Bs[b][kk][wc + 16 * j + fi];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bv[b][j], acc[b][i][j], 0, 0, 0);
    }
    __syncthreads();  // the step's LDS reads are done before the next stage()
  }

  // ---- epilogue
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wr + 16 * i + 4 * fk + r, col = n0 + wc + 16 * j + fi;
        if (row < row_end && col < N) {
          float v;
          if constexpr (SWIGLU) {
            float g = acc[0][i][j][r], u = acc[1][i][j][r];
            if (clamp > 0.0f) {
              g = clampf(g, clamp);
              u = clampf(u, clamp);
            }
            v = g / (1.0f + expf(-g)) * u;
          } else {
            v = acc[0][i][j][r];
          }
          out[(size_t)row * N + col] = v;
        }
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
  const long long rows = (long long)c.T * c.top_k;
  if (rows == 0) return hipSuccess;
  const dim3 grid(ceil_div(rows, kF32BM) + c.E, ceil_div(c.F, kF32BN));
  ffn_f32_gemm_kernel<true><<<grid, 256, 0, s>>>(x_perm, offsets, c.E, c.D, c.F, Wg, Wu, c.clamp, H);
  return hipGetLastError();
}

hipError_t launch_ffn_f32_down(const moe_cfg& c, const float* H, const int32_t* offsets,
                               const float* Wd, float* y_perm, hipStream_t s) {
  const long long rows = (long long)c.T * c.top_k;
  if (rows == 0) return hipSuccess;
  const dim3 grid(ceil_div(rows, kF32BM) + c.E, ceil_div(c.D, kF32BN));
  ffn_f32_gemm_kernel<false><<<grid, 256, 0, s>>>(H, offsets, c.E, c.F, c.D, Wd, nullptr, 0.0f,
                                                   y_perm);
  return hipGetLastError();
}

}  // namespace moe

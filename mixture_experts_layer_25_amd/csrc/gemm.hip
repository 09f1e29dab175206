// Grouped expert GEMMs on MFMA (bf16 in, fp32 accumulate).
//
// "ops-transformer MoE operator on Ascend NPU", optimisation 3: every
// expert's matmul in one launch, with a different row count per expert.
// "FFN, SwiGLU and MoE" sec. 2: H = SiLU(X W_gate) * (X W_up), Y = H W_down.
// "DeepSeek-V4.1-Flash fine-grained MoE (5A)" sec. 1, 3: gate and up are
// clamped to [-L, L] before SiLU(gate)*up; routed experts may be FP4
// (here MXFP4: e2m1 codes with an e8m0 scale per 32 K-elements).
//
// Tile: 128 rows x 512 B-columns x 32 K per stage, 256 threads (4 waves).
//   SwiGLU: the 512 B-columns are 256 gate and the same 256 up columns, so
//   each wave's accumulators hold gate and up of the same (row, f) and the
//   epilogue forms h = SiLU(clamp(g)) * clamp(u) in registers and stores
//   bf16 H; the gate/up intermediate never reaches memory.
//   Down: 512 output columns, fp32 stores.
// Each wave computes 128 rows x 128 B-columns with v_mfma_f32_32x32x16_bf16
// (4 x 4 tiles, 256 fp32 accumulators per lane).
//
// Operands reach MFMA K-contiguous: a lane's fragment is 8 consecutive k of
// one row (A) or one column (B). X rows are K-contiguous in memory. bf16
// weights are [K][N] (N-contiguous), so each thread loads an 8 x 8 block
// (8 rows of 16 bytes), transposes it in registers and writes 8 columns of
// 8 k to LDS. MXFP4 weights are stored K-contiguous per column: a thread
// loads one column's 32 codes and its scale and writes 32 exact bf16 values
// (e2m1 times a power of two fits bf16 exactly).
//
// LDS per stage: A [4 k-groups][128 rows] and B [4 k-groups][512 cols] of
// 16-byte entries, rows/columns XOR-swizzled within groups of 8 so that the
// 8 lanes sharing an LDS cycle hit 8 different 16-byte bank groups on both
// the writes and the MFMA fragment reads. Two stages; the next stage's
// global loads are in flight while the current stage's MFMAs run.
//
// Workgroup -> tile: tiles are numbered M-tile fastest, so consecutive tiles
// share one weight N-tile; workgroup b runs on XCD (b mod 8), and b is
// remapped so that each XCD takes a contiguous range of tiles and its L2
// serves the weight tile to all of them.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BM = kBM;   // 128
constexpr int BK = 32;
constexpr int BNB = 512;  // B-columns per tile
constexpr int A_STAGE = BM * BK * 2;
constexpr int B_STAGE = BNB * BK * 2;
constexpr int STAGE = A_STAGE + B_STAGE;
constexpr int NSTAGE = 2;

enum { MODE_SWIGLU = 0, MODE_DOWN = 1 };

struct Args {
  const uint16_t* A;
  const int32_t* tilemap;
  const int32_t* offsets;
  int rows, max_tiles, K, N, n_tiles_n, per_xcd;
  const void* B0;
  const void* B1;
  const uint8_t* S0;
  const uint8_t* S1;
  float clamp;
  void* out;
};

__device__ __forceinline__ int swz_a(int m, int q) { return m ^ (((m >> 3) ^ (q << 1)) & 7); }
__device__ __forceinline__ int swz_b(int n) { return n ^ ((n >> 3) & 7); }

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

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Transpose an 8x8 bf16 block held as 8 rows (k) of 8 columns and write
// column c (8 consecutive k) to its LDS entry.
__device__ __forceinline__ void store_b_transposed(unsigned char* Bs, const uint4 (&rb)[8], int nb,
                                                   int kb) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int p = c >> 1;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x0 = u4get(rb[2 * q], p);
      const uint32_t x1 = u4get(rb[2 * q + 1], p);
      o[q] = (c & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
    }
    const int n = 8 * nb + c;
    *reinterpret_cast<uint4*>(Bs + (kb * BNB + swz_b(n)) * 16) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// One column's 32 MXFP4 codes (k0..k0+31) and scale -> 4 LDS entries of
// 8 bf16 each.
__device__ __forceinline__ void store_b_mx(unsigned char* Bs, const uint4& codes, uint32_t s, int n) {
  const float sc = e8m0_scale(s);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t word = u4get(codes, q);  // codes of k = 8q .. 8q+7
    uint4 o;
    o.x = mx_pair(word & 0xFFu, sc);
    o.y = mx_pair((word >> 8) & 0xFFu, sc);
    o.z = mx_pair((word >> 16) & 0xFFu, sc);
    o.w = mx_pair(word >> 24, sc);
    *reinterpret_cast<uint4*>(Bs + (q * BNB + swz_b(n)) * 16) = o;
  }
}

template <int MODE, bool MX>
__global__ __launch_bounds__(256) void gemm_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[NSTAGE * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // workgroup -> tile (XCD-contiguous ranges, M-tile fastest)
  const int b = blockIdx.x;
  const int L = (b & 7) * a.per_xcd + (b >> 3);
  if (L >= a.max_tiles * a.n_tiles_n) return;
  const int mt = L % a.max_tiles;
  const int nt = L / a.max_tiles;
  int e, row0, row_end;
  if (a.tilemap) {
    if (mt >= a.tilemap[0]) return;
    e = a.tilemap[1 + 2 * mt];
    row0 = a.tilemap[2 + 2 * mt];
    row_end = a.offsets[e + 1];
  } else {
    e = 0;
    row0 = mt * BM;
    if (row0 >= a.rows) return;
    row_end = a.rows;
  }
  const int K = a.K, N = a.N;
  const int n0 = MODE == MODE_SWIGLU ? nt * 256 : nt * 512;

  // ---- global -> register staging
  // A: 2 x 16 bytes per thread: rows tid/4 and tid/4 + 64, k-group tid%4
  const int a_q = tid & 3;
  const int a_m0 = tid >> 2, a_m1 = a_m0 + 64;
  const uint16_t* a_src0 = a.A + (size_t)min(row0 + a_m0, row_end - 1) * K + 8 * a_q;
  const uint16_t* a_src1 = a.A + (size_t)min(row0 + a_m1, row_end - 1) * K + 8 * a_q;
  const int a_off0 = (a_q * BM + swz_a(a_m0, a_q)) * 16;
  const int a_off1 = (a_q * BM + swz_a(a_m1, a_q)) * 16;
  // B (bf16 [K][N]): an 8 x 8 block, columns 8*nb.., rows 8*kb..
  const int nb = tid & 63, kb = tid >> 6;
  const uint16_t* b_src = nullptr;
  bool b_ok = false;
  // B (MXFP4 [N][K/2]): LDS columns tid and tid + 256
  const uint8_t* mx_src0 = nullptr;
  const uint8_t* mx_src1 = nullptr;
  const uint8_t* mx_scl0 = nullptr;
  const uint8_t* mx_scl1 = nullptr;
  bool mx_ok0 = false, mx_ok1 = false;
  if (!MX) {
    int col;
    const uint16_t* base;
    if (MODE == MODE_SWIGLU) {
      const bool up = nb >= 32;
      col = n0 + 8 * (nb & 31);
      base = static_cast<const uint16_t*>(up ? a.B1 : a.B0);
    } else {
      col = n0 + 8 * nb;
      base = static_cast<const uint16_t*>(a.B0);
    }
    b_ok = col + 8 <= N;
    b_src = base + ((size_t)e * K + 8 * kb) * N + (b_ok ? col : 0);
  } else {
    int col0, col1;
    const uint8_t *codes0, *codes1, *scl0, *scl1;
    if (MODE == MODE_SWIGLU) {
      col0 = col1 = n0 + tid;
      codes0 = static_cast<const uint8_t*>(a.B0);
      codes1 = static_cast<const uint8_t*>(a.B1);
      scl0 = a.S0;
      scl1 = a.S1;
    } else {
      col0 = n0 + tid;
      col1 = n0 + tid + 256;
      codes0 = codes1 = static_cast<const uint8_t*>(a.B0);
      scl0 = scl1 = a.S0;
    }
    mx_ok0 = col0 < N;
    mx_ok1 = col1 < N;
    const size_t r0 = (size_t)e * N + (mx_ok0 ? col0 : 0);
    const size_t r1 = (size_t)e * N + (mx_ok1 ? col1 : 0);
    mx_src0 = codes0 + r0 * (K / 2);
    mx_src1 = codes1 + r1 * (K / 2);
    mx_scl0 = scl0 + r0 * (K / 32);
    mx_scl1 = scl1 + r1 * (K / 32);
  }

  uint4 ra0, ra1;
  uint4 rb[8];
  uint4 rm0, rm1;
  uint32_t rs0 = 127u, rs1 = 127u;

#define MOE_LOAD_GLOBAL(k0)                                                                   \
  do {                                                                                        \
    ra0 = *reinterpret_cast<const uint4*>(a_src0 + (k0));                                    \
    ra1 = *reinterpret_cast<const uint4*>(a_src1 + (k0));                                    \
    if (!MX) {                                                                                \
      _Pragma("unroll") for (int r = 0; r < 8; ++r) rb[r] =                                   \
          b_ok ? *reinterpret_cast<const uint4*>(b_src + (size_t)((k0) + r) * N)              \
               : make_uint4(0, 0, 0, 0);                                                      \
    } else {                                                                                  \
      rm0 = mx_ok0 ? *reinterpret_cast<const uint4*>(mx_src0 + (k0) / 2) : make_uint4(0, 0, 0, 0); \
      rm1 = mx_ok1 ? *reinterpret_cast<const uint4*>(mx_src1 + (k0) / 2) : make_uint4(0, 0, 0, 0); \
      rs0 = mx_ok0 ? mx_scl0[(k0) / 32] : 127u;                                               \
      rs1 = mx_ok1 ? mx_scl1[(k0) / 32] : 127u;                                               \
    }                                                                                         \
  } while (0)

#define MOE_STORE_LDS(stage)                                                                  \
  do {                                                                                        \
    unsigned char* As_ = smem + (stage) * STAGE;                                              \
    unsigned char* Bs_ = As_ + A_STAGE;                                                       \
    *reinterpret_cast<uint4*>(As_ + a_off0) = ra0;                                            \
    *reinterpret_cast<uint4*>(As_ + a_off1) = ra1;                                            \
    if (!MX) {                                                                                \
      store_b_transposed(Bs_, rb, nb, kb);                                                    \
    } else {                                                                                  \
      store_b_mx(Bs_, rm0, rs0, tid);                                                         \
      store_b_mx(Bs_, rm1, rs1, tid + 256);                                                   \
    }                                                                                         \
  } while (0)

  // wave's B-column bases in the tile
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (MODE == MODE_SWIGLU)
      bcol[j] = (j < 2 ? 0 : 256) + 64 * wave + 32 * (j & 1);
    else
      bcol[j] = 128 * wave + 32 * j;
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = K / BK;
  MOE_LOAD_GLOBAL(0);
  MOE_STORE_LDS(0);
  __syncthreads();
  const int lrow = lane & 31;
  const int lq = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) MOE_LOAD_GLOBAL((kt + 1) * BK);
    const unsigned char* As = smem + stage * STAGE;
    const unsigned char* Bs = As + A_STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int q = 2 * kk + lq;
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (q * BM + swz_a(32 * i + lrow, q)) * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (q * BNB + swz_b(bcol[j] + lrow)) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_STORE_LDS(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue. Accumulator r of lane l: row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32 of its 32x32 tile.
  if (MODE == MODE_SWIGLU) {
    uint16_t* H = static_cast<uint16_t*>(a.out);
    const bool clampit = a.clamp > 0.0f;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int f = n0 + 64 * wave + 32 * jp + lrow;
      if (f >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * i + 8 * (r >> 2) + 4 * lq + (r & 3);
          const int grow = row0 + m;
          if (grow < row_end) {
            float g = acc[i][jp][r], u = acc[i][jp + 2][r];
            if (clampit) {
              g = clampf(g, a.clamp);
              u = clampf(u, a.clamp);
            }
            H[(size_t)grow * N + f] = static_cast<uint16_t>(f32_to_bf16(silu_f32(g) * u));
          }
        }
      }
    }
  } else {
    float* Y = static_cast<float*>(a.out);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 128 * wave + 32 * j + lrow;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * i + 8 * (r >> 2) + 4 * lq + (r & 3);
          const int grow = row0 + m;
          if (grow < row_end) Y[(size_t)grow * N + n] = acc[i][j][r];
        }
      }
    }
  }
}

#undef MOE_LOAD_GLOBAL
#undef MOE_STORE_LDS

hipError_t launch_gemm(const GemmProblem& p, int mode, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  Args a;
  a.A = static_cast<const uint16_t*>(p.A);
  a.tilemap = p.tilemap;
  a.offsets = p.offsets;
  a.rows = p.rows;
  a.max_tiles = p.max_tiles;
  a.K = p.K;
  a.N = p.N;
  a.n_tiles_n = mode == MODE_SWIGLU ? ceil_div(p.N, 256) : ceil_div(p.N, 512);
  const long long total = (long long)a.max_tiles * a.n_tiles_n;
  a.per_xcd = ceil_div(total, 8);
  a.B0 = p.B0;
  a.B1 = p.B1;
  a.S0 = p.S0;
  a.S1 = p.S1;
  a.clamp = p.clamp;
  a.out = p.out;
  const dim3 grid(8 * a.per_xcd);
  if (mode == MODE_SWIGLU) {
    if (p.mxfp4) gemm_kernel<MODE_SWIGLU, true><<<grid, 256, 0, s>>>(a);
    else gemm_kernel<MODE_SWIGLU, false><<<grid, 256, 0, s>>>(a);
  } else {
    if (p.mxfp4) gemm_kernel<MODE_DOWN, true><<<grid, 256, 0, s>>>(a);
    else gemm_kernel<MODE_DOWN, false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_swiglu(const GemmProblem& p, hipStream_t s) { return launch_gemm(p, MODE_SWIGLU, s); }
hipError_t launch_gemm_down(const GemmProblem& p, hipStream_t s) { return launch_gemm(p, MODE_DOWN, s); }

}  // namespace moe

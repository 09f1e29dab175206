// Grouped expert GEMMs with MXFP4 weights and MXFP8 activation operands, on
// the gfx950 block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4.
//
// "DeepSeek-V4.1-Flash fine-grained MoE (5A)" sec. 1, 3: the routed experts
// are stored in FP4 (here MXFP4, OCP MX v1.0: e2m1 codes, one e8m0 scale per
// 32 K-elements); gate and up are clamped before SiLU(gate)*up. "FFN,
// SwiGLU and MoE" sec. 2: H = SiLU(X W_gate) * (X W_up), Y = H W_down.
// In this mode the activation operands (the x rows and H) enter the
// products as MXFP8 (e4m3 codes, one e8m0 scale per 32 K-elements), so the
// MFMA multiplies the stored codes directly, each 32-element block scaled
// by its two e8m0 exponents, at the fp8 rate (twice the bf16 rate) and
// with no conversion work on the vector ALUs.
//
// quant_mxfp8_kernel: bf16 rows -> MXFP8 (one thread per 32-element block):
// the block's exponent is floor(log2(max |v|)) - 8 (8: the exponent of
// e4m3's largest normal), clamped to the e8m0 range; each element is v
// times 2^-exponent, saturated to +-448 and rounded to nearest even by
// v_cvt_pk_fp8_f32.
//
// gemm_a8_kernel<MODE>: the tile schedule and tile shape of the bf16 kernel
// (256 x 256 tiles, 8 waves, wave (wm, wn) owns rows 128wm.. and B-columns
// bcol[j] + 0..31, j = 0, 1; for SwiGLU j = 0 is gate, j = 1 up), 64 k per
// step. MFMA lane layout (32x32x64, fp8 A, fp4 B, checked on the device):
// lane l supplies row l%32 of A with k = 16h..16h+15 and 32+16h..32+16h+15
// (h = l/32) in its 8 registers, column l%32 of B with k = 32h..32h+31 in
// its 4 registers, and the e8m0 scales of row (column) l%32, k-block h.
// Per step and stage (28 KB, 5 stages):
//   A codes  256 rows x 64 bytes, 16-byte k-groups swizzled as in the bf16
//            kernel (slot = group ^ swz4(row)); a lane reads groups h, h+2;
//   A scales 2 blocks x 256 rows, a dword each;
//   B codes  2 blocks x 256 columns x 16 bytes (block-major storage: one
//            contiguous run per block and weight matrix);
//   B scales 2 blocks x 256 columns, a dword each.
// Every operand byte goes global -> LDS with global_load_lds (5 copies per
// thread and step). One barrier per step; each step's LDS reads sit in one
// asm block that waits for them (the compiler cannot tell the fragment
// reads from the copies in flight), then the step's 8 MFMAs.
// Epilogues: SwiGLU forms h = SiLU(clamp(g)) * clamp(u) in fp32 and writes
// it as MXFP8 (each wave's 32 f-columns of a row are one block: codes
// [rows][F] and scales [rows][F/32]); down stores fp32 rows.
#include "gemm_tile.h"

namespace moe {
namespace {

constexpr int BK8 = 64;                    // k per step
constexpr int A8_BYTES = TM * BK8;         // 16 KB of A codes
constexpr int A8S_BYTES = 2 * TM * 4;      // 2 KB of A scales
constexpr int B8C_BYTES = 2 * TN * 16;     // 8 KB of B codes
constexpr int B8S_BYTES = 2 * TN * 4;      // 2 KB of B scales
constexpr int SB8 = A8_BYTES + A8S_BYTES + B8C_BYTES + B8S_BYTES;
constexpr int NST8 = 5;                    // 140 KB of the 160 KB LDS
constexpr int PER8 = 5;                    // copies per thread per step
static_assert(NST8 * SB8 <= 160 * 1024, "LDS");
static_assert(NST8 * SB8 >= 8 * 128 * 128, "the epilogue stages 16 KB per wave");

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

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

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                          long long nblocks,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_t w = src[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[8 * i + 2 * c] = __uint_as_float(w[c] << 16);
      v[8 * i + 2 * c + 1] = __uint_as_float(w[c] & 0xFFFF0000u);
    }
  }
  uint32_t q[8];
  const uint32_t s = mxfp8_block(v, q);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + b * 32);
  dst[0] = u32x4_t{q[0], q[1], q[2], q[3]};
  dst[1] = u32x4_t{q[4], q[5], q[6], q[7]};
  scales[b] = (uint8_t)s;
}

template <int MODE>
__global__ __launch_bounds__(512) void gemm_a8_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[NST8 * SB8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2;  // row half
  const int wn = wave & 3;   // column quarter

  Job jb;
  if (!schedule_tile<BK8>(a, blockIdx.x, jb)) return;
  const int e = jb.e, row0 = jb.row0, row_end = jb.row_end, nt = jb.nt;
  const int kt_begin = jb.kt_begin, nk = jb.nk;
  const int K = a.K, N = a.N, KB = K / 32;
  const int n0 = MODE == MODE_SWIGLU ? nt * 128 : nt * 256;

  // weight column of tile column c (0..255), as in the bf16 kernel
  auto b_column = [&](int c, bool& up) __attribute__((always_inline)) {
    int col;
    if (MODE == MODE_SWIGLU) {
      up = c >= 128;
      col = n0 + (c & 127);
    } else {
      up = false;
      col = n0 + c;
    }
    return col < N ? col : 0;
  };
  auto a_row = [&](int m) __attribute__((always_inline)) {
    int r = min(row0 + m, row_end - 1);
    if (a.gather) r = (int)min((unsigned)a.gather[r], (unsigned)(a.gather_rows - 1));
    return r;
  };

  // ---- copy sources (advanced by one step per issue) and LDS offsets
  const uint8_t* A = static_cast<const uint8_t*>(a.A);
  const uint8_t* a_g[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int p = 512 * r + tid, m = p >> 2, q = (p & 3) ^ swz4(m);
    a_g[r] = A + (size_t)a_row(m) * K + kt_begin * BK8 + 16 * q;
  }
  const int blk = tid >> 8, c = tid & 255;
  const uint8_t* as_g = a.SA + (size_t)a_row(c) * KB + 2 * kt_begin + blk;
  const uint8_t* bc_g;
  const uint8_t* bs_g;
  {
    bool up;
    const int col = b_column(c, up);
    const size_t bi = ((size_t)e * KB + 2 * kt_begin + blk) * N + col;
    bc_g = static_cast<const uint8_t*>(up ? a.B1 : a.B0) + bi * 16;
    bs_g = (up ? a.S1 : a.S0) + bi;
  }
  const size_t bc_step = (size_t)2 * N * 16, bs_step = (size_t)2 * N;
  auto issue = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    unsigned char* st = smem + so;
    const int k = kt - kt_begin;
    dma16(a_g[0] + k * BK8, st + wave * 1024);
    dma16(a_g[1] + k * BK8, st + 8192 + wave * 1024);
    dma1(as_g + 2 * k, st + A8_BYTES + wave * 256);
    dma16(bc_g + k * bc_step, st + A8_BYTES + A8S_BYTES + wave * 1024);
    dma1(bs_g + k * bs_step, st + A8_BYTES + A8S_BYTES + B8C_BYTES + wave * 256);
  };

  int bcol[2];
  if (MODE == MODE_SWIGLU) {
    bcol[0] = 32 * wn;
    bcol[1] = 128 + 32 * wn;
  } else {
    bcol[0] = 64 * wn;
    bcol[1] = 64 * wn + 32;
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int lrow = lane & 31, h = lane >> 5;
  // per-lane LDS addresses in stage 0 (fragment i of A is 32 rows = 2048
  // bytes, and its scales 128 bytes, further; swz4 repeats every 32 rows)
  const uint32_t base = lds_addr(smem);
  uint32_t a_lo, a_hi, as_a, bc_a[2], bs_a[2];
  {
    const int m = 128 * wm + lrow;
    a_lo = base + m * 64 + ((h ^ swz4(m)) * 16);
    a_hi = base + m * 64 + (((h + 2) ^ swz4(m)) * 16);
    as_a = base + A8_BYTES + h * 1024 + m * 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = bcol[j] + lrow;
      bc_a[j] = base + A8_BYTES + A8S_BYTES + h * 4096 + col * 16;
      bs_a[j] = base + A8_BYTES + A8S_BYTES + B8C_BYTES + h * 1024 + col * 4;
    }
  }

  // a wave whose rows all lie past the segment end keeps copying and
  // synchronising but skips its reads and MFMAs
  const bool idle = __builtin_amdgcn_readfirstlane(row_end - row0 <= 128 * wm) != 0;

#pragma unroll
  for (int s = 0; s < NST8 - 1; ++s)
    if (s < nk) issue(kt_begin + s, s * SB8);

  uint32_t so = 0;                           // stage of step kt
  uint32_t si = (uint32_t)(NST8 - 1) * SB8;  // stage of step kt + NST8 - 1
  for (int kt = 0; kt < nk; ++kt) {
    // copies of step kt have landed (steps up to kt + NST8 - 2 were issued)
    wait_copy_groups<PER8>(min(nk - 1, kt + NST8 - 2) - kt);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // every wave is done reading step kt - 1, whose stage takes step kt + NST8 - 1
    if (kt + NST8 - 1 < nk) issue(kt_begin + kt + NST8 - 1, si);
    if (!idle) {
      i32x4_t l0, l1, l2, l3, g0, g1, g2, g3, b0, b1;
      int s0, s1, s2, s3, t0, t1;
      asm volatile(
          "s_nop 4\n\t"
          "ds_read_b128 %[l0], %[alo]\n\t"
          "ds_read_b128 %[g0], %[ahi]\n\t"
          "ds_read_b128 %[l1], %[alo] offset:2048\n\t"
          "ds_read_b128 %[g1], %[ahi] offset:2048\n\t"
          "ds_read_b128 %[l2], %[alo] offset:4096\n\t"
          "ds_read_b128 %[g2], %[ahi] offset:4096\n\t"
          "ds_read_b128 %[l3], %[alo] offset:6144\n\t"
          "ds_read_b128 %[g3], %[ahi] offset:6144\n\t"
          "ds_read_b128 %[b0], %[bc0]\n\t"
          "ds_read_b128 %[b1], %[bc1]\n\t"
          "ds_read_b32 %[s0], %[as]\n\t"
          "ds_read_b32 %[s1], %[as] offset:128\n\t"
          "ds_read_b32 %[s2], %[as] offset:256\n\t"
          "ds_read_b32 %[s3], %[as] offset:384\n\t"
          "ds_read_b32 %[t0], %[bs0]\n\t"
          "ds_read_b32 %[t1], %[bs1]\n\t"
          "s_waitcnt lgkmcnt(0)"
          : [l0] "=&v"(l0), [l1] "=&v"(l1), [l2] "=&v"(l2), [l3] "=&v"(l3), [g0] "=&v"(g0),
            [g1] "=&v"(g1), [g2] "=&v"(g2), [g3] "=&v"(g3), [b0] "=&v"(b0), [b1] "=&v"(b1),
            [s0] "=&v"(s0), [s1] "=&v"(s1), [s2] "=&v"(s2), [s3] "=&v"(s3), [t0] "=&v"(t0),
            [t1] "=&v"(t1)
          : [alo] "v"(a_lo + so), [ahi] "v"(a_hi + so), [bc0] "v"(bc_a[0] + so),
            [bc1] "v"(bc_a[1] + so), [as] "v"(as_a + so), [bs0] "v"(bs_a[0] + so),
            [bs1] "v"(bs_a[1] + so)
          : "memory");
      const i32x8_t fa[4] = {
          i32x8_t{l0[0], l0[1], l0[2], l0[3], g0[0], g0[1], g0[2], g0[3]},
          i32x8_t{l1[0], l1[1], l1[2], l1[3], g1[0], g1[1], g1[2], g1[3]},
          i32x8_t{l2[0], l2[1], l2[2], l2[3], g2[0], g2[1], g2[2], g2[3]},
          i32x8_t{l3[0], l3[1], l3[2], l3[3], g3[0], g3[1], g3[2], g3[3]}};
      const i32x8_t fb[2] = {i32x8_t{b0[0], b0[1], b0[2], b0[3], 0, 0, 0, 0},
                             i32x8_t{b1[0], b1[1], b1[2], b1[3], 0, 0, 0, 0}};
      const int sa[4] = {s0, s1, s2, s3};
      const int sb[2] = {t0, t1};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 0 /* A e4m3 */, 4 /* B e2m1 */, 0, sa[i], 0, sb[j]);
    }
    so = so + SB8 == NST8 * SB8 ? 0u : so + SB8;
    si = si + SB8 == NST8 * SB8 ? 0u : si + SB8;
  }

  if (jb.S > 1 && !split_exchange(a, jb, acc, wave, lane, tid)) return;

  __syncthreads();  // every wave is done with the operand stages
  if (MODE == MODE_SWIGLU) {
    // wave tile: 128 rows x 32 f of fp32 h = SiLU(clamp(g)) * clamp(u), one
    // MXFP8 block per row
    unsigned char* wl = smem + wave * (128 * 128);
    const bool clampit = a.clamp > 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        float g = acc[i][0][r], u = acc[i][1][r];
        if (clampit) {
          g = __builtin_amdgcn_fmed3f(g, -a.clamp, a.clamp);
          u = __builtin_amdgcn_fmed3f(u, -a.clamp, a.clamp);
        }
        *reinterpret_cast<float*>(wl + m * 128 + lrow * 4) =
            g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own wave's tile only
    uint8_t* Hc = static_cast<uint8_t*>(a.out);
    uint8_t* Hs = Hc + (size_t)a.rows * N;  // scales follow the codes
    const int f0 = n0 + 32 * wn;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int m = 64 * half + lane;
      const int grow = row0 + 128 * wm + m;
      float v[32];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const float4 w4 = *reinterpret_cast<const float4*>(wl + m * 128 + cc * 16);
        v[4 * cc] = w4.x;
        v[4 * cc + 1] = w4.y;
        v[4 * cc + 2] = w4.z;
        v[4 * cc + 3] = w4.w;
      }
      uint32_t q[8];
      const uint32_t s = mxfp8_block(v, q);
      if (grow < row_end && f0 < N) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Hc + (size_t)grow * N + f0);
        dst[0] = u32x4_t{q[0], q[1], q[2], q[3]};
        dst[1] = u32x4_t{q[4], q[5], q[6], q[7]};
        Hs[(size_t)grow * (N / 32) + f0 / 32] = (uint8_t)s;
      }
    }
  } else {
    store_down_tile(a, acc, smem, wave, lane, row0 + 128 * wm, row_end, n0, bcol);
  }
}

}  // namespace

hipError_t launch_quant_mxfp8(const void* x, long long rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const long long nb = rows * (K / 32);
  if (nb <= 0) return hipSuccess;
  quant_mxfp8_kernel<<<(unsigned)ceil_div(nb, 256), 256, 0, s>>>(static_cast<const uint16_t*>(x),
                                                                 nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_gemm_a8(const GemmProblem& p, bool swiglu, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  Args a{};
  a.A = p.A;
  a.SA = p.SA;
  a.gather = p.gather;
  a.gather_rows = p.gather_rows;
  a.tilemap = p.tilemap;
  a.offsets = p.offsets;
  a.rows = p.rows;
  a.max_tiles = p.max_tiles;
  a.K = p.K;
  a.N = p.N;
  a.n_tiles_n = swiglu ? ceil_div(p.N, 128) : ceil_div(p.N, 256);
  a.split_ws = p.split_ws;
  a.split_flags = p.split_flags;
  a.B0 = p.B0;
  a.B1 = p.B1;
  a.S0 = p.S0;
  a.S1 = p.S1;
  a.clamp = p.clamp;
  a.out = p.out;
  const long long total = (long long)a.max_tiles * a.n_tiles_n;
  const dim3 grid(8 * (ceil_div(total, 8) + kCUsPerXCD));
  if (swiglu) gemm_a8_kernel<MODE_SWIGLU><<<grid, 512, 0, s>>>(a);
  else gemm_a8_kernel<MODE_DOWN><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe

// Grouped expert GEMMs on MFMA: bf16 activations, MXFP4 weights, fp32
// accumulate.
//
// "ops-transformer MoE operator on Ascend NPU", optimisation 3: every
// expert's matmul in one launch, with a different row count per expert.
// "FFN, SwiGLU and MoE" sec. 2: H = SiLU(X W_gate) * (X W_up), Y = H W_down.
// "DeepSeek-V4.1-Flash fine-grained MoE (5A)" sec. 1, 3: gate and up are
// clamped to [-L, L] before SiLU(gate)*up; routed experts may be FP4
// (here MXFP4: e2m1 codes with an e8m0 scale per 32 K-elements).
//
// gemm_kernel<MODE> takes MXFP4 weights and converts them to bf16 in
// registers for v_mfma_f32_32x32x16_bf16. bf16 weights run on the 16x16x32
// MFMA in gemm16.hip (same tile, copies and schedule); MXFP8 activations
// with MXFP4 weights run on the block-scaled MFMA in gemm_a8.hip.
//
// Tile: 256 rows x 256 B-columns, 32 k per step, 512 threads (8 waves, two
// per SIMD). SwiGLU: the 256 B-columns are 128 gate and the same 128 up
// columns, so gate and up of the same (row, f) meet in one lane and the
// epilogue forms h = SiLU(clamp(g)) * clamp(u) in registers and stores bf16
// H; the gate/up intermediate never reaches memory. Down: 256 output
// columns, fp32 stores. A square tile moves the fewest bytes per flop that
// 64K fp32 accumulators per CU allow. Each wave computes 128 rows x 64
// B-columns with v_mfma_f32_32x32x16_bf16 (4 x 2 MFMA tiles, 128
// accumulators): wave (wm, wn) owns rows 128wm.. and, for SwiGLU,
// f = 32wn..32wn+31 (gate B-column 32wn + l, up B-column 128 + 32wn + l).
//
// Operands reach MFMA K-contiguous: a lane's fragment is 8 consecutive k of
// one row (A) or one column (B).
//   A (X rows, K-contiguous): copied as 16-byte pieces to LDS rows of 64
//   bytes (4 k-groups, slot = k-group ^ swz4(row)), read with ds_read_b128.
//   With a gather list (the fused layer passes perm_token), routed row r
//   is copied from row gather[r] of x: each copy lane looks its two row
//   addresses up once per tile, so the dispatched copy of x is never built.
//   B MXFP4 (stored by 32-k blocks, block-major, so that a step's codes of
//   consecutive columns are consecutive 16-byte pieces; stored K-contiguous
//   per column, every copy lane touched its own cache line and the B
//   copies cost a quarter of the step): each column's 16 code bytes of
//   the step and its e8m0 scale are copied to LDS; a lane reads the 4 code
//   bytes of its k-group and the scale and converts them exactly to bf16
//   with v_cvt_scalef32_pk_bf16_fp4 (fp32 products for the scale codes at
//   the ends of the range). The weights cross HBM, L2 and LDS at 4 bits.
// The swizzles make the 16 lanes of each 256-byte LDS cycle (64 banks on
// gfx950) hit distinct bank groups (LDS bank-conflict counter: 0).
//
// Pipeline. Global data goes straight to LDS with global_load_lds (no
// register staging) into a ring of 7 stages of 21 KB. Each 32-k step is two half-steps of 16 k; the MFMA fragments
// of a half-step are read from LDS while the MFMAs of the previous
// half-step run (two register sets). One barrier per two steps, in the
// middle of every odd step kt, certifies the copies of steps kt+1 and kt+2
// and that every wave is done reading the stages of steps up to kt; each
// step issues the copies of step kt - 1 + NSTAGE (into the stage of step
// kt - 1). The copy instructions sit between the MFMAs of the asm blocks
// (an even step puts its copies into both of its blocks, an odd step all of
// them after its barrier, where the stage of step kt - 1 becomes free), so
// that a copy whose issue waits for room in the memory pipeline stalls
// while the MFMA pipe is busy anyway; issued between the blocks, the copies
// cost a fifth more cycles per step.
//
// Tile schedule (schedule_tile, gemm_tile.h): the real tiles, in expert_tile_of order,
// are cut into 8 contiguous ranges, one per XCD (workgroup b runs on XCD
// b mod 8). Whole rounds of 32 tiles (one per CU of the XCD) run as whole
// tiles; the tiles of the last, partial round are split along K so that
// the last round keeps every CU busy, their fp32 partial sums meeting in a
// workspace in a fixed order.
#include "gemm_tile.h"

namespace moe {
namespace {

constexpr int BK = 32;                  // k per step
constexpr int A_BYTES = TM * BK * 2;    // 16 KB of A per step
constexpr int MXC_BYTES = TN * 16;      // 4 KB of MXFP4 codes per step
constexpr int MXS_BYTES = TN * 4;       // 1 KB of scales (one dword each) per step

constexpr int SB = A_BYTES + MXC_BYTES + MXS_BYTES;  // one stage
constexpr int NST = 7;                               // 147 KB of the 160 KB LDS
constexpr int PER = 3;                               // copies per thread per step
static_assert(NST >= 4, "a barrier every two steps needs four stages");

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

__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Two fragments (8 e2m1 codes each, k-consecutive, low nibble first, with
// their e8m0 scales) -> two MFMA fragments of 8 bf16. The hardware
// conversion multiplies by the fp32 scale exactly for scale codes 2..252,
// where 2^(s - 127) is the float with exponent field s; when either code is
// outside that range (tiny or huge blocks) both fragments are formed from
// fp32 products instead. One range test serves both fragments.
template <int I>
__device__ __forceinline__ uint32_t mx_cvt(uint32_t codes, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, I));
}
__device__ __forceinline__ void mx_fragments(uint32_t c0, uint32_t s0, uint32_t c1, uint32_t s1,
                                             bf16x8_t& f0, bf16x8_t& f1) {
  u32x4_t o0, o1;
  if (max(s0 - 2u, s1 - 2u) < 251u) {
    const float a0 = __uint_as_float(s0 << 23), a1 = __uint_as_float(s1 << 23);
    o0.x = mx_cvt<0>(c0, a0);
    o0.y = mx_cvt<1>(c0, a0);
    o0.z = mx_cvt<2>(c0, a0);
    o0.w = mx_cvt<3>(c0, a0);
    o1.x = mx_cvt<0>(c1, a1);
    o1.y = mx_cvt<1>(c1, a1);
    o1.z = mx_cvt<2>(c1, a1);
    o1.w = mx_cvt<3>(c1, a1);
  } else {
    const float a0 = e8m0_scale(s0), a1 = e8m0_scale(s1);
    o0.x = mx_pair(c0 & 0xFFu, a0);
    o0.y = mx_pair((c0 >> 8) & 0xFFu, a0);
    o0.z = mx_pair((c0 >> 16) & 0xFFu, a0);
    o0.w = mx_pair(c0 >> 24, a0);
    o1.x = mx_pair(c1 & 0xFFu, a1);
    o1.y = mx_pair((c1 >> 8) & 0xFFu, a1);
    o1.z = mx_pair((c1 >> 16) & 0xFFu, a1);
    o1.w = mx_pair(c1 >> 24, a1);
  }
  f0 = __builtin_bit_cast(bf16x8_t, o0);
  f1 = __builtin_bit_cast(bf16x8_t, o1);
}




template <int MODE>
__global__ __launch_bounds__(512) void gemm_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[NST * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;  // 0..7
  const int wm = wave >> 2;   // row half
  const int wn = wave & 3;    // column quarter

  Job jb;
  if (!schedule_tile<BK>(a, blockIdx.x, jb)) return;
  const int e = jb.e, row0 = jb.row0, row_end = jb.row_end, nt = jb.nt;
  const int S = jb.S, part = jb.part, slot0 = jb.slot0, kt_begin = jb.kt_begin, nk = jb.nk;
  const int K = a.K, N = a.N;
  const int n0 = MODE == MODE_SWIGLU ? nt * 128 : nt * 256;

  // Weight column of tile column c (0..255): SwiGLU gate columns n0.. then
  // the same up columns; columns past N read column 0 (any valid data,
  // never stored).
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

  // ---- A copies: LDS entry p = 4m + s (16 bytes) holds k-group s ^ swz4(m)
  // of row m; copy r of wave w fills entries 512r + 64w .. +63.
  const uint16_t* a_g[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int p = 512 * r + tid, m = p >> 2, q = (p & 3) ^ swz4(m);
    int arow = min(row0 + m, row_end - 1);
    if (a.gather) arow = min((unsigned)a.gather[arow], (unsigned)(a.gather_rows - 1));
    a_g[r] = static_cast<const uint16_t*>(a.A) + (size_t)arow * K + kt_begin * BK + 8 * q;
  }
  // ---- B copies: waves 0-3 copy the 16 code bytes of tile columns
  // 64w + l, waves 4-7 the scales of tile columns 64(w - 4) + l (one per
  // lane). Block-major storage: step kt's codes of column col at
  // ((e K/32 + kt) N + col) 16, its scale at (e K/32 + kt) N + col.
  const unsigned char* b_g;
  {
    bool up;
    const int col = b_column(64 * (wave & 3) + lane, up);
    if (wave < 4) {
      const uint8_t* base = static_cast<const uint8_t*>(up ? a.B1 : a.B0);
      b_g = base + (((size_t)e * (K / 32) + kt_begin) * N + col) * 16;
    } else {
      const uint8_t* base = up ? a.S1 : a.S0;
      b_g = base + ((size_t)e * (K / 32) + kt_begin) * N + col;
    }
  }
  auto issue_a = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    unsigned char* As = smem + so;
    const int k0 = kt * BK;
    dma16(a_g[0] + k0, As + wave * 1024);
    dma16(a_g[1] + k0, As + 8192 + wave * 1024);
  };
  auto issue_b = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    unsigned char* Bs = smem + so + A_BYTES;
    if (wave < 4) dma16(b_g + (size_t)kt * N * 16, Bs + wave * 1024);
    else dma1(b_g + (size_t)kt * N, Bs + MXC_BYTES + (wave - 4) * 256);
  };

  // wave's B-column bases: j = 0 gate (or first half), j = 1 up (second)
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

  const int lrow = lane & 31;
  const int lq = lane >> 5;
  const uint32_t smem_addr = lds_addr(smem);
  // Per-lane LDS byte addresses, in stage 0, of the MFMA fragments.
  //   A: row m = 128 wm + lrow, k-group 2 kk + lq (fragment i is 32 rows =
  //      2048 bytes further).
  //   B: code bytes 4 lq.. of column bcol[j] + lrow (kk = 1 is 8
  //      bytes further) and that column's scale dword.
  uint32_t a_addr[2], b_addr[2], s_addr[2];
  {
    const int m = 128 * wm + lrow;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      a_addr[kk] = smem_addr + m * 64 + (((2 * kk + lq) ^ swz4(m)) * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = bcol[j] + lrow;
      b_addr[j] = smem_addr + A_BYTES + col * 16 + 4 * lq;
      s_addr[j] = smem_addr + A_BYTES + MXC_BYTES + col * 4;
    }
  }

  // Fragment registers, two sets: while the MFMAs of one half-step read one
  // set, the LDS reads of the next half-step fill the other. Each read and
  // its MFMAs sit in one asm block that ends by waiting for the reads, so no
  // load is in flight outside the block that issued it (the compiler cannot
  // tell the fragment reads apart from the LDS writes of the copies still in
  // flight, and would wait for all of those). Each block starts with a few
  // wait states so that a register the compiler wrote just before (zeroed
  // accumulators, a fragment it assembled or converted) is settled before an
  // MFMA reads it.
  bf16x8_t xa0, xa1, xa2, xa3, xb0, xb1;
  bf16x8_t ya0, ya1, ya2, ya3, yb0, yb1;
  uint32_t cw0, cw1, sw0, sw1;  // code words and scales of B 0, 1
#define G_MF                                                                         \
  "v_mfma_f32_32x32x16_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"                        \
  "v_mfma_f32_32x32x16_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"                        \
  "v_mfma_f32_32x32x16_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"                        \
  "v_mfma_f32_32x32x16_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"                        \
  "v_mfma_f32_32x32x16_bf16 %[c20], %[a2], %[b0], %[c20]\n\t"                        \
  "v_mfma_f32_32x32x16_bf16 %[c21], %[a2], %[b1], %[c21]\n\t"                        \
  "v_mfma_f32_32x32x16_bf16 %[c30], %[a3], %[b0], %[c30]\n\t"                        \
  "v_mfma_f32_32x32x16_bf16 %[c31], %[a3], %[b1], %[c31]\n\t"
// the MFMAs of G_MF with up to four copies between them (copy X: 16 bytes
// per lane from global address %[gX] to LDS at M0 = %[mX] + 16 lane)
#define G_MFI(I, J) "v_mfma_f32_32x32x16_bf16 %[c" #I #J "], %[a" #I "], %[b" #J "], %[c" #I #J "]\n\t"
#define G_CP16(X) "s_mov_b32 m0, %[m" #X "]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[g" #X "], off\n\t"
#define G_MF_CP(C0, C1, C2, C3)                                                      \
  G_MFI(0, 0) C0 G_MFI(0, 1) G_MFI(1, 0) C1 G_MFI(1, 1) G_MFI(2, 0) C2 G_MFI(2, 1)     \
  G_MFI(3, 0) C3 G_MFI(3, 1)
#define G_NOCOPY [g0] "n"(0)
#define G_RA                                                                         \
  "ds_read_b128 %[na0], %[aa]\n\t"                                                   \
  "ds_read_b128 %[na1], %[aa] offset:2048\n\t"                                       \
  "ds_read_b128 %[na2], %[aa] offset:4096\n\t"                                       \
  "ds_read_b128 %[na3], %[aa] offset:6144\n\t"
#define G_RB_MX(OFF)                                                                 \
  "ds_read_b32 %[cw0], %[ba0] offset:" OFF "\n\t"                                    \
  "ds_read_b32 %[cw1], %[ba1] offset:" OFF "\n\t"                                    \
  "ds_read_b32 %[sw0], %[sa0]\n\t"                                                   \
  "ds_read_b32 %[sw1], %[sa1]\n\t"
#define G_ACC                                                                        \
  [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]),               \
      [c11] "+v"(acc[1][1]), [c20] "+v"(acc[2][0]), [c21] "+v"(acc[2][1]),           \
      [c30] "+v"(acc[3][0]), [c31] "+v"(acc[3][1])
  // reads of a half-step into set N (A at AA; codes at BA0/BA1 + MXOFF,
  // scales at SA0/SA1) while the MFMAs (string MF) consume set C; then set
  // N's B fragments are converted
#define G_BLOCK(MXOFF, AA, BA0, BA1, SA0, SA1, N, C, MF, ...)                         \
  do {                                                                               \
      asm volatile("s_nop 4\n\t" G_RA G_RB_MX(MXOFF) MF                               \
                   "s_waitcnt lgkmcnt(0)"                                            \
                   : [na0] "=&v"(N##a0), [na1] "=&v"(N##a1), [na2] "=&v"(N##a2),      \
                     [na3] "=&v"(N##a3), [cw0] "=&v"(cw0), [cw1] "=&v"(cw1),          \
                     [sw0] "=&v"(sw0), [sw1] "=&v"(sw1), G_ACC                       \
                   : [a0] "v"(C##a0), [a1] "v"(C##a1), [a2] "v"(C##a2),               \
                     [a3] "v"(C##a3), [b0] "v"(C##b0), [b1] "v"(C##b1),               \
                     [aa] "v"(AA), [ba0] "v"(BA0), [ba1] "v"(BA1), [sa0] "v"(SA0),    \
                     [sa1] "v"(SA1), __VA_ARGS__                                     \
                   : "memory", "m0");                                                \
      mx_fragments(cw0, sw0, cw1, sw1, N##b0, N##b1);                                \
  } while (0)
  // MFMAs only, on set y (the last half-step)
#define G_MMA(MF)                                                                    \
  asm volatile("s_nop 4\n\t" MF                                                      \
               : G_ACC                                                               \
               : [a0] "v"(ya0), [a1] "v"(ya1), [a2] "v"(ya2), [a3] "v"(ya3),          \
                 [b0] "v"(yb0), [b1] "v"(yb1))

  // A wave whose 128 rows all lie past the segment end (the segment tail
  // of an expert often fills less than half of its last tile) skips its
  // LDS reads and MFMAs and only keeps the copies and barriers going.
  const bool idle = __builtin_amdgcn_readfirstlane(row_end - row0 <= 128 * wm) != 0;

  // copies of the first NST - 1 steps in flight, then wait for steps 0 and 1
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) {
      issue_a(s, s * SB);
      issue_b(s, s * SB);
    }
  wait_copy_groups<PER>(min(NST - 2, nk - 1) - min(1, nk - 1));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  if (idle) {
    uint32_t si = (uint32_t)(NST - 1) * SB;
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const int is = kt - 1 + NST;  // step whose copies this iteration issues
      if (kt & 1) {
        wait_copy_groups<PER>(min(nk - 1, kt - 2 + NST) - min(kt + 2, nk - 1));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      if (is < nk) {
        issue_a(is, si);
        issue_b(is, si);
      }
      si = si + SB == NST * SB ? 0u : si + SB;
    }
  } else {
    // fragments of half-step (0, 0) -> set x
    {
      asm volatile(G_RA G_RB_MX("0") "s_waitcnt lgkmcnt(0)"
                   : [na0] "=&v"(xa0), [na1] "=&v"(xa1), [na2] "=&v"(xa2), [na3] "=&v"(xa3),
                     [cw0] "=&v"(cw0), [cw1] "=&v"(cw1), [sw0] "=&v"(sw0), [sw1] "=&v"(sw1)
                   : [aa] "v"(a_addr[0]), [ba0] "v"(b_addr[0]), [ba1] "v"(b_addr[1]),
                     [sa0] "v"(s_addr[0]), [sa1] "v"(s_addr[1])
                   : "memory");
      mx_fragments(cw0, sw0, cw1, sw1, xb0, xb1);
    }

    // Step kt: (kt, 1) is read into set y while (kt, 0) multiplies set x;
    // after odd steps the barrier certifies the copies of steps kt+1 and
    // kt+2; then (kt+1, 0) is read into set x while (kt, 1) multiplies set
    // y. The copies of step kt - 1 + NST go to the stage of step kt - 1,
    // which every wave finished reading before the last barrier.
    int kt = 0;
    uint32_t so = 0;                         // byte offset of stage kt % NST
    uint32_t si = (uint32_t)(NST - 1) * SB;  // stage of step kt - 1 + NST
    auto next_stage = [](uint32_t o) { return o + SB == NST * SB ? 0u : o + SB; };
    {
      // Pairs of steps (kt even, kt + 1 odd) that both issue copies, the A
      // copies inside the asm blocks (M0: A copy r of wave w at stage +
      // 8192 r + 1024 w). The B copies, one per thread and step, of a size
      // that depends on the wave, stay between the blocks.
      const uint32_t lds_a = __builtin_amdgcn_readfirstlane(smem_addr + wave * 1024);
      for (; kt + NST < nk; kt += 2) {
        const uint32_t so1 = next_stage(so), so2 = next_stage(so1), si1 = next_stage(si);
        // step kt: copies of step kt - 1 + NST into the stage of step kt - 1
        int is = kt - 1 + NST;
        uint64_t ga0 = (uint64_t)(a_g[0] + is * BK), ga1 = (uint64_t)(a_g[1] + is * BK);
        G_BLOCK("8", a_addr[1] + so, b_addr[0] + so, b_addr[1] + so, s_addr[0] + so,
                s_addr[1] + so, y, x, G_MF_CP(G_CP16(0), "", G_CP16(1), ""), [g0] "v"(ga0),
                [g1] "v"(ga1), [m0] "s"(lds_a + si), [m1] "s"(lds_a + si + 8192));
        G_BLOCK("0", a_addr[0] + so1, b_addr[0] + so1, b_addr[1] + so1, s_addr[0] + so1,
                s_addr[1] + so1, x, y, G_MF, G_NOCOPY);
        issue_b(is, si);
        // step kt + 1: after the barrier, copies of step kt + NST into the
        // stage of step kt
        G_BLOCK("8", a_addr[1] + so1, b_addr[0] + so1, b_addr[1] + so1, s_addr[0] + so1,
                s_addr[1] + so1, y, x, G_MF, G_NOCOPY);
        wait_vmcnt<PER * (NST - 4)>();  // steps up to kt + 3 have landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        is = kt + NST;
        ga0 = (uint64_t)(a_g[0] + is * BK);
        ga1 = (uint64_t)(a_g[1] + is * BK);
        G_BLOCK("0", a_addr[0] + so2, b_addr[0] + so2, b_addr[1] + so2, s_addr[0] + so2,
                s_addr[1] + so2, x, y, G_MF_CP(G_CP16(0), "", G_CP16(1), ""), [g0] "v"(ga0),
                [g1] "v"(ga1), [m0] "s"(lds_a + si1), [m1] "s"(lds_a + si1 + 8192));
        issue_b(is, si1);
        so = so2;
        si = next_stage(si1);
      }
    }
    // the remaining steps: copies (while any are left) between the blocks
    for (; kt + 1 < nk; ++kt) {
      const uint32_t so1 = so + SB == NST * SB ? 0u : so + SB;
      const int is = kt - 1 + NST;  // step whose copies this iteration issues
      G_BLOCK("8", a_addr[1] + so, b_addr[0] + so, b_addr[1] + so, s_addr[0] + so,
              s_addr[1] + so, y, x, G_MF, G_NOCOPY);
      if (kt & 1) {
        // certify steps kt+1 and kt+2; every wave is done with steps < kt+1
        wait_copy_groups<PER>(min(nk - 1, kt - 2 + NST) - min(kt + 2, nk - 1));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      if (is < nk) issue_a(is, si);
      G_BLOCK("0", a_addr[0] + so1, b_addr[0] + so1, b_addr[1] + so1, s_addr[0] + so1,
              s_addr[1] + so1, x, y, G_MF, G_NOCOPY);
      if (is < nk) issue_b(is, si);
      so = so1;
      si = next_stage(si);
    }
    // last step; these blocks end with the MFMA result wait states since
    // the compiler may move accumulators right after them
    G_BLOCK("8", a_addr[1] + so, b_addr[0] + so, b_addr[1] + so, s_addr[0] + so,
            s_addr[1] + so, y, x, G_MF MFMA_TAIL, G_NOCOPY);
    G_MMA(G_MF MFMA_TAIL);
  }
  // the last MFMAs finish writing the accumulators before any VALU reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#undef G_MMA
#undef G_BLOCK
#undef G_ACC
#undef G_RB_MX
#undef G_RA
#undef G_MF

  // ---- split tiles: partial sums through the workspace
  if (S > 1 && !split_exchange(a, jb, acc, wave, lane, tid)) return;

  // ---- epilogue through LDS, so that global stores are 16 bytes per lane.
  // Accumulator r of lane l: row 8*(r/4) + 4*(l/32) + r%4, column l%32 of
  // its 32x32 tile.
  __syncthreads();  // every wave is done with the operand stages
  if (MODE == MODE_SWIGLU) {
    // wave tile: 128 rows x 32 f of bf16 h = SiLU(clamp(g)) * clamp(u)
    unsigned char* wl = smem + wave * (128 * 64);
    const bool clampit = a.clamp > 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * i + 8 * (r >> 2) + 4 * lq + (r & 3);
        float g = acc[i][0][r], u = acc[i][1][r];
        if (clampit) {
          g = __builtin_amdgcn_fmed3f(g, -a.clamp, a.clamp);
          u = __builtin_amdgcn_fmed3f(u, -a.clamp, a.clamp);
        }
        // SiLU(g) u with the hardware exp2 and reciprocal (about 1 ulp
        // each) and the hardware round-to-nearest-even bf16 conversion
        const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        *reinterpret_cast<__bf16*>(wl + m * 64 + lrow * 2) = (__bf16)h;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own wave's tile only
    uint16_t* H = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 64 + lane, m = idx >> 2, ch = idx & 3;
      const int grow = row0 + 128 * wm + m, f = n0 + 32 * wn + 8 * ch;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wl + m * 64 + ch * 16);
      if (grow < row_end && f < N) *reinterpret_cast<u32x4_t*>(H + (size_t)grow * N + f) = v;
    }
  } else {
    store_down_tile(a, acc, smem, wave, lane, row0 + 128 * wm, row_end, n0, bcol);
  }
}

hipError_t launch_gemm(const GemmProblem& p, int mode, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (!p.mxfp4) return launch_gemm16(p, mode == MODE_SWIGLU, s);
  Args a;
  a.A = p.A;
  a.gather = p.gather;
  a.gather_rows = p.gather_rows;
  a.tilemap = p.tilemap;
  a.offsets = p.offsets;
  a.rows = p.rows;
  a.max_tiles = p.max_tiles;
  a.K = p.K;
  a.N = p.N;
  a.n_tiles_n = mode == MODE_SWIGLU ? ceil_div(p.N, 128) : ceil_div(p.N, 256);
  a.split_ws = p.split_ws;
  a.split_flags = p.split_flags;
  a.B0 = p.B0;
  a.B1 = p.B1;
  a.S0 = p.S0;
  a.S1 = p.S1;
  a.clamp = p.clamp;
  a.out = p.out;
  // an XCD's share of the worst-case tiles plus the split parts of its last round
  const long long total = (long long)a.max_tiles * a.n_tiles_n;
  const dim3 grid(8 * (ceil_div(total, 8) + kCUsPerXCD));
  if (mode == MODE_SWIGLU) gemm_kernel<MODE_SWIGLU><<<grid, 512, 0, s>>>(a);
  else gemm_kernel<MODE_DOWN><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_swiglu(const GemmProblem& p, hipStream_t s) { return launch_gemm(p, MODE_SWIGLU, s); }
hipError_t launch_gemm_down(const GemmProblem& p, hipStream_t s) { return launch_gemm(p, MODE_DOWN, s); }

}  // namespace moe

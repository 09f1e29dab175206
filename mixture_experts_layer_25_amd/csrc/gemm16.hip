// Grouped expert GEMMs with bf16 activations and bf16 weights on the
// 16x16x32 MFMA (v_mfma_f32_16x16x32_bf16).
//
// "ops-transformer MoE operator on Ascend NPU", optimisation 3: every
// expert's matmul in one launch. "FFN, SwiGLU and MoE" sec. 2:
// H = SiLU(X W_gate) * (X W_up), Y = H W_down. "DeepSeek-V4.1-Flash
// fine-grained MoE (5A)" sec. 1, 3: gate and up clamped before SiLU*up.
//
// Tile, schedule, pipeline and epilogue as gemm_kernel (gemm.hip, MXFP4
// weights): 256 rows x 256 B-columns per workgroup (SwiGLU: 128 gate and
// the same 128 up columns), 8 waves of 128 rows x 64 B-columns, a ring of 5
// stages of 32 KB filled by global_load_lds, one barrier per two steps, the
// copies placed between the MFMAs. The MFMA shape differs: under full load
// the GEMMs are power-bound, and the 16x16x32 instruction does the same
// multiply-adds for less power than 32x32x16: back-to-back on every SIMD with
// no memory traffic, 16x16x32 sustains 2.12-2.27 PFLOP/s where 32x32x16
// sustains 1.80-2.06 (the clock settles higher).
//
// Operands in LDS. A (X rows, K-contiguous): 16-byte k-groups in rows of 64
// bytes, slot = k-group ^ swz4(row), read with ds_read_b128. B ([K][N],
// N-contiguous): k-rows of 512 bytes (32 chunks of 8 columns, slot = chunk ^
// 4 (k mod 4)) stored as they are; the MFMA fragment (8 k of one column) is
// read with the gfx950 transposing load ds_read_b64_tr_b16 (within a 16-lane
// group, lane i receives element i of the 4 rows the group points at), two
// per fragment, so no transpose runs on the vector ALUs. Both swizzles put
// the 16 lanes of an LDS cycle in distinct bank groups.
//
// MFMA lane layout (checked on the device against a CPU product): lane l
// supplies row l%16 of A and column l%16 of B, each with k = 8 (l/16) ..
// 8 (l/16) + 7, and holds rows 4 (l/16) + r, r = 0..3, of column l%16 of the
// 16x16 result. A wave computes 128 rows x 64 B-columns as 8 x 4 such tiles
// (128 accumulators). A 32-k step is two halves: row tiles 0-3 (A set P)
// then 4-7 (A set Q), 16 MFMAs each, every MFMA taking the full 32 k. The
// four B fragments (one per column tile, 8 k of one column per lane) serve
// both halves; they live in fixed registers v240..v255 so that the two
// transposing LDS reads of a fragment (ds_read_b64_tr_b16, 4 k each) can
// name its halves. Per step a wave reads 8 A and 8 B pieces from LDS, the
// same bytes as the 32x32 kernel.
//
// Blocks (asm): the first half of step kt reads Q of step kt and the last B
// fragment of step kt (whose read the second half of step kt - 1 deferred,
// so that no read sits after a block's last MFMA); the second half reads P
// of step kt + 1 and, after each column tile's last MFMA, that tile's B
// fragment of step kt + 1. Column tiles are multiplied in order 0..3, so B
// fragment 3 is needed last in the first half: its read has 12 MFMAs to
// land, and the block waits for it (lgkmcnt) only before those MFMAs.
#include "gemm_tile.h"

namespace moe {
namespace {

constexpr int BK16 = 32;                   // k per step
constexpr int A16_BYTES = TM * BK16 * 2;   // 16 KB of A per step
constexpr int B16_BYTES = TN * BK16 * 2;   // 16 KB of B per step
constexpr int SB16 = A16_BYTES + B16_BYTES;
constexpr int NST16 = 5;                   // 160 KB of LDS
constexpr int PER16 = 4;                   // copies per thread per step

typedef short s16x4_16 __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(512) void gemm16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[NST16 * SB16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;  // 0..7
  const int wm = wave >> 2;   // row half
  const int wn = wave & 3;    // column quarter

  Job jb;
  if (!schedule_tile<BK16>(a, blockIdx.x, jb)) return;
  const int e = jb.e, row0 = jb.row0, row_end = jb.row_end, nt = jb.nt;
  const int kt_begin = jb.kt_begin, nk = jb.nk;
  const int K = a.K, N = a.N;
  const int n0 = MODE == MODE_SWIGLU ? nt * 128 : nt * 256;

  // weight column of tile column c (0..255), as in gemm_kernel
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

  // ---- copies (as gemm_kernel with bf16 weights): A entry p = 4m + s
  // holds k-group s ^ swz4(m) of row m; B k-row slot c holds 8-column
  // chunk c ^ 4 (k mod 4)
  const uint16_t* a_g[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int p = 512 * r + tid, m = p >> 2, q = (p & 3) ^ swz4(m);
    int arow = min(row0 + m, row_end - 1);
    if (a.gather) arow = min((unsigned)a.gather[arow], (unsigned)(a.gather_rows - 1));
    a_g[r] = static_cast<const uint16_t*>(a.A) + (size_t)arow * K + kt_begin * BK16 + 8 * q;
  }
  const unsigned char* b_g[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int k = 4 * wave + 2 * r + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (k & 3));
    bool up;
    const int col = b_column(8 * c, up);
    const uint16_t* base = static_cast<const uint16_t*>(up ? a.B1 : a.B0);
    b_g[r] = reinterpret_cast<const unsigned char*>(base + ((size_t)e * K + kt_begin * BK16 + k) * N + col);
  }
  auto issue = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    unsigned char* st = smem + so;
    const int k0 = (kt - kt_begin) * BK16;
    dma16(a_g[0] + k0, st + wave * 1024);
    dma16(a_g[1] + k0, st + 8192 + wave * 1024);
    const size_t step = (size_t)(kt - kt_begin) * BK16 * N * 2;
    dma16(b_g[0] + step, st + A16_BYTES + (4 * wave) * 512);
    dma16(b_g[1] + step, st + A16_BYTES + (4 * wave + 2) * 512);
  };

  // wave's column tiles: SwiGLU 0, 1 gate (f = 32wn..), 2, 3 the same up
  // columns; down 64wn + 16j
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bcol[j] = MODE == MODE_SWIGLU ? (j < 2 ? 32 * wn + 16 * j : 128 + 32 * wn + 16 * (j - 2))
                                  : 64 * wn + 16 * j;

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int l16 = lane & 15, g = lane >> 4;
  // LDS addresses in stage 0. A: row 128wm + l16 of row tile 0, k-group g
  // (row tile i is 16 rows = 1024 bytes further; swz4 repeats every 16
  // rows). B: the transposing read of column tile j: the lane points at
  // k-row 8g + (l16 >> 2) and 4 columns bcol[j] + 4 (l & 3); the second
  // read of a fragment is 4 k-rows (2048 bytes) further.
  const uint32_t base = lds_addr(smem);
  uint32_t a_addr, b_addr[4];
  {
    const int m = 128 * wm + l16;
    a_addr = base + m * 64 + ((g ^ swz4(m)) * 16);
    const int tr_row = l16 >> 2;
    const int r0 = 8 * g + tr_row;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = bcol[j] + 4 * (lane & 3);
      b_addr[j] = base + A16_BYTES + r0 * 512 + ((col >> 3) ^ (4 * tr_row)) * 16 + (col & 7) * 2;
    }
  }

  // A fragment sets P (row tiles 0-3) and Q (4-7); B fragments pinned
  bf16x8_t p0, p1, p2, p3, q0, q1, q2, q3;
  bf16x8_t B0, B1, B2, B3;
#define M16(C, A, B) "v_mfma_f32_16x16x32_bf16 %[" C "], %[" A "], " B ", %[" C "]\n\t"
#define RB0 "v[240:243]"
#define RB1 "v[244:247]"
#define RB2 "v[248:251]"
#define RB3 "v[252:255]"
  // B fragment j of the stage at offset SO: two transposing reads
#define RDB(REG_LO, REG_HI, BA) \
  "ds_read_b64_tr_b16 " REG_LO ", %[" BA "]\n\tds_read_b64_tr_b16 " REG_HI ", %[" BA "] offset:2048\n\t"
#define RDB0 RDB("v[240:241]", "v[242:243]", "bb0")
#define RDB1 RDB("v[244:245]", "v[246:247]", "bb1")
#define RDB2 RDB("v[248:249]", "v[250:251]", "bb2")
#define RDB3 RDB("v[252:253]", "v[254:255]", "bb3")
#define RDA(OUT, OFF) "ds_read_b128 %[" OUT "], %[aa] offset:" OFF "\n\t"
  // the 16 MFMAs of a half (A operands x0..x3, accumulators c00..c33), by
  // column tile; X0..X15 are inserted after the MFMAs (reads, copies)
#define HALF(X0, X1, X2, X3, X4, X5, X6, X7, X8, X9, X10, X11, X12, X13, X14, X15)     \
  M16("c00", "x0", RB0) X0 M16("c10", "x1", RB0) X1 M16("c20", "x2", RB0) X2          \
  M16("c30", "x3", RB0) X3 M16("c01", "x0", RB1) X4 M16("c11", "x1", RB1) X5          \
  M16("c21", "x2", RB1) X6 M16("c31", "x3", RB1) X7 M16("c02", "x0", RB2) X8          \
  M16("c12", "x1", RB2) X9 M16("c22", "x2", RB2) X10 M16("c32", "x3", RB2) X11        \
  M16("c03", "x0", RB3) X12 M16("c13", "x1", RB3) X13 M16("c23", "x2", RB3) X14       \
  M16("c33", "x3", RB3) X15
#define HALF_X(...) HALF(__VA_ARGS__)
#define ACC16(I0)                                                                    \
  [c00] "+v"(acc[I0][0]), [c10] "+v"(acc[I0 + 1][0]), [c20] "+v"(acc[I0 + 2][0]),     \
      [c30] "+v"(acc[I0 + 3][0]), [c01] "+v"(acc[I0][1]), [c11] "+v"(acc[I0 + 1][1]),  \
      [c21] "+v"(acc[I0 + 2][1]), [c31] "+v"(acc[I0 + 3][1]), [c02] "+v"(acc[I0][2]),  \
      [c12] "+v"(acc[I0 + 1][2]), [c22] "+v"(acc[I0 + 2][2]), [c32] "+v"(acc[I0 + 3][2]), \
      [c03] "+v"(acc[I0][3]), [c13] "+v"(acc[I0 + 1][3]), [c23] "+v"(acc[I0 + 2][3]),  \
      [c33] "+v"(acc[I0 + 3][3])
#define BPIN                                                                         \
  [B0] "+{v[240:243]}"(B0), [B1] "+{v[244:247]}"(B1), [B2] "+{v[248:251]}"(B2),        \
      [B3] "+{v[252:255]}"(B3)
  // copy X: 16 bytes per lane from global %[gX] to LDS at M0 = %[mX] + 16 lane
#define CP(X) "s_mov_b32 m0, %[m" #X "]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[g" #X "], off\n\t"
#define NOCOPY [g0] "n"(0)
  // first half of a step (stage offset SO): P x B, reading Q of the step
  // (row tiles 4-7: A offsets 4096..7168) and its B fragment 3 (first, so
  // that the wait before the column-3 MFMAs leaves Q in flight); C0..C3:
  // copies between the MFMAs
#define H1(SO, C0, C1, C2, C3, ...)                                                   \
  asm volatile("s_nop 4\n\t" RDB3                                                    \
               HALF_X(RDA("nq0", "4096"), C0, RDA("nq1", "5120"), "", RDA("nq2", "6144"), C1, \
                      RDA("nq3", "7168"), "", C2, "", "", "s_waitcnt lgkmcnt(4)\n\t", C3, "", \
                      "", "")                                                        \
               "s_waitcnt lgkmcnt(0)"                                                \
               : [nq0] "=&v"(q0), [nq1] "=&v"(q1), [nq2] "=&v"(q2), [nq3] "=&v"(q3),  \
                 ACC16(0), BPIN                                                      \
               : [x0] "v"(p0), [x1] "v"(p1), [x2] "v"(p2), [x3] "v"(p3),              \
                 [aa] "v"(a_addr + (SO)), [bb3] "v"(b_addr[3] + (SO)), __VA_ARGS__    \
               : "memory", "m0")
  // second half (P of the next step at stage offset SO): Q x B, reading P
  // of the next step and, after each column tile's last MFMA, its B
  // fragment (0-2; fragment 3 is read by the next first half)
#define H2(SO, C0, C1, C2, C3, ...)                                                   \
  asm volatile("s_nop 4\n\t"                                                         \
               HALF_X(RDA("np0", "0"), C0, RDA("np1", "1024"), RDB0, RDA("np2", "2048"), C1, \
                      RDA("np3", "3072"), RDB1, C2, "", "", RDB2, C3, "", "", "")      \
               "s_waitcnt lgkmcnt(0)"                                                \
               : [np0] "=&v"(p0), [np1] "=&v"(p1), [np2] "=&v"(p2), [np3] "=&v"(p3),  \
                 ACC16(4), BPIN                                                      \
               : [x0] "v"(q0), [x1] "v"(q1), [x2] "v"(q2), [x3] "v"(q3),              \
                 [aa] "v"(a_addr + (SO)), [bb0] "v"(b_addr[0] + (SO)),                \
                 [bb1] "v"(b_addr[1] + (SO)), [bb2] "v"(b_addr[2] + (SO)), __VA_ARGS__ \
               : "memory", "m0")
  // the last second half: MFMAs only, then the result wait states
#define H2_LAST()                                                                    \
  asm volatile("s_nop 4\n\t" HALF("", "", "", "", "", "", "", "", "", "", "", "", "", "", "", "") \
               MFMA_TAIL                                                             \
               : ACC16(4), BPIN                                                      \
               : [x0] "v"(q0), [x1] "v"(q1), [x2] "v"(q2), [x3] "v"(q3))

  // A wave whose 128 rows all lie past the segment end skips its reads and
  // MFMAs and only keeps the copies and barriers going.
  const bool idle = __builtin_amdgcn_readfirstlane(row_end - row0 <= 128 * wm) != 0;

  // copies of the first NST16 - 1 steps in flight, then wait for steps 0, 1
#pragma unroll
  for (int s = 0; s < NST16 - 1; ++s)
    if (s < nk) issue(kt_begin + s, s * SB16);
  wait_copy_groups<PER16>(min(NST16 - 2, nk - 1) - min(1, nk - 1));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  if (idle) {
    uint32_t si = (uint32_t)(NST16 - 1) * SB16;
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const int is = kt - 1 + NST16;  // step whose copies this iteration issues
      if (kt & 1) {
        wait_copy_groups<PER16>(min(nk - 1, kt - 2 + NST16) - min(kt + 2, nk - 1));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      if (is < nk) issue(kt_begin + is, si);
      si = si + SB16 == NST16 * SB16 ? 0u : si + SB16;
    }
  } else {
    // P and B fragments 0-2 of step 0 (fragment 3 is read by the first half)
    asm volatile(RDA("np0", "0") RDA("np1", "1024") RDA("np2", "2048") RDA("np3", "3072")
                 RDB0 RDB1 RDB2 "s_waitcnt lgkmcnt(0)"
                 : [np0] "=&v"(p0), [np1] "=&v"(p1), [np2] "=&v"(p2), [np3] "=&v"(p3), BPIN
                 : [aa] "v"(a_addr), [bb0] "v"(b_addr[0]), [bb1] "v"(b_addr[1]),
                   [bb2] "v"(b_addr[2])
                 : "memory");

    int kt = 0;
    uint32_t so = 0;                            // stage of step kt
    uint32_t si = (uint32_t)(NST16 - 1) * SB16;  // stage of step kt - 1 + NST16
    auto next_stage = [](uint32_t o) { return o + SB16 == NST16 * SB16 ? 0u : o + SB16; };
    {
      // Pairs of steps (kt even, kt + 1 odd) that both issue copies, the
      // copies inside the blocks (M0: A copy r of wave w at stage + 8192 r +
      // 1024 w, B copy r at stage + A16_BYTES + 2048 w + 1024 r).
      const uint32_t lds_a = __builtin_amdgcn_readfirstlane(base + wave * 1024);
      const uint32_t lds_b = __builtin_amdgcn_readfirstlane(base + A16_BYTES + wave * 2048);
      for (; kt + NST16 < nk; kt += 2) {
        const uint32_t so1 = next_stage(so), so2 = next_stage(so1), si1 = next_stage(si);
        // step kt: copies of step kt - 1 + NST16 into the stage of step kt - 1
        int is = kt - 1 + NST16;
        uint64_t ga0 = (uint64_t)(a_g[0] + is * BK16), ga1 = (uint64_t)(a_g[1] + is * BK16);
        uint64_t gb0 = (uint64_t)(b_g[0] + (size_t)is * BK16 * N * 2);
        uint64_t gb1 = (uint64_t)(b_g[1] + (size_t)is * BK16 * N * 2);
        H1(so, CP(0), "", CP(1), "", [g0] "v"(ga0), [g1] "v"(ga1), [m0] "s"(lds_a + si),
           [m1] "s"(lds_a + si + 8192));
        H2(so1, CP(0), "", CP(1), "", [g0] "v"(gb0), [g1] "v"(gb1), [m0] "s"(lds_b + si),
           [m1] "s"(lds_b + si + 1024));
        // step kt + 1: after the barrier, copies of step kt + NST16 into the
        // stage of step kt
        H1(so1, "", "", "", "", NOCOPY);
        wait_vmcnt<PER16 * (NST16 - 4)>();  // steps up to kt + 3 have landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        is = kt + NST16;
        ga0 = (uint64_t)(a_g[0] + is * BK16);
        ga1 = (uint64_t)(a_g[1] + is * BK16);
        gb0 = (uint64_t)(b_g[0] + (size_t)is * BK16 * N * 2);
        gb1 = (uint64_t)(b_g[1] + (size_t)is * BK16 * N * 2);
        H2(so2, CP(0), CP(1), CP(2), CP(3), [g0] "v"(ga0), [g1] "v"(ga1), [g2] "v"(gb0),
           [g3] "v"(gb1), [m0] "s"(lds_a + si1), [m1] "s"(lds_a + si1 + 8192),
           [m2] "s"(lds_b + si1), [m3] "s"(lds_b + si1 + 1024));
        so = so2;
        si = next_stage(si1);
      }
    }
    // the remaining steps: copies (while any are left) between the blocks
    for (; kt + 1 < nk; ++kt) {
      const uint32_t so1 = next_stage(so);
      const int is = kt - 1 + NST16;
      H1(so, "", "", "", "", NOCOPY);
      if (kt & 1) {
        wait_copy_groups<PER16>(min(nk - 1, kt - 2 + NST16) - min(kt + 2, nk - 1));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      if (is < nk) issue(kt_begin + is, si);
      H2(so1, "", "", "", "", NOCOPY);
      so = so1;
      si = next_stage(si);
    }
    // last step
    H1(so, "", "", "", "", NOCOPY);
    H2_LAST();
  }
  // the last MFMAs finish writing the accumulators before any VALU reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#undef H2_LAST
#undef H2
#undef H1
#undef NOCOPY
#undef CP
#undef BPIN
#undef ACC16
#undef HALF_X
#undef HALF
#undef RDA
#undef RDB3
#undef RDB2
#undef RDB1
#undef RDB0
#undef RDB
#undef RB3
#undef RB2
#undef RB1
#undef RB0
#undef M16

  // ---- split tiles: partial sums through the workspace (float4 q = 4 i + j)
  if (jb.S > 1 && !split_exchange(
                      a, jb,
                      [&](int q) {
                        const f32x4_t& t = acc[q >> 2][q & 3];
                        return make_float4(t[0], t[1], t[2], t[3]);
                      },
                      [&](int q, float4 v) {
                        f32x4_t& t = acc[q >> 2][q & 3];
                        t[0] += v.x;
                        t[1] += v.y;
                        t[2] += v.z;
                        t[3] += v.w;
                      },
                      wave, lane, tid))
    return;

  // ---- epilogue through LDS (16-byte global stores). Accumulator r of lane
  // l in tile (i, j): row 16i + 4 (l/16) + r, column bcol[j] + l%16.
  __syncthreads();  // every wave is done with the operand stages
  if (MODE == MODE_SWIGLU) {
    // wave tile: 128 rows x 32 f of bf16 h = SiLU(clamp(g)) * clamp(u),
    // gate in column tiles 0, 1 and the matching up in 2, 3
    unsigned char* wl = smem + wave * (128 * 64);
    const bool clampit = a.clamp > 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * i + 4 * g + r;
          float gv = acc[i][j][r], uv = acc[i][j + 2][r];
          if (clampit) {
            gv = __builtin_amdgcn_fmed3f(gv, -a.clamp, a.clamp);
            uv = __builtin_amdgcn_fmed3f(uv, -a.clamp, a.clamp);
          }
          // SiLU(g) u with the hardware exp2 and reciprocal and the hardware
          // round-to-nearest-even bf16 conversion
          const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          *reinterpret_cast<__bf16*>(wl + m * 64 + (16 * j + l16) * 2) = (__bf16)h;
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
    // wave tile: 128 rows x 64 fp32 columns, in two halves of 32 columns
    unsigned char* wl = smem + wave * (128 * 128);
    float* Y = static_cast<float*>(a.out);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * g + r;
            *reinterpret_cast<float*>(wl + m * 128 + (16 * jj + l16) * 4) = acc[i][2 * hh + jj][r];
          }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int idx = it * 64 + lane, m = idx >> 3, ch = idx & 7;
        const int grow = row0 + 128 * wm + m, n = n0 + 64 * wn + 32 * hh + 4 * ch;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wl + m * 128 + ch * 16);
        if (grow < row_end && n < N) *reinterpret_cast<u32x4_t*>(Y + (size_t)grow * N + n) = v;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next half overwrites
    }
  }
}

}  // namespace

hipError_t launch_gemm16(const GemmProblem& p, bool swiglu, hipStream_t s) {
  if (p.max_tiles <= 0) return hipSuccess;
  Args a{};
  a.A = p.A;
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
  a.clamp = p.clamp;
  a.out = p.out;
  const long long total = (long long)a.max_tiles * a.n_tiles_n;
  const dim3 grid(8 * (ceil_div(total, 8) + kCUsPerXCD));
  if (swiglu) gemm16_kernel<MODE_SWIGLU><<<grid, 512, 0, s>>>(a);
  else gemm16_kernel<MODE_DOWN><<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe

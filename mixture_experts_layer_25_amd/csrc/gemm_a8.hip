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
// v_cvt_pk_fp8_f32. Scales are stored row-major ([rows][K/32]) or, for the
// GEMM, grouped: [ceil(K/512)][rows][16] (the 16 scales of 8 GEMM steps of
// a row in one 16-byte piece).
//
// gemm_a8_kernel<MODE>: the tile schedule and tile shape of the bf16 kernel
// (256 x 256 tiles, 8 waves, wave (wm, wn) owns rows 128wm.. and B-columns
// bcol[j] + 0..31, j = 0, 1; for SwiGLU j = 0 is gate, j = 1 up), 64 k per
// step. MFMA lane layout (32x32x64, fp8 A, fp4 B, checked on the device):
// lane l supplies row l%32 of A with k = 16h..16h+15 and 32+16h..32+16h+15
// (h = l/32) in its 8 registers, column l%32 of B with k = 32h..32h+31 in
// its 4 registers, and the e8m0 scales of row (column) l%32, k-block h.
// Per step and stage (24.5 KB, 5 stages):
//   A codes  256 rows x 64 bytes, 16-byte k-groups swizzled as in the bf16
//            kernel (slot = group ^ swz4(row)); a lane reads groups h, h+2;
//   B codes  2 blocks x 256 columns x 16 bytes (block-major storage: one
//            contiguous run per block and weight matrix);
//   B scales 2 blocks x 256 columns, one byte each (copied as dwords).
// A scales: a ring of 3 groups of 8 steps (16 bytes per row, 4 KB each).
// Every operand byte goes global -> LDS with global_load_lds. A copy
// instruction costs about the same whatever its width (measured: one byte
// per lane from 64 rows cost as much per instruction as 16 bytes), so the
// scales travel in as few instructions as possible: per step and CU 16
// instructions of A, 8 of B codes, 2 of B scales and half of one of A
// scales, against 40 when every scale byte had a lane of its own. One
// barrier per step (a barrier every second step, with six stages, left one
// step fewer in flight and was 13 % slower). A step is two halves of 4
// MFMAs (row tiles 0-1, then 2-3); each half is one asm block whose LDS
// reads (the other half's fragments) sit between its MFMAs, issued at
// least two MFMAs before the block's final wait.
// A rows: MXFP8 x_perm from the dispatch, H, or (fused layer) the MXFP8
// copy of x through the gather list.
// Epilogues: SwiGLU forms h = SiLU(clamp(g)) * clamp(u) in fp32 and writes
// it as MXFP8 (each wave's 32 f-columns of a row are one block: codes
// [rows][F], then grouped scales); down stores fp32 rows.
#include "gemm_tile.h"
#include "mxfp8.h"

namespace moe {
namespace {

constexpr int BK8 = 64;                    // k per step
constexpr int A8_BYTES = TM * BK8;         // 16 KB of A codes per step
constexpr int B8C_BYTES = 2 * TN * 16;     // 8 KB of B codes per step
constexpr int B8S_BYTES = 2 * TN;          // 512 B of B scales per step
constexpr int SB8 = A8_BYTES + B8C_BYTES + B8S_BYTES;
constexpr int NST8 = 5;                    // operand stages
constexpr int kSG = 8;                     // steps per A-scale group
constexpr int ASG_BYTES = TM * 16;         // one group of A scales: 16 bytes per row
constexpr int AS_OFF = NST8 * SB8;         // ring of 3 A-scale groups after the stages
constexpr int LDS8 = AS_OFF + 3 * ASG_BYTES;  // 134.5 KB of the 160 KB LDS
static_assert(LDS8 <= 160 * 1024, "LDS");
static_assert(LDS8 >= 8 * 128 * 128, "the epilogue stages 16 KB per wave");

// Wide tiles (an expert's last M-tile of at most 128 rows): 128 rows x 512
// B-columns, the 8 waves side by side on the same rows. Stage: 8 KB of A
// codes, 16 KB of B codes, 1 KB of B scales; A-scale groups of 2 KB.
template <bool WIDE>
struct ShapeA8 {
  static constexpr int ROWS = WIDE ? TMW : TM;
  static constexpr int COLS = WIDE ? TNW : TN;
  static constexpr int A_BYTES = ROWS * BK8;
  static constexpr int BC_BYTES = 2 * COLS * 16;
  static constexpr int BS_BYTES = 2 * COLS;
  static constexpr int SB = A_BYTES + BC_BYTES + BS_BYTES;
  static constexpr int ASG = ROWS * 16;
  static constexpr int AS_OFF = NST8 * SB;
  static constexpr int LDS = AS_OFF + 3 * ASG;
  static constexpr int ACP = ROWS * 4 / 512;    // A copies per thread and step
  static constexpr int BCP = COLS * 2 / 512;    // B code copies per thread and step
  static constexpr int NBS = COLS / 128;        // waves copying B scales (one dword a lane)
  static constexpr int NAS = ROWS / 64;         // waves copying A-scale groups
};
static_assert(ShapeA8<false>::LDS == LDS8, "the regular shape is the one above");
static_assert(ShapeA8<true>::LDS <= LDS8 && ShapeA8<true>::LDS >= 8 * 128 * 128, "wide LDS");

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(n) for a count known only at run time (n <= 15)
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
}

// the two 16-byte halves of an MFMA A operand as one 8-register value
__device__ __forceinline__ i32x8_t join8(i32x4_t lo, i32x4_t hi) {
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool GROUPED>
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                          long long rows, int KB,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= rows * KB) return;
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
  scales[GROUPED ? grouped_scale(b / KB, (int)(b % KB), rows) : (size_t)b] = (uint8_t)s;
}

template <int MODE, bool WIDE>
__device__ __forceinline__ void gemm_a8_body(const Args& a, const Job& jb, unsigned char* smem) {
  using SH = ShapeA8<WIDE>;
  constexpr int A8_BYTES = SH::A_BYTES, B8C_BYTES = SH::BC_BYTES, SB8 = SH::SB;
  constexpr int ASG_BYTES = SH::ASG, AS_OFF = SH::AS_OFF, COLS = SH::COLS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (an SGPR): the per-wave choices below become scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = WIDE ? 0 : wave >> 2;   // row half
  const int wn = WIDE ? wave : wave & 3; // column block

  const int e = jb.e, row0 = jb.row0, row_end = jb.row_end, nt = jb.nt;
  const int kt_begin = jb.kt_begin, nk = jb.nk;
  const int K = a.K, N = a.N, KB = K / 32;
  const int n0 = MODE == MODE_SWIGLU ? nt * (COLS / 2) : nt * COLS;

  // weight column of tile column c (0..COLS-1), as in the bf16 kernel
  auto b_column = [&](int c, bool& up) __attribute__((always_inline)) {
    int col;
    if (MODE == MODE_SWIGLU) {
      up = c >= COLS / 2;
      col = n0 + (c & (COLS / 2 - 1));
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

  // ---- copy sources and destinations. Per step and thread: ACP 16-byte
  // pieces of A and BCP of B codes (regular: 2 and 1, wide: 1 and 2); the
  // first NBS waves also copy the step's two blocks of B scales (one dword
  // per lane: 4 columns). The A scales come in groups of 8 steps (16 bytes
  // per row, grouped layout): wave w < NAS copies its 64 rows of group G + 2
  // at the step of group G whose index within the group is w, into a ring
  // of 3 group buffers; the first groups of the tile's k-range are copied
  // before the loop.
  const uint8_t* A = static_cast<const uint8_t*>(a.A);
  const uint8_t* a_g[SH::ACP];
#pragma unroll
  for (int r = 0; r < SH::ACP; ++r) {
    const int p = 512 * r + tid, m = p >> 2, q = (p & 3) ^ swz4(m);
    a_g[r] = A + (size_t)a_row(m) * K + kt_begin * BK8 + 16 * q;
  }
  // B code copy r of thread t: block (regular) t / 256 or (wide) r, tile
  // column t % 256 or t
  const uint8_t* bc_g[SH::BCP];
#pragma unroll
  for (int r = 0; r < SH::BCP; ++r) {
    const int blk = WIDE ? r : tid >> 8, c = WIDE ? tid : tid & 255;
    bool up;
    const int col = b_column(c, up);
    const size_t bi = ((size_t)e * KB + 2 * kt_begin + blk) * N + col;
    bc_g[r] = static_cast<const uint8_t*>(up ? a.B1 : a.B0) + bi * 16;
  }
  const size_t bc_step = (size_t)2 * N * 16;
  // B scales: wave w < NBS copies block w / (NBS / 2) of each step, lane l
  // the 4 columns of tile columns 4 c4.., c4 = 64 (w % (NBS / 2)) + l
  // (SwiGLU: gate for c4 < COLS / 8, up above)
  const uint8_t* bs_g = nullptr;
  if (wave < SH::NBS) {
    const int c4 = 64 * (wave % (SH::NBS / 2)) + lane, blk = wave / (SH::NBS / 2);
    const bool up = MODE == MODE_SWIGLU && c4 >= COLS / 8;
    int col = MODE == MODE_SWIGLU ? n0 + 4 * (c4 & (COLS / 8 - 1)) : n0 + 4 * c4;
    if (col >= N) col = 0;  // any valid columns; never stored
    bs_g = (up ? a.S1 : a.S0) + ((size_t)e * KB + 2 * kt_begin + blk) * N + col;
  }
  const size_t bs_step = (size_t)2 * N;
  // A scales: row 64 w + lane of the tile, grouped layout
  const long long sa_rows = a.gather ? a.gather_rows : a.rows;
  const uint8_t* as_g = wave < SH::NAS ? a.SA + (size_t)a_row(64 * wave + lane) * 16 : nullptr;
  const int g_last = (kt_begin + nk - 1) / kSG;  // last group of the k-range
  auto issue_group = [&](int g) __attribute__((always_inline)) {
    g = min(g, g_last);  // past the range: copy the last group again (same bytes)
    dma16(as_g + (size_t)g * sa_rows * 16, smem + AS_OFF + (g % 3) * ASG_BYTES + wave * 1024);
  };
  // the steps are issued in order, each once: the sources advance a step
  // per call
  auto issue = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    (void)kt;
    unsigned char* st = smem + so;
#pragma unroll
    for (int r = 0; r < SH::ACP; ++r) {
      dma16(a_g[r], st + 8192 * r + wave * 1024);
      a_g[r] += BK8;
    }
#pragma unroll
    for (int r = 0; r < SH::BCP; ++r) {
      dma16(bc_g[r], st + A8_BYTES + 8192 * r + wave * 1024);
      bc_g[r] += bc_step;
    }
    if (wave < SH::NBS) {
      dma4(bs_g, st + A8_BYTES + B8C_BYTES + wave * 256);
      bs_g += bs_step;
    }
  };
  const int per = SH::ACP + SH::BCP + (wave < SH::NBS ? 1 : 0);  // this wave's copies per step

  int bcol[2];
  if (MODE == MODE_SWIGLU) {
    bcol[0] = 32 * wn;
    bcol[1] = COLS / 2 + 32 * wn;
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
  // per-lane LDS addresses: operands in stage 0 (fragment i of A is 32
  // rows = 2048 bytes further; swz4 repeats every 32 rows), A scales in
  // group buffer 0 at step 0 of the group (fragment i: 512 bytes further)
  const uint32_t base = lds_addr(smem);
  uint32_t a_lo, a_hi, as_a, bc_a[2], bs_a[2];
  {
    const int m = 128 * wm + lrow;
    a_lo = base + m * 64 + ((h ^ swz4(m)) * 16);
    a_hi = base + m * 64 + (((h + 2) ^ swz4(m)) * 16);
    as_a = base + AS_OFF + m * 16 + h;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = bcol[j] + lrow;
      bc_a[j] = base + A8_BYTES + h * (COLS * 16) + col * 16;
      bs_a[j] = base + A8_BYTES + B8C_BYTES + h * COLS + col;
    }
  }
  // A-scale offset of absolute step t: group buffer (t / 8) % 3, 2 bytes a step
  auto as_off = [](int t) { return (uint32_t)((t / kSG) % 3 * ASG_BYTES + (t % kSG) * 2); };
  // the same, kept step by step in the loop: t % kSG and (t / kSG) % 3
  int t_r = kt_begin % kSG, t_g = kt_begin / kSG % 3;
  auto ao_cur = [&]() { return (uint32_t)(t_g * ASG_BYTES + t_r * 2); };
  auto ao_next = [&]() {
    if (++t_r == kSG) {
      t_r = 0;
      t_g = t_g == 2 ? 0 : t_g + 1;
    }
  };

  // a wave whose rows all lie past the segment end keeps copying and
  // synchronising but skips its reads and MFMAs
  const bool idle = __builtin_amdgcn_readfirstlane(row_end - row0 <= 128 * wm) != 0;

  // Fragments. A step is two halves: rows 0-63 of the wave (MFMA row tiles
  // 0, 1; set P) and rows 64-127 (tiles 2, 3; set Q). The MFMAs of one half
  // run in one asm block with LDS reads between them; the block ends by
  // waiting for its reads, so no load stays in flight outside the block that
  // issued it. The first half reads Q of the same step; the second half
  // reads P of the next step between its MFMAs and, after its last MFMA,
  // the next step's B fragments (16 code bytes of block h per column tile)
  // and B scales into the registers its MFMAs have just read. A rows
  // 32i + lrow: k-groups h (l) and h + 2 (g), joined into one 8-register
  // operand; scales one dword each. Read addresses are formed inside the
  // blocks (lane base + stage offset) in two alternating registers.
  i32x4_t pl0, pg0, pl1, pg1, ql0, qg0, ql1, qg1, b0, b1;
  int sa0, sa1, sa2, sa3, t0, t1;
#define A8_MF(I, J, AR, BR, SA, SB)                                                  \
  "v_mfma_scale_f32_32x32x64_f8f6f4 %[c" #I #J "], %[" AR "], %[" BR "], %[c" #I #J   \
  "], %[" SA "], %[" SB "] op_sel_hi:[0,0,0] blgp:4\n\t"
  // MFMAs of tiles I0, I1 (A operands a0, a1; scales s0, s1) on B b0 then
  // b1 (scales t0, t1): R0 before them, R1 after the first, R2 after the
  // second (the last use of b0), R3 after the third, R4 after the fourth
#define A8_HALF(I0, I1, R0, R1, R2, R3, R4)                                          \
  R0 A8_MF(I0, 0, "a0", "b0", "s0", "t0") R1 A8_MF(I1, 0, "a1", "b0", "s1", "t0") R2    \
  A8_MF(I0, 1, "a0", "b1", "s0", "t1") R3 A8_MF(I1, 1, "a1", "b1", "s1", "t1") R4
#define A8_HALF_X(...) A8_HALF(__VA_ARGS__)  // expands a read list into R0..R4
  // read OUT (16 or 4 bytes) at lane base ADDR + stage offset (register so)
  // + OFF, forming the address in register TMP
#define A8_R(OUT, ADDR, OFF, TMP)                                                    \
  "v_add_u32 %[" TMP "], %[so], %[" ADDR "]\n\t"                                     \
  "ds_read_b128 %[" OUT "], %[" TMP "] offset:" OFF "\n\t"
  // read one scale byte at lane base ADDR + offset register OREG + OFF
#define A8_RB(OUT, ADDR, OREG, OFF, TMP)                                             \
  "v_add_u32 %[" TMP "], %[" OREG "], %[" ADDR "]\n\t"                               \
  "ds_read_u8 %[" OUT "], %[" TMP "] offset:" OFF "\n\t"
  // A fragments of two row tiles (k-groups h and h + 2 of the lane's rows, at
  // byte offsets O0 and O1 of the stage), the two lane addresses formed once
#define A8_RA(O0, O1)                                                                \
  "v_add_u32 %[u0], %[so], %[alo]\n\t"                                               \
  "v_add_u32 %[u1], %[so], %[ahi]\n\t"                                               \
  "ds_read_b128 %[nl0], %[u0] offset:" O0 "\n\t"                                     \
  "ds_read_b128 %[ng0], %[u1] offset:" O0 "\n\t"                                     \
  "ds_read_b128 %[nl1], %[u0] offset:" O1 "\n\t"                                     \
  "ds_read_b128 %[ng1], %[u1] offset:" O1 "\n\t"
  // their A scales (the scale ring at the A-scale offset) at O0 and O1
#define A8_RS(O0, O1)                                                                \
  "v_add_u32 %[u0], %[ao], %[as]\n\t"                                                \
  "ds_read_u8 %[ns0], %[u0] offset:" O0 "\n\t"                                       \
  "ds_read_u8 %[ns1], %[u0] offset:" O1 "\n\t"
  // first half: this step's second B fragment and its scale (b1, t1: the
  // oldest reads, needed by the third MFMA), then Q of this step (A rows
  // 64.., their scales 1024..)
#define A8_RQ                                                                        \
  A8_R("b1", "bc1", "0", "u0") A8_RB("t1", "bs1", "so", "0", "u1"),                  \
      A8_RA("4096", "6144") A8_RS("1024", "1536"),                                   \
      "s_waitcnt lgkmcnt(6)\n\t", "", ""
  // second half: P of the next step, then (after the last use of b0) its
  // first B fragment and scale; its b1, t1 are read by its first half
#define A8_RP                                                                        \
  "", A8_RA("0", "2048") A8_RS("0", "512"),                                          \
      A8_R("b0", "bc0", "0", "u0") A8_RB("t0", "bs0", "so", "0", "u1"), "", ""
#define A8_BASES                                                                     \
  [alo] "v"(a_lo), [ahi] "v"(a_hi), [bc0] "v"(bc_a[0]), [bc1] "v"(bc_a[1]),          \
      [as] "v"(as_a), [bs0] "v"(bs_a[0]), [bs1] "v"(bs_a[1])
#define A8_ACC                                                                       \
  [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]),               \
      [c11] "+v"(acc[1][1]), [c20] "+v"(acc[2][0]), [c21] "+v"(acc[2][1]),           \
      [c30] "+v"(acc[3][0]), [c31] "+v"(acc[3][1])
  uint32_t u0, u1;  // address registers of the blocks
  // first half of step kt (stage offset SO, A-scale offset AO): tiles 0, 1
  // from P; reads Q
#define A8_H1(SO, AO)                                                                \
  asm volatile("s_nop 4\n\t" A8_HALF_X(0, 1, A8_RQ) "s_waitcnt lgkmcnt(0)"           \
               : [nl0] "=&v"(ql0), [ng0] "=&v"(qg0), [nl1] "=&v"(ql1), [ng1] "=&v"(qg1), \
                 [ns0] "=&v"(sa2), [ns1] "=&v"(sa3), [u0] "=&v"(u0), [u1] "=&v"(u1),  \
                 [b1] "=&v"(b1), [t1] "=&v"(t1), A8_ACC                              \
               : [a0] "v"(join8(pl0, pg0)), [a1] "v"(join8(pl1, pg1)), [b0] "v"(b0),  \
                 [s0] "v"(sa0), [s1] "v"(sa1), [t0] "v"(t0), [so] "s"(SO), [ao] "s"(AO), \
                 A8_BASES                                                            \
               : "memory")
  // second half: tiles 2, 3 from Q; reads P, B and B scales of the next
  // step (stage offset SO, A-scale offset AO)
#define A8_H2(SO, AO)                                                                \
  asm volatile("s_nop 4\n\t" A8_HALF_X(2, 3, A8_RP) "s_waitcnt lgkmcnt(0)"           \
               : [nl0] "=&v"(pl0), [ng0] "=&v"(pg0), [nl1] "=&v"(pl1), [ng1] "=&v"(pg1), \
                 [ns0] "=&v"(sa0), [ns1] "=&v"(sa1), [u0] "=&v"(u0), [u1] "=&v"(u1),  \
                 [b0] "+v"(b0), [t0] "+v"(t0), A8_ACC                                \
               : [a0] "v"(join8(ql0, qg0)), [a1] "v"(join8(ql1, qg1)), [b1] "v"(b1),  \
                 [s0] "v"(sa2), [s1] "v"(sa3), [t1] "v"(t1), [so] "s"(SO), [ao] "s"(AO), \
                 A8_BASES                                                            \
               : "memory")
#define A8_H2_LAST()                                                                 \
  asm volatile("s_nop 4\n\t" A8_HALF(2, 3, "", "", "", "", "") MFMA_TAIL             \
               : A8_ACC                                                              \
               : [a0] "v"(join8(ql0, qg0)), [a1] "v"(join8(ql1, qg1)), [b0] "v"(b0),  \
                 [b1] "v"(b1), [s0] "v"(sa2), [s1] "v"(sa3), [t0] "v"(t0), [t1] "v"(t1))
  // Step kt of a wave with rows in the segment: first half; then wait until
  // steps <= kt + 1 have landed and barrier (every wave is then done reading
  // the stage of step kt, which takes step kt + NST8); then the second
  // half. Waves past the segment end run the same waits, barriers and
  // copies.
  // The wait: this wave's copies issued after those of step kt + 1 may stay
  // in flight (they complete in order): the step batches of kt + 2 ..
  // kt + NST8 - 1 and the A-scale group copies of the syncs of steps
  // kt - NST8 + 1 .. kt - 1 (each sync issues its batch, then its group copy).
  // Every wave copies at least ACP + BCP pieces per step, so while NST8 - 2
  // later batches are in flight, waiting down to NMIN copies is at least as
  // strict as the exact count (a constant wait, no branches); the exact count
  // is formed only for the last steps.
  constexpr int NMIN = (SH::ACP + SH::BCP) * (NST8 - 2);
#define A8_SYNC()                                                                    \
  do {                                                                               \
    if (kt + NST8 - 1 <= nk - 1) {                                                   \
      wait_vmcnt<NMIN>();                                                            \
    } else {                                                                         \
      int n = per * (min(nk - 1, kt + NST8 - 1) - min(kt + 1, nk - 1));              \
      const int lo = max(0, kt - (NST8 - 1)), hi = kt - 1;                           \
      if (wave < SH::NAS && hi >= lo)                                                \
        n += ((wave - (kt_begin + lo) % kSG + kSG) % kSG) <= hi - lo;                \
      wait_vmcnt_dyn(n);                                                             \
    }                                                                                \
    __builtin_amdgcn_s_barrier();                                                    \
    asm volatile("" ::: "memory");                                                   \
    if (kt + NST8 < nk) issue(kt_begin + kt + NST8, so);                             \
    if (wave < SH::NAS && (unsigned)(kt_begin + kt) % kSG == (unsigned)wave)          \
      issue_group((unsigned)(kt_begin + kt) / kSG + 2);                              \
  } while (0)

  // the first A-scale groups, then the copies of the first NST8 steps
  if (wave < SH::NAS) {
    const int g0 = kt_begin / kSG;
    issue_group(g0);
    issue_group(g0 + 1);
    issue_group(g0 + 2);
  }
#pragma unroll
  for (int s = 0; s < NST8; ++s)
    if (s < nk) issue(kt_begin + s, s * SB8);
  wait_vmcnt_dyn(per * min(nk - 1, NST8 - 1));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int kt = 0;
  uint32_t so = 0;  // stage offset of step kt
  auto next_stage = [](uint32_t o) { return o + SB8 == NST8 * SB8 ? 0u : o + SB8; };
  if (idle) {
    for (; kt < nk; ++kt) {
      A8_SYNC();
      so = next_stage(so);
    }
  } else {
    // step 0's P, B and scales
    asm volatile(A8_R("nl0", "alo", "0", "u0") A8_R("ng0", "ahi", "0", "u1")
                 A8_R("nl1", "alo", "2048", "u0") A8_R("ng1", "ahi", "2048", "u1")
                 A8_R("nb0", "bc0", "0", "u0") A8_RB("ns0", "as", "ao", "0", "u1")
                 A8_RB("ns1", "as", "ao", "512", "u0") A8_RB("nt0", "bs0", "so", "0", "u1")
                 "s_waitcnt lgkmcnt(0)"
                 : [nl0] "=&v"(pl0), [ng0] "=&v"(pg0), [nl1] "=&v"(pl1), [ng1] "=&v"(pg1),
                   [nb0] "=&v"(b0), [ns0] "=&v"(sa0), [ns1] "=&v"(sa1), [nt0] "=&v"(t0),
                   [u0] "=&v"(u0), [u1] "=&v"(u1)
                 : [so] "s"(0u), [ao] "s"(as_off(kt_begin)), A8_BASES
                 : "memory");
    for (; kt + 1 < nk; ++kt) {
      const uint32_t so1 = next_stage(so);
      const uint32_t ao0 = ao_cur();
      ao_next();
      A8_H1(so, ao0);
      A8_SYNC();
      A8_H2(so1, ao_cur());
      so = so1;
    }
    A8_H1(so, ao_cur());
    A8_SYNC();
    A8_H2_LAST();
  }
  // the last MFMAs finish writing the accumulators before any VALU reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#undef A8_SYNC
#undef A8_H2_LAST
#undef A8_H2
#undef A8_H1
#undef A8_ACC
#undef A8_BASES
#undef A8_RP
#undef A8_RQ
#undef A8_RS
#undef A8_RA
#undef A8_RB
#undef A8_R
#undef A8_HALF_X
#undef A8_HALF
#undef A8_MF

  bool lost = false;  // a wave that lost a split part stores NaN
  if (jb.S > 1 && !split_exchange(a, jb, acc, wave, lane, tid, lost)) return;

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
    uint8_t* Hs = Hc + (size_t)a.rows * N;  // grouped scales follow the codes
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
      uint32_t s = mxfp8_block(v, q);
      if (lost) {  // e4m3 NaN codes and the e8m0 NaN scale
        s = 0xFFu;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = 0x7F7F7F7Fu;
      }
      if (grow < row_end && f0 < N) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Hc + (size_t)grow * N + f0);
        dst[0] = u32x4_t{q[0], q[1], q[2], q[3]};
        dst[1] = u32x4_t{q[4], q[5], q[6], q[7]};
        Hs[grouped_scale(grow, f0 / 32, a.rows)] = (uint8_t)s;
      }
    }
  } else {
    store_down_tile(a, acc, smem, wave, lane, row0 + 128 * wm, row_end, n0, bcol, lost);
  }
}

template <int MODE>
__global__ __launch_bounds__(512) void gemm_a8_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS8];
  Job jb;
  if (!schedule_tile<BK8>(a, blockIdx.x, jb)) return;
  // (Half-row waves skipping the MFMAs of rows 64-127, as in gemm16.hip,
  // made this kernel's gate/up 14 % slower; not used here.)
  if (__builtin_amdgcn_readfirstlane((int)jb.wide)) gemm_a8_body<MODE, true>(a, jb, smem);
  else gemm_a8_body<MODE, false>(a, jb, smem);
}

}  // namespace

hipError_t launch_quant_mxfp8(const void* x, long long rows, int K, uint8_t* codes, uint8_t* scales,
                              bool grouped, hipStream_t s) {
  const long long nb = rows * (K / 32);
  if (nb <= 0) return hipSuccess;
  const unsigned grid = (unsigned)ceil_div(nb, 256);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (grouped) quant_mxfp8_kernel<true><<<grid, 256, 0, s>>>(xb, rows, K / 32, codes, scales);
  else quant_mxfp8_kernel<false><<<grid, 256, 0, s>>>(xb, rows, K / 32, codes, scales);
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
  a.n_tiles_n = swiglu ? ceil_div(p.N, TN / 2) : ceil_div(p.N, TN);
  a.n_tiles_w = swiglu ? ceil_div(p.N, TNW / 2) : ceil_div(p.N, TNW);
  a.split_ws = p.split_ws;
  a.split_flags = p.split_flags;
  a.split_wait = p.split_wait;
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

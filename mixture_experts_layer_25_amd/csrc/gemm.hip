// Grouped expert GEMMs on MFMA (bf16 in, fp32 accumulate).
//
// "ops-transformer MoE operator on Ascend NPU", optimisation 3: every
// expert's matmul in one launch, with a different row count per expert.
// "FFN, SwiGLU and MoE" sec. 2: H = SiLU(X W_gate) * (X W_up), Y = H W_down.
// "DeepSeek-V4.1-Flash fine-grained MoE (5A)" sec. 1, 3: gate and up are
// clamped to [-L, L] before SiLU(gate)*up; routed experts may be FP4
// (here MXFP4: e2m1 codes with an e8m0 scale per 32 K-elements).
//
// Two kernels share the operand formats below.
//
// MXFP4 weights (gemm_kernel<MODE, true>): tile 128 rows x 512 B-columns x
// 32 k per stage, 256 threads (4 waves, 128 x 128 each, 256 accumulators).
//   SwiGLU: the 512 B-columns are 256 gate and the same 256 up columns, so
//   each wave's accumulators hold gate and up of the same (row, f) and the
//   epilogue forms h = SiLU(clamp(g)) * clamp(u) in registers and stores
//   bf16 H; the gate/up intermediate never reaches memory.
//   Down: 512 output columns, fp32 stores.
//   Two LDS stages and three register sets: during step kt the MFMAs read
//   LDS stage kt%2, the registers holding step kt+1 are stored to the other
//   stage, and the global loads of steps kt+2 and kt+3 are in flight.
// bf16 weights (gemm_bf16_kernel<MODE>): 256 x 256 tiles, 8 waves,
//   asynchronous global->LDS copies five stages deep (described at the
//   kernel).
//
// Operands reach MFMA (v_mfma_f32_32x32x16_bf16) K-contiguous: a lane's
// fragment is 8 consecutive k of one row (A) or one column (B).
//   A (X rows, K-contiguous): 16-byte loads, stored as [row][4 k-groups] and
//   read with ds_read_b128.
//   B bf16 ([K][N], N-contiguous): whole k-rows are stored untouched; the
//   MFMA fragment is read with the gfx950 transposing LDS load
//   ds_read_b64_tr_b16 (within a 16-lane group, lane i receives element i of
//   the 4 rows the group points at), two per fragment, so no transpose runs
//   on the vector ALUs.
//   B MXFP4 (stored K-contiguous per column): each thread loads one column's
//   32 codes and scale, converts them exactly to bf16 with
//   v_cvt_scalef32_pk_bf16_fp4 and stores [column][4 k-groups] like A.
// LDS 16-byte slots are XOR-swizzled (A and MXFP4 B: k-group ^ (row/2 mod 4);
// bf16 B: chunk ^ 4*(k mod 4)) so that the 16 lanes sharing a 256-byte
// LDS cycle (64 banks on gfx950) hit 16 distinct 16-byte bank groups on the
// stores and on the MFMA fragment reads (checked with the LDS bank-conflict
// counter).
//
// Workgroup -> tile: workgroup b runs on XCD (b mod 8), and each XCD walks a
// contiguous range of the tile order (tile_of, expert_tile_of), whose
// neighbours share weight and activation slabs in that XCD's L2.
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
  float* split_ws;      // partial accumulators of split tiles (bf16 kernel), or nullptr
  int32_t* split_flags; // one ready flag per partial slot, zero between launches
};


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

// Slot permutation of the 4 k-groups of a 64-byte row: rows r..r+15 then
// put any one k-group in 16 distinct 16-byte bank groups, and so do rows
// r..r+3 with all 4 k-groups (the store pattern).
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Workgroup barrier for LDS hand-off: waits for this wave's LDS accesses,
// not for its global loads in flight (a plain __syncthreads also drains
// those, which would empty the prefetch pipeline).
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// 32 MXFP4 codes of one column (k0..k0+31) and its scale -> 4 LDS entries of
// 8 bf16 (k-group q at slot q ^ swz4(n) of the column's 64 bytes).
// The hardware conversion scales each e2m1 pair by 2^(s-127) exactly; for
// scale codes at the ends of the range the product is formed in fp32 instead.
__device__ __forceinline__ void store_b_mx(unsigned char* Bs, u32x4_t codes, uint32_t s, int n) {
  const float sc = e8m0_scale(s);
  const bool hw = s >= 2u && s <= 252u;
  unsigned char* col = Bs + n * 64;
  const int sw = swz4(n);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t word = codes[q];  // codes of k = 8q .. 8q+7
    u32x4_t o;
    if (hw) {
      o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0));
      o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1));
      o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2));
      o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3));
    } else {
      o.x = mx_pair(word & 0xFFu, sc);
      o.y = mx_pair((word >> 8) & 0xFFu, sc);
      o.z = mx_pair((word >> 16) & 0xFFu, sc);
      o.w = mx_pair(word >> 24, sc);
    }
    *reinterpret_cast<u32x4_t*>(col + ((q ^ sw) * 16)) = o;
  }
}

// Tile order: N-tiles in groups of 4; inside a group, M-tile major and the
// 4 N-tiles minor. The 32 workgroups an XCD runs at once then cover about
// 8 M-tiles x 4 N-tiles (one expert's weight columns), so its L2 serves each
// weight slab to ~8 workgroups and each x_perm slab to 4.
__device__ __forceinline__ void tile_of(int L, int MT, int NT, int& mt, int& nt) {
  constexpr int G = 4;
  const int g = L / (MT * G);
  const int rem = L - g * MT * G;
  const int gs = min(G, NT - g * G);
  mt = rem / gs;
  nt = g * G + rem % gs;
}

// Tile order of the bf16 kernel, by expert: an expert's tiles are
// contiguous, in groups of up to 8 of its M-tiles; inside a group N-tile
// major and M-tile minor. The 32 workgroups an XCD runs at once then cover
// about 8 M-tiles x 4 N-tiles of one expert, so each weight slab is fetched
// once and shared by all those M-tiles, and each activation slab by 4
// N-tiles. With a tile map, the M-tiles t / NT and the tile's own belong
// to the same expert (an expert's tiles span whole rows of NT), which
// gives the expert's first M-tile and count without a search.
__device__ __forceinline__ void expert_tile_of(int t, int MT, int NT, const int32_t* tilemap,
                                               const int32_t* offsets, int bm, int& mt, int& nt) {
  constexpr int MG = 8;
  int first = 0, m = MT;
  if (tilemap) {
    const int g = t / NT;
    const int e = tilemap[1 + 2 * g];
    const int seg = offsets[e];
    first = g - (tilemap[2 + 2 * g] - seg) / bm;
    m = (offsets[e + 1] - seg + bm - 1) / bm;
  }
  const int r = t - first * NT;
  const int gi = r / (MG * NT);
  const int gsz = min(MG, m - gi * MG);
  const int rr = r - gi * MG * NT;
  nt = rr / gsz;
  mt = first + gi * MG + rr % gsz;
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
  int mt, nt;
  tile_of(L, a.max_tiles, a.n_tiles_n, mt, nt);
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
  const int nk = K / BK;

  // ---- A: LDS [128 rows][4 slots of 8 k], 64 bytes per row; k-group q of
  // row m sits at slot q ^ swz4(m). Thread t moves chunks t and
  // t + 256 (row chunk/4, k-group chunk%4): 4 threads read 64 contiguous
  // bytes of a row.
  const int am0 = tid >> 2, am1 = am0 + 64, aq = tid & 3;
  const uint16_t* a_g0 = a.A + (size_t)min(row0 + am0, row_end - 1) * K + 8 * aq;
  const uint16_t* a_g1 = a.A + (size_t)min(row0 + am1, row_end - 1) * K + 8 * aq;
  const int a_l0 = am0 * 64 + ((aq ^ swz4(am0)) * 16);
  const int a_l1 = am1 * 64 + ((aq ^ swz4(am1)) * 16);

  // ---- B bf16 ([K][N] rows): LDS [32 k-rows][64 chunks of 8 columns],
  // 1 KB per row; chunk c of row k sits at slot c ^ (2*(k & 3)). Wave w
  // moves rows 8w..8w+7, lane l chunk l of each: 512 contiguous bytes of
  // W_gate and of W_up (or 1 KB of W_down) per row.
  const uint16_t* b_g = nullptr;
  if (!MX) {
    int col;
    const uint16_t* base;
    if (MODE == MODE_SWIGLU) {
      col = n0 + 8 * (lane & 31);
      base = static_cast<const uint16_t*>(lane >= 32 ? a.B1 : a.B0);
    } else {
      col = n0 + 8 * lane;
      base = static_cast<const uint16_t*>(a.B0);
    }
    if (col + 8 > N) col = 0;  // columns past N: any valid data, never stored
    b_g = base + ((size_t)e * K + 8 * wave) * N + col;
  }
  // ---- B MXFP4 (K-contiguous codes per column): LDS [512 columns][4 slots]
  // like A; thread t converts columns t and t + 256.
  const uint8_t* mx_src0 = nullptr;
  const uint8_t* mx_src1 = nullptr;
  const uint8_t* mx_scl0 = nullptr;
  const uint8_t* mx_scl1 = nullptr;
  if (MX) {
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
    const size_t r0 = (size_t)e * N + (col0 < N ? col0 : 0);
    const size_t r1 = (size_t)e * N + (col1 < N ? col1 : 0);
    mx_src0 = codes0 + r0 * (K / 2);
    mx_src1 = codes1 + r1 * (K / 2);
    mx_scl0 = scl0 + r0 * (K / 32);
    mx_scl1 = scl1 + r1 * (K / 32);
  }

  // One stage's worth of global data waits in registers between its load
  // and its LDS store; there are two such register sets (suffix 0 / 1).
#define MOE_DECL_SET(S)                                    \
  u32x4_t ra0_##S, ra1_##S, rb_##S[8], rm0_##S, rm1_##S;  \
  uint32_t rs0_##S = 127u, rs1_##S = 127u;
#define MOE_LOAD_SET(S, kt_)                                                                   \
  do {                                                                                         \
    const int k0_ = (kt_) * BK;                                                                \
    ra0_##S = *reinterpret_cast<const u32x4_t*>(a_g0 + k0_);                                     \
    ra1_##S = *reinterpret_cast<const u32x4_t*>(a_g1 + k0_);                                     \
    if (!MX) {                                                                                 \
      const uint16_t* bp_ = b_g + (size_t)k0_ * N;                                             \
      rb_##S[0] = *reinterpret_cast<const u32x4_t*>(bp_);                                        \
      rb_##S[1] = *reinterpret_cast<const u32x4_t*>(bp_ + (size_t)N);                            \
      rb_##S[2] = *reinterpret_cast<const u32x4_t*>(bp_ + (size_t)2 * N);                        \
      rb_##S[3] = *reinterpret_cast<const u32x4_t*>(bp_ + (size_t)3 * N);                        \
      rb_##S[4] = *reinterpret_cast<const u32x4_t*>(bp_ + (size_t)4 * N);                        \
      rb_##S[5] = *reinterpret_cast<const u32x4_t*>(bp_ + (size_t)5 * N);                        \
      rb_##S[6] = *reinterpret_cast<const u32x4_t*>(bp_ + (size_t)6 * N);                        \
      rb_##S[7] = *reinterpret_cast<const u32x4_t*>(bp_ + (size_t)7 * N);                        \
    } else {                                                                                   \
      rm0_##S = *reinterpret_cast<const u32x4_t*>(mx_src0 + k0_ / 2);                            \
      rm1_##S = *reinterpret_cast<const u32x4_t*>(mx_src1 + k0_ / 2);                            \
      rs0_##S = mx_scl0[k0_ / 32];                                                             \
      rs1_##S = mx_scl1[k0_ / 32];                                                             \
    }                                                                                          \
  } while (0)
#define MOE_STORE_SET(S, stage_)                                                               \
  do {                                                                                         \
    unsigned char* As_ = smem + (stage_) * STAGE;                                              \
    unsigned char* Bs_ = As_ + A_STAGE;                                                        \
    *reinterpret_cast<u32x4_t*>(As_ + a_l0) = ra0_##S;                                           \
    *reinterpret_cast<u32x4_t*>(As_ + a_l1) = ra1_##S;                                           \
    if (!MX) {                                                                                 \
      unsigned char* bw_ = Bs_ + (8 * wave) * 1024;                                            \
      *reinterpret_cast<u32x4_t*>(bw_ + 0 * 1024 + ((lane ^ 0) * 16)) = rb_##S[0];               \
      *reinterpret_cast<u32x4_t*>(bw_ + 1 * 1024 + ((lane ^ 4) * 16)) = rb_##S[1];               \
      *reinterpret_cast<u32x4_t*>(bw_ + 2 * 1024 + ((lane ^ 8) * 16)) = rb_##S[2];               \
      *reinterpret_cast<u32x4_t*>(bw_ + 3 * 1024 + ((lane ^ 12) * 16)) = rb_##S[3];               \
      *reinterpret_cast<u32x4_t*>(bw_ + 4 * 1024 + ((lane ^ 0) * 16)) = rb_##S[4];               \
      *reinterpret_cast<u32x4_t*>(bw_ + 5 * 1024 + ((lane ^ 4) * 16)) = rb_##S[5];               \
      *reinterpret_cast<u32x4_t*>(bw_ + 6 * 1024 + ((lane ^ 8) * 16)) = rb_##S[6];               \
      *reinterpret_cast<u32x4_t*>(bw_ + 7 * 1024 + ((lane ^ 12) * 16)) = rb_##S[7];               \
    } else {                                                                                   \
      store_b_mx(Bs_, rm0_##S, rs0_##S, tid);                                                  \
      store_b_mx(Bs_, rm1_##S, rs1_##S, tid + 256);                                            \
    }                                                                                          \
  } while (0)
  MOE_DECL_SET(0)
  MOE_DECL_SET(1)
  MOE_DECL_SET(2)

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

  const int lrow = lane & 31;
  const int lq = lane >> 5;
  // per-lane parts of the transposed B read (16-lane groups): k-row within
  // 4, column offset
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  auto compute = [&](int stage) __attribute__((always_inline)) {
    const unsigned char* As = smem + stage * STAGE;
    const unsigned char* Bs = As + A_STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int q = 2 * kk + lq;
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 32 * i + lrow;
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + m * 64 + ((q ^ swz4(m)) * 16));
      }
      if (MX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = bcol[j] + lrow;
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + n * 64 + ((q ^ swz4(n)) * 16));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = bcol[j] + tr_col;
          const int chunk = col >> 3;
          const int byte = (col & 7) * 2;
          const int r0 = 16 * kk + 8 * lq + tr_row;  // r0 & 3 == tr_row
          const s16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(Bs + r0 * 1024 + ((chunk ^ (4 * tr_row)) * 16) + byte));
          const s16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(Bs + (r0 + 4) * 1024 + ((chunk ^ (4 * tr_row)) * 16) + byte));
          const s16x8_t hv = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          bfr[j] = __builtin_bit_cast(bf16x8_t, hv);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // Three register sets: while step kt is multiplied from LDS stage kt%2,
  // the registers holding step kt+1 are stored to the other stage and the
  // loads of steps kt+2 and kt+3 are in flight, so about three steps of
  // MFMA work cover the memory latency. Loads are issued unconditionally
  // (clamped to the last step) so that the wait before each store covers
  // only its own set.
  MOE_LOAD_SET(0, 0);
  MOE_LOAD_SET(1, min(1, nk - 1));
  MOE_LOAD_SET(2, min(2, nk - 1));
  MOE_STORE_SET(0, 0);
  block_barrier();
#define MOE_STEP(L, S, k_)                                                  \
  do {                                                                      \
    MOE_LOAD_SET(L, min((k_) + 3, nk - 1));                                 \
    asm volatile("" ::: "memory"); /* loads before this step's LDS reads */ \
    compute((k_) & 1);                                                      \
    asm volatile("" ::: "memory"); /* stores after this step's LDS reads */ \
    MOE_STORE_SET(S, ((k_) + 1) & 1);                                       \
    block_barrier();                                                        \
  } while (0)
  int kt = 0;
  for (; kt + 3 < nk; kt += 3) {
    MOE_STEP(0, 1, kt);
    MOE_STEP(1, 2, kt + 1);
    MOE_STEP(2, 0, kt + 2);
  }
  // last 1..3 steps: their data is already in sets 0, 1, 2
  compute(kt & 1);
  if (kt + 1 < nk) {
    MOE_STORE_SET(1, (kt + 1) & 1);
    block_barrier();
    compute((kt + 1) & 1);
    if (kt + 2 < nk) {
      MOE_STORE_SET(2, (kt + 2) & 1);
      block_barrier();
      compute((kt + 2) & 1);
    }
  }
#undef MOE_STEP
#undef MOE_DECL_SET
#undef MOE_LOAD_SET
#undef MOE_STORE_SET

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

// ---------------------------------------------------------------------------
// bf16 weights: 256 x 256 tiles, 8 waves (two per SIMD), asynchronous
// global->LDS copies.
//
// Tile: 256 rows x 256 B-columns x 32 k per stage (SwiGLU: 128 gate and
// the same 128 up columns). A square tile moves the fewest bytes per flop
// that 64K fp32 accumulators per CU allow: 32 KB per 32-k step for 4.2 MFLOP.
// Each wave computes 128 rows x 64 B-columns (4 x 2 MFMA tiles, 128 fp32
// accumulators), so two waves share each SIMD and one's LDS waits are
// covered by the other's MFMAs. SwiGLU: wave (wm, wn) owns rows
// 128wm..128wm+127 and f = 32wn..32wn+31, i.e. gate B-column 32wn + l and
// up B-column 128 + 32wn + l.
// Global data goes straight to LDS with global_load_lds_dwordx4 (no
// register staging), NSTAGE_DMA stages deep: the copies of step kt+5 are
// issued in the middle of step kt, right after the barrier that certifies
// the copies of step kt+1 and that every wave is done reading stage kt.
// Each 32-k step is two half-steps of 16 k; the MFMA fragments of a
// half-step are read from LDS while the MFMAs of the previous half-step
// run (two register sets), so LDS latency hides behind MFMA work.
constexpr int BM2 = kBM_BF16;       // 256
constexpr int BN2 = 256;            // B-columns per tile
constexpr int A_STAGE2 = BM2 * BK * 2;   // 16 KB
constexpr int B_STAGE2 = BN2 * BK * 2;   // 16 KB
constexpr int STAGE2 = A_STAGE2 + B_STAGE2;
constexpr int kCUsPerXCD = 32;      // MI355X: 256 CUs in 8 XCDs
constexpr int kMaxSplit = 8;        // K-parts of a split tile
// Wait states after an asm block's last MFMA so that whatever the compiler
// places next (a register move, a spill, a VALU read) sees the finished
// accumulator: the compiler does not look inside asm for MFMA hazards.
#define MFMA_TAIL "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
constexpr int NSTAGE_DMA = 5;       // 5 x 32 KB = 160 KB, all of the LDS
static_assert(NSTAGE_DMA >= 2 && NSTAGE_DMA <= 5, "copy waits are written for 2..5 stages");

typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(p);
}
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_base, 16, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---- bf16 kernels: workgroup -> (tile, k-range). Workgroup b runs on XCD
// x = b mod 8 as that XCD's i-th workgroup. The real tiles (M-tiles from
// the tile map x N-tiles, in expert_tile_of order) are cut into 8
// contiguous ranges, one per XCD. An XCD's whole rounds of kCUsPerXCD
// tiles run as whole tiles; the tiles of its last, partial round are each
// split along K into S parts (S x remainder <= kCUsPerXCD) so that the
// last round keeps every CU busy. Parts 0..S-2 leave fp32 partial sums in
// a workspace slot and raise its flag; part S-1 (the highest workgroup
// index of the tile, so the parts it waits for were dispatched before it)
// adds them in part order and runs the epilogue.
struct Job {
  int e, row0, row_end, nt, S, part, slot0, kt_begin, nk;
};
__device__ __forceinline__ bool schedule_bf16(const Args& a, int b, Job& j) {
  const int xcd = b & 7, wi = b >> 3;
  const int MT = a.tilemap ? a.tilemap[0] : a.max_tiles;
  const int total = MT * a.n_tiles_n;
  const int t_lo = (int)((long long)total * xcd / 8);
  const int t_hi = (int)((long long)total * (xcd + 1) / 8);
  const int whole = (t_hi - t_lo) / kCUsPerXCD * kCUsPerXCD;
  const int rem = t_hi - t_lo - whole;
  const int nk_all = a.K / BK;
  int tile;
  j.S = 1;
  j.part = 0;
  j.slot0 = 0;
  if (wi < whole) {
    tile = t_lo + wi;
  } else {
    if (a.split_flags && rem > 0) j.S = min(min(kMaxSplit, kCUsPerXCD / rem), nk_all);
    const int u = wi - whole;
    if (u >= rem * j.S) return false;
    tile = t_lo + whole + u / j.S;
    j.part = u % j.S;
    j.slot0 = xcd * kCUsPerXCD + (u / j.S) * (j.S - 1);
  }
  int mt;
  expert_tile_of(tile, MT, a.n_tiles_n, a.tilemap, a.offsets, kBM_BF16, mt, j.nt);
  if (a.tilemap) {
    j.e = a.tilemap[1 + 2 * mt];
    j.row0 = a.tilemap[2 + 2 * mt];
    j.row_end = a.offsets[j.e + 1];
  } else {
    j.e = 0;
    j.row0 = mt * kBM_BF16;
    j.row_end = a.rows;
  }
  j.kt_begin = j.part * nk_all / j.S;
  j.nk = (j.part + 1) * nk_all / j.S - j.kt_begin;
  return true;
}

template <int MODE>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[NSTAGE_DMA * STAGE2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;  // 0..7
  const int wm = wave >> 2;   // row half
  const int wn = wave & 3;    // column quarter

  Job jb;
  if (!schedule_bf16(a, blockIdx.x, jb)) return;
  const int e = jb.e, row0 = jb.row0, row_end = jb.row_end, nt = jb.nt;
  const int S = jb.S, part = jb.part, slot0 = jb.slot0, kt_begin = jb.kt_begin, nk = jb.nk;
  const int K = a.K, N = a.N;
  const int n0 = MODE == MODE_SWIGLU ? nt * 128 : nt * 256;

  // ---- A copies: LDS entry p = 4m + s (16 bytes) holds k-group s ^ swz4(m)
  // of row m; copy r of wave w fills entries 512r + 64w .. +63.
  const uint16_t* a_g[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int p = 512 * r + tid, m = p >> 2, q = (p & 3) ^ swz4(m);
    a_g[r] = a.A + (size_t)min(row0 + m, row_end - 1) * K + kt_begin * BK + 8 * q;
  }
  // ---- B copies: LDS k-row (512 bytes = 32 chunks of 8 columns) slot c
  // holds chunk c ^ (4*(k & 3)); copy r of wave w fills rows 4w + 2r and
  // 4w + 2r + 1 (lanes 0-31 and 32-63).
  const uint16_t* b_g[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int k = 4 * wave + 2 * r + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (k & 3));
    int col;
    const uint16_t* base;
    if (MODE == MODE_SWIGLU) {
      col = n0 + 8 * (c & 15);
      base = static_cast<const uint16_t*>(c >= 16 ? a.B1 : a.B0);
    } else {
      col = n0 + 8 * c;
      base = static_cast<const uint16_t*>(a.B0);
    }
    if (col + 8 > N) col = 0;  // columns past N: any valid data, never stored
    b_g[r] = base + ((size_t)e * K + kt_begin * BK + k) * N + col;
  }
  // copies of step kt into the stage at byte offset `so`
  auto issue = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    unsigned char* As = smem + so;
    unsigned char* Bs = As + A_STAGE2;
    const int k0 = kt * BK;
    dma16(a_g[0] + k0, As + wave * 1024);
    dma16(a_g[1] + k0, As + 8192 + wave * 1024);
    dma16(b_g[0] + (size_t)k0 * N, Bs + (4 * wave) * 512);
    dma16(b_g[1] + (size_t)k0 * N, Bs + (4 * wave + 2) * 512);
  };
  auto issue_a = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    unsigned char* As = smem + so;
    const int k0 = kt * BK;
    dma16(a_g[0] + k0, As + wave * 1024);
    dma16(a_g[1] + k0, As + 8192 + wave * 1024);
  };
  auto issue_b = [&](int kt, uint32_t so) __attribute__((always_inline)) {
    unsigned char* Bs = smem + so + A_STAGE2;
    const int k0 = kt * BK;
    dma16(b_g[0] + (size_t)k0 * N, Bs + (4 * wave) * 512);
    dma16(b_g[1] + (size_t)k0 * N, Bs + (4 * wave + 2) * 512);
  };
  constexpr int PER = 4;  // copies per thread per stage

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
  //   A: row m = 128 wm + lrow, k-group 2 kk + lq of the 32-k step
  //      (fragment i is 32 rows = 2048 bytes further).
  //   B: transposed reads of k-rows 8 lq + tr_row and 8 lq + tr_row + 4
  //      (2048 bytes apart) of the half-step kk (kk = 1 is 16 k-rows =
  //      8192 bytes further), for the wave's two B-column bases.
  uint32_t a_addr[2], b_addr[2];
  {
    const int m = 128 * wm + lrow;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      a_addr[kk] = smem_addr + m * 64 + (((2 * kk + lq) ^ swz4(m)) * 16);
    const int tr_row = (lane & 15) >> 2;
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = bcol[j] + tr_col;
      const int r0 = 8 * lq + tr_row;  // r0 & 3 == tr_row
      b_addr[j] = smem_addr + A_STAGE2 + r0 * 512 + ((col >> 3) ^ (4 * tr_row)) * 16 + (col & 7) * 2;
    }
  }

  // Fragment registers, two sets: while the MFMAs of one half-step read one
  // set, the LDS reads of the next half-step fill the other. Each read and
  // its MFMAs sit in one asm block that ends by waiting for the reads, so no
  // load is ever in flight outside the block that issued it (the transposing
  // read is written in asm because the compiler cannot tell it apart from
  // the LDS writes of the copies still in flight). Each block starts with a
  // few wait states so that a register the compiler wrote just before (the
  // zeroed accumulators, a fragment half it had to move) is settled before
  // an MFMA reads it.
  bf16x8_t xa0, xa1, xa2, xa3, xb0, xb1;
  bf16x8_t ya0, ya1, ya2, ya3, yb0, yb1;
  s16x4_t h0, h1, h2, h3;
#define MOE_JOIN_B(B0, B1)                                                           \
  do {                                                                               \
    const s16x8_t v0 = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};    \
    const s16x8_t v1 = {h2[0], h2[1], h2[2], h2[3], h3[0], h3[1], h3[2], h3[3]};    \
    B0 = __builtin_bit_cast(bf16x8_t, v0);                                          \
    B1 = __builtin_bit_cast(bf16x8_t, v1);                                          \
  } while (0)
#define MOE_MF_4                                                                    \
  "v_mfma_f32_32x32x16_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"                       \
  "v_mfma_f32_32x32x16_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"                       \
  "v_mfma_f32_32x32x16_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"                       \
  "v_mfma_f32_32x32x16_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"                       \
  "v_mfma_f32_32x32x16_bf16 %[c20], %[a2], %[b0], %[c20]\n\t"                       \
  "v_mfma_f32_32x32x16_bf16 %[c21], %[a2], %[b1], %[c21]\n\t"                       \
  "v_mfma_f32_32x32x16_bf16 %[c30], %[a3], %[b0], %[c30]\n\t"                       \
  "v_mfma_f32_32x32x16_bf16 %[c31], %[a3], %[b1], %[c31]\n\t"
#define MOE_READS(OFF0, OFF1)                                                       \
  "ds_read_b128 %[na0], %[aa]\n\t"                                                  \
  "ds_read_b128 %[na1], %[aa] offset:2048\n\t"                                      \
  "ds_read_b128 %[na2], %[aa] offset:4096\n\t"                                      \
  "ds_read_b128 %[na3], %[aa] offset:6144\n\t"                                      \
  "ds_read_b64_tr_b16 %[h0], %[ba0] offset:" OFF0 "\n\t"                            \
  "ds_read_b64_tr_b16 %[h1], %[ba0] offset:" OFF1 "\n\t"                            \
  "ds_read_b64_tr_b16 %[h2], %[ba1] offset:" OFF0 "\n\t"                            \
  "ds_read_b64_tr_b16 %[h3], %[ba1] offset:" OFF1 "\n\t"
#define MOE_ACC_OUT                                                                 \
  [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]),              \
      [c11] "+v"(acc[1][1]), [c20] "+v"(acc[2][0]), [c21] "+v"(acc[2][1]),          \
      [c30] "+v"(acc[3][0]), [c31] "+v"(acc[3][1])
  // reads of a half-step into set N (A at AA, B at BA0/BA1 + OFF0/OFF1) while
  // the MFMAs (string MF) consume set C
#define MOE_RM_ASM(OFF0, OFF1, AA, BA0, BA1, N, C, MF)                              \
  asm volatile("s_nop 4\n\t" MOE_READS(OFF0, OFF1) MF "s_waitcnt lgkmcnt(0)"       \
               : [na0] "=&v"(N##a0), [na1] "=&v"(N##a1), [na2] "=&v"(N##a2),         \
                 [na3] "=&v"(N##a3), [h0] "=&v"(h0), [h1] "=&v"(h1),                 \
                 [h2] "=&v"(h2), [h3] "=&v"(h3), MOE_ACC_OUT                        \
               : [a0] "v"(C##a0), [a1] "v"(C##a1), [a2] "v"(C##a2),                  \
                 [a3] "v"(C##a3), [b0] "v"(C##b0), [b1] "v"(C##b1),                  \
                 [aa] "v"(AA), [ba0] "v"(BA0), [ba1] "v"(BA1)                        \
               : "memory")
#define MOE_READ_MMA(OFF0, OFF1, AA, BA0, BA1, N, C)                                \
  do {                                                                              \
    MOE_RM_ASM(OFF0, OFF1, AA, BA0, BA1, N, C, MOE_MF_4);                           \
    MOE_JOIN_B(N##b0, N##b1);                                                       \
  } while (0)
  // MFMAs only, on set y (the last half-step)
#define MOE_MMA_ASM(MF)                                                             \
  asm volatile("s_nop 4\n\t" MF                                                   \
               : MOE_ACC_OUT                                                        \
               : [a0] "v"(ya0), [a1] "v"(ya1), [a2] "v"(ya2), [a3] "v"(ya3),         \
                 [b0] "v"(yb0), [b1] "v"(yb1))

  // A wave whose 128 rows all lie past the segment end (the segment tail
  // of an expert often fills less than half of its last tile) skips its
  // LDS reads and MFMAs and only keeps the copies and barriers going.
  const bool idle = __builtin_amdgcn_readfirstlane(row_end - row0 <= 128 * wm) != 0;

  // copies of the first NSTAGE_DMA steps in flight, then wait for step 0's
#pragma unroll
  for (int s = 0; s < NSTAGE_DMA; ++s)
    if (s < nk) issue(s, s * STAGE2);
  {
    const int ahead = min(NSTAGE_DMA - 1, nk - 1);  // copy groups that may still fly
    if (ahead >= 4) wait_vmcnt<4 * PER>();
    else if (ahead == 3) wait_vmcnt<3 * PER>();
    else if (ahead == 2) wait_vmcnt<2 * PER>();
    else if (ahead == 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if (idle) {
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const int ahead = min(NSTAGE_DMA - 2, nk - 2 - kt);
      if (ahead >= 3) wait_vmcnt<3 * PER>();
      else if (ahead == 2) wait_vmcnt<2 * PER>();
      else if (ahead == 1) wait_vmcnt<PER>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + NSTAGE_DMA < nk) issue(kt + NSTAGE_DMA, (uint32_t)(kt % NSTAGE_DMA) * STAGE2);
    }
  } else {
    // fragments of half-step (0, 0) -> set x
    asm volatile(MOE_READS("0", "2048") "s_waitcnt lgkmcnt(0)"
                 : [na0] "=&v"(xa0), [na1] "=&v"(xa1), [na2] "=&v"(xa2), [na3] "=&v"(xa3),
                   [h0] "=&v"(h0), [h1] "=&v"(h1), [h2] "=&v"(h2), [h3] "=&v"(h3)
                 : [aa] "v"(a_addr[0]), [ba0] "v"(b_addr[0]), [ba1] "v"(b_addr[1])
                 : "memory");
    MOE_JOIN_B(xb0, xb1);

    // Step kt: (kt, 1) is read into set y while (kt, 0) multiplies set x;
    // then the copies of step kt+1 are waited for and the barrier certifies
    // them (and that every wave is done reading stage kt, which the copies of
    // step kt+NSTAGE_DMA then overwrite); then (kt+1, 0) is read into set x while
    // (kt, 1) multiplies set y.
    int kt = 0;
    uint32_t so = 0;  // byte offset of stage kt % NSTAGE_DMA
    for (; kt + 1 < nk; ++kt) {
      const uint32_t so1 = so + STAGE2 == NSTAGE_DMA * STAGE2 ? 0u : so + STAGE2;
      MOE_READ_MMA("8192", "10240", a_addr[1] + so, b_addr[0] + so, b_addr[1] + so, y, x);
      const int ahead = min(NSTAGE_DMA - 2, nk - 2 - kt);
      if (ahead >= 3) wait_vmcnt<3 * PER>();
      else if (ahead == 2) wait_vmcnt<2 * PER>();
      else if (ahead == 1) wait_vmcnt<PER>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + NSTAGE_DMA < nk) issue_a(kt + NSTAGE_DMA, so);
      MOE_READ_MMA("0", "2048", a_addr[0] + so1, b_addr[0] + so1, b_addr[1] + so1, x, y);
      if (kt + NSTAGE_DMA < nk) issue_b(kt + NSTAGE_DMA, so);
      so = so1;
    }
    {
      // last step: (kt, 1) into set y while (kt, 0) multiplies, then (kt, 1);
      // both blocks end with the MFMA result wait states (the compiler may
      // move accumulators after them)
      MOE_RM_ASM("8192", "10240", a_addr[1] + so, b_addr[0] + so, b_addr[1] + so, y, x,
                 MOE_MF_4 MFMA_TAIL);
      MOE_JOIN_B(yb0, yb1);
      MOE_MMA_ASM(MOE_MF_4 MFMA_TAIL);
    }
  }
  // the last MFMAs finish writing the accumulators before any VALU reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#undef MOE_MMA_ASM
#undef MOE_READ_MMA
#undef MOE_RM_ASM
#undef MOE_ACC_OUT
#undef MOE_READS
#undef MOE_MF_4
#undef MOE_JOIN_B

  // ---- split tiles: partial sums through the workspace. A slot holds the
  // 256 x 256 accumulators in register order, 16 bytes per lane per store:
  // float4 (wave, q, lane) with q = 4 (2i + j) + r/4 holds acc[i][j][r..r+3].
  if (S > 1) {
    float4* mine = reinterpret_cast<float4*>(a.split_ws) + wave * 32 * 64 + lane;
    if (part < S - 1) {
      float4* dst = mine + (size_t)(slot0 + part) * (BM2 * BN2 / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            dst[((2 * i + j) * 4 + rq) * 64] =
                make_float4(acc[i][j][4 * rq], acc[i][j][4 * rq + 1], acc[i][j][4 * rq + 2],
                            acc[i][j][4 * rq + 3]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();  // every wave's partial sums are in memory
      if (tid == 0) {
        __hip_atomic_store(a.split_flags + slot0 + part, 1, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    for (int p = 0; p < S - 1; ++p) {
      if (tid == 0) {
        // bounded wait: the part was dispatched before this workgroup and
        // never waits itself, so the flag rises within its run time
        for (int spin = 0; spin < (1 << 24); ++spin) {
          if (__hip_atomic_load(a.split_flags + slot0 + p, __ATOMIC_ACQUIRE,
                                __HIP_MEMORY_SCOPE_AGENT) != 0)
            break;
          __builtin_amdgcn_s_sleep(2);
        }
        __hip_atomic_store(a.split_flags + slot0 + p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const float4* src = mine + (size_t)(slot0 + p) * (BM2 * BN2 / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const float4 v = src[((2 * i + j) * 4 + rq) * 64];
            acc[i][j][4 * rq] += v.x;
            acc[i][j][4 * rq + 1] += v.y;
            acc[i][j][4 * rq + 2] += v.z;
            acc[i][j][4 * rq + 3] += v.w;
          }
    }
  }

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
          g = clampf(g, a.clamp);
          u = clampf(u, a.clamp);
        }
        *reinterpret_cast<uint16_t*>(wl + m * 64 + lrow * 2) =
            static_cast<uint16_t>(f32_to_bf16(silu_f32(g) * u));
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
    // wave tile: 128 rows x 64 fp32 columns, in two halves of 32 columns
    unsigned char* wl = smem + wave * (128 * 128);
    float* Y = static_cast<float*>(a.out);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * i + 8 * (r >> 2) + 4 * lq + (r & 3);
          *reinterpret_cast<float*>(wl + m * 128 + lrow * 4) = acc[i][j][r];
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int idx = it * 64 + lane, m = idx >> 3, ch = idx & 7;
        const int grow = row0 + 128 * wm + m, n = n0 + bcol[j] + 4 * ch;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wl + m * 128 + ch * 16);
        if (grow < row_end && n < N) *reinterpret_cast<u32x4_t*>(Y + (size_t)grow * N + n) = v;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next half overwrites
    }
  }
}

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
  if (p.mxfp4)
    a.n_tiles_n = mode == MODE_SWIGLU ? ceil_div(p.N, 256) : ceil_div(p.N, 512);
  else
    a.n_tiles_n = mode == MODE_SWIGLU ? ceil_div(p.N, 128) : ceil_div(p.N, 256);
  const long long total = (long long)a.max_tiles * a.n_tiles_n;
  a.per_xcd = ceil_div(total, 8);
  a.split_ws = p.split_ws;
  a.split_flags = p.split_flags;
  a.B0 = p.B0;
  a.B1 = p.B1;
  a.S0 = p.S0;
  a.S1 = p.S1;
  a.clamp = p.clamp;
  a.out = p.out;
  const dim3 grid(8 * a.per_xcd);
  // bf16: an XCD's share of the tiles plus the split parts of its last round
  const dim3 grid_bf16(8 * (a.per_xcd + kCUsPerXCD));
  if (mode == MODE_SWIGLU) {
    if (p.mxfp4) gemm_kernel<MODE_SWIGLU, true><<<grid, 256, 0, s>>>(a);
    else gemm_bf16_kernel<MODE_SWIGLU><<<grid_bf16, 512, 0, s>>>(a);
  } else {
    if (p.mxfp4) gemm_kernel<MODE_DOWN, true><<<grid, 256, 0, s>>>(a);
    else gemm_bf16_kernel<MODE_DOWN><<<grid_bf16, 512, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_swiglu(const GemmProblem& p, hipStream_t s) { return launch_gemm(p, MODE_SWIGLU, s); }
hipError_t launch_gemm_down(const GemmProblem& p, hipStream_t s) { return launch_gemm(p, MODE_DOWN, s); }

}  // namespace moe

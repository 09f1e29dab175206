// Tile schedule, operand-copy helpers and the split-tile exchange shared by
// the grouped GEMM kernels (gemm16.hip: bf16 activations; gemm_a8.hip: MXFP8
// activations with MXFP4 weights). All compute 256 x 256 tiles with 8
// waves; they differ in the k covered per step, the MFMA shape and the
// operand formats. The kernel with MXFP4 weights and bf16 activations also
// runs wide tiles of 128 rows x 512 B-columns for the last M-tile of an
// expert when it holds at most 128 rows: every wave then has a full 128 x
// 64 block of work, where a 256-row tile would leave half the waves idle.
#pragma once

#include "common.h"
#include "launch.h"

// The bf16 kernel's asm blocks that issue LDS copies set M0 themselves and
// list it as clobbered; clang warns about clobbering a reserved register.
#pragma clang diagnostic ignored "-Winline-asm"

// Wait states after an asm block's last MFMA so that whatever the compiler
// places next (a register move, a spill, a VALU read) sees the finished
// accumulator: the compiler does not look inside asm for MFMA hazards.
#define MFMA_TAIL "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"

namespace moe {
namespace {

constexpr int TM = kBM;                 // 256 rows per tile
constexpr int TN = 256;                 // B-columns per tile
constexpr int TMW = 128;                // wide tiles: rows
constexpr int TNW = 512;                // wide tiles: B-columns
constexpr int kCUsPerXCD = 32;          // MI355X: 256 CUs in 8 XCDs
constexpr int kMaxSplit = 8;            // K-parts of a split tile
constexpr int kMinPartK = 1024;         // shortest K range of a split part

enum { MODE_SWIGLU = 0, MODE_DOWN = 1 };

struct Args {
  const void* A;          // bf16 rows, or MXFP8 codes (MXFP8 A)
  const uint8_t* SA;      // MXFP8 A: e8m0 scales, grouped [ceil(K/512)][A rows][16]
  const int32_t* gather;  // A row of tile row r: gather[r] (< gather_rows), or r when nullptr
  int gather_rows;
  const int32_t* tilemap;
  const int32_t* offsets;
  int rows, max_tiles, K, N, n_tiles_n;
  int n_tiles_w;          // N-tiles of a wide tile row (the tile map lists wide tiles)
  const void* B0;
  const void* B1;
  const uint8_t* S0;
  const uint8_t* S1;
  float clamp;
  void* out;
  float* split_ws;       // partial accumulators of split tiles, or nullptr
  int32_t* split_flags;  // one ready flag per partial slot, zero before the launch
  int split_wait;        // polls of a ready flag before a split tile gives up
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Slot permutation of the 4 k-groups of a 64-byte A row: rows r..r+15 then
// put any one k-group in 16 distinct 16-byte bank groups, and so do rows
// r..r+3 with all 4 k-groups.
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(p);
}
// Asynchronous copies global -> LDS: lane l's 16 bytes land at
// lds_base + 16 l (dma16); lane l's byte lands, zero-extended to a dword,
// at lds_base + 4 l (dma1).
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma1(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_base, 1, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most `groups` steps of this thread's copies are in flight
template <int PER>
__device__ __forceinline__ void wait_copy_groups(int groups) {
  switch (groups) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER>(); break;
    case 2: wait_vmcnt<2 * PER>(); break;
    case 3: wait_vmcnt<3 * PER>(); break;
    case 4: wait_vmcnt<4 * PER>(); break;
    case 5: wait_vmcnt<5 * PER>(); break;
    default: wait_vmcnt<6 * PER>(); break;
  }
}

// Tile map (tilemap_kernel): [0] = regular M-tiles MR, [1] = wide M-tiles
// MW (-1: wide tiles off, every M-tile regular), then the (expert, first
// row) of the MR regular M-tiles in expert order and of the MW wide ones.
// With wide tiles on, an expert of r rows has r / 256 full M-tiles, its
// remainder r % 256 (if any) is one more regular M-tile above 128 rows and
// a wide M-tile otherwise.
__device__ __forceinline__ int regular_mtiles(int rows, bool wide_on) {
  const int rem = rows % TM;
  return rows / TM + (rem > (wide_on ? TMW : 0) ? 1 : 0);
}

// Regular tile order, by expert: an expert's tiles are contiguous, in groups of up
// to 16 of its M-tiles; inside a group N-tile major and M-tile minor. The 32
// workgroups an XCD runs at once then cover all M-tiles of one expert (up
// to 16) for a few N-tiles, so each weight slab is fetched once and shared
// by all those M-tiles, and each activation slab by the N-tiles. (Groups of
// 8 M-tiles were 1 % slower on the 8-expert layer, groups of 2 10 %.) With a tile map, M-tile
// t / NT and the tile's own belong to the same expert (an expert's tiles
// span whole rows of NT), which gives the expert's first M-tile and count
// without a search.
__device__ __forceinline__ void expert_tile_of(int t, int MT, int NT, const int32_t* tilemap,
                                               const int32_t* offsets, int& mt, int& nt) {
  constexpr int MG = 16;
  int first = 0, m = MT;
  if (tilemap) {
    const int g = t / NT;
    const int e = tilemap[2 + 2 * g];
    const int seg = offsets[e];
    first = g - (tilemap[3 + 2 * g] - seg) / TM;
    m = regular_mtiles(offsets[e + 1] - seg, tilemap[1] >= 0);
  }
  const int r = t - first * NT;
  const int gi = r / (MG * NT);
  const int gsz = min(MG, m - gi * MG);
  const int rr = r - gi * MG * NT;
  nt = rr / gsz;
  mt = first + gi * MG + rr % gsz;
}

// Workgroup -> (tile, k-range). The regular tiles, in expert_tile_of
// order, and the wide ones (wide M-tile major, N-tile minor) are each cut
// into 8 contiguous ranges, one per XCD; an XCD runs its regular range,
// then its wide range (every XCD gets its share of the wide tiles).
// Workgroup b runs on XCD b mod 8 as that
// XCD's (b / 8)-th workgroup. An XCD's whole rounds of kCUsPerXCD tiles run
// as whole tiles; each tile of its last, partial round is split along K
// into S parts (S x remainder <= kCUsPerXCD, each part at least kMinPartK
// deep: with K = 1024 on the 384-expert layer, 8 parts of 128 made the
// down GEMM 7 % slower than no split, while 4 parts of 3584 make the
// 8-expert down GEMM 8 % faster). Parts 0..S-2 leave fp32
// partial sums in a workspace slot and raise its flag; part S-1 (the
// highest workgroup index of the tile, so the parts it waits for were
// dispatched before it) adds them in part order and runs the epilogue.
struct Job {
  int e, row0, row_end, nt, S, part, slot0, kt_begin, nk;
  bool wide;
};
template <int BK>
__device__ __forceinline__ bool schedule_tile(const Args& a, int b, Job& j) {
  const int xcd = b & 7, wi = b >> 3;
  const int MT = a.tilemap ? a.tilemap[0] : a.max_tiles;
  const int MW = a.tilemap ? max(a.tilemap[1], 0) : 0;
  const int total_reg = MT * a.n_tiles_n, total_w = MW * a.n_tiles_w;
  const int r_lo = (int)((long long)total_reg * xcd / 8);
  const int r_n = (int)((long long)total_reg * (xcd + 1) / 8) - r_lo;
  const int w_lo = (int)((long long)total_w * xcd / 8);
  const int n = r_n + (int)((long long)total_w * (xcd + 1) / 8) - w_lo;
  const int whole = n / kCUsPerXCD * kCUsPerXCD;
  const int rem = n - whole;
  const int nk_all = a.K / BK;
  int li;  // the tile's place in this XCD's list
  j.S = 1;
  j.part = 0;
  j.slot0 = 0;
  if (wi < whole) {
    li = wi;
  } else {
    if (a.split_flags && rem > 0)
      j.S = max(1, min(min(kMaxSplit, kCUsPerXCD / rem), a.K / kMinPartK));
    const int u = wi - whole;
    if (u >= rem * j.S) return false;
    li = whole + u / j.S;
    j.part = u % j.S;
    j.slot0 = xcd * kCUsPerXCD + (u / j.S) * (j.S - 1);
  }
  int mt;
  j.wide = li >= r_n;
  if (j.wide) {
    const int u = w_lo + li - r_n;
    mt = MT + u / a.n_tiles_w;
    j.nt = u % a.n_tiles_w;
  } else {
    expert_tile_of(r_lo + li, MT, a.n_tiles_n, a.tilemap, a.offsets, mt, j.nt);
  }
  if (a.tilemap) {
    j.e = a.tilemap[2 + 2 * mt];
    j.row0 = a.tilemap[3 + 2 * mt];
    j.row_end = a.offsets[j.e + 1];
  } else {
    j.e = 0;
    j.row0 = mt * TM;
    j.row_end = a.rows;
  }
  j.kt_begin = j.part * nk_all / j.S;
  j.nk = (j.part + 1) * nk_all / j.S - j.kt_begin;
  return true;
}

// Split tiles: partial sums through the workspace. A slot holds a tile's
// 256 x 256 accumulators in register order: each lane's 128 accumulators as
// 32 float4, slot entry (wave, q, lane) holding float4 q of the lane (16
// bytes per lane per store). get(q) returns the lane's float4 q, add(q, v)
// adds v to it. Parts 0..S-2 store theirs, raise their flag and return
// false; part S-1 adds the others' in part order and returns true (it runs
// the epilogue).
//
// Part S-1 is the highest workgroup index of its tile, so the parts it
// waits for were dispatched before it (the dispatcher hands out workgroups
// in index order) and never wait themselves: their flags rise within their
// run time. Each wave polls a flag itself (all lanes one address, so one
// request per poll), at most a.split_wait times. A wave whose flag does not
// rise in time sets `lost` and adds nothing from that slot; the epilogue
// then stores NaN for the wave's outputs, so a broken hand-off shows up as
// NaN, never as a plausible partial sum. Flags are not reset here: the
// gate/up and down launches of one layer use separate flag banks, both
// zeroed by the tile-map kernel before the gate/up launch, so a flag that
// rises after its consumer gave up cannot mislead a later launch.
template <class Get, class Add>
__device__ __forceinline__ bool split_exchange(const Args& a, const Job& jb, Get get, Add add,
                                               int wave, int lane, int tid, bool& lost) {
  const int S = jb.S, part = jb.part, slot0 = jb.slot0;
  float4* mine = reinterpret_cast<float4*>(a.split_ws) + wave * 32 * 64 + lane;
  if (part < S - 1) {
    float4* dst = mine + (size_t)(slot0 + part) * (TM * TN / 4);
#pragma unroll
    for (int q = 0; q < 32; ++q) dst[q * 64] = get(q);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();  // every wave's partial sums are in memory
    if (tid == 0) {
      __hip_atomic_store(a.split_flags + slot0 + part, 1, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    return false;
  }
  lost = false;
  for (int p = 0; p < S - 1; ++p) {
    const int32_t* flag = a.split_flags + slot0 + p;
    bool up = false;
    for (int n = 0; n < a.split_wait; ++n) {
      if (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!up) {
      lost = true;
      continue;
    }
    const float4* src = mine + (size_t)(slot0 + p) * (TM * TN / 4);
#pragma unroll
    for (int q = 0; q < 32; ++q) add(q, src[q * 64]);
  }
  return true;
}

// split_exchange for the 32x32 accumulator layout acc[4][2] (f32x16):
// float4 q = 4 (2i + j) + r/4 holds acc[i][j][r..r+3]
__device__ __forceinline__ bool split_exchange(const Args& a, const Job& jb, f32x16_t (&acc)[4][2],
                                               int wave, int lane, int tid, bool& lost) {
  return split_exchange(
      a, jb,
      [&](int q) {
        const f32x16_t& t = acc[q >> 3][(q >> 2) & 1];
        const int r = 4 * (q & 3);
        return make_float4(t[r], t[r + 1], t[r + 2], t[r + 3]);
      },
      [&](int q, float4 v) {
        f32x16_t& t = acc[q >> 3][(q >> 2) & 1];
        const int r = 4 * (q & 3);
        t[r] += v.x;
        t[r + 1] += v.y;
        t[r + 2] += v.z;
        t[r + 3] += v.w;
      },
      wave, lane, tid, lost);
}

// Down-projection epilogue: the wave's 128 rows x 64 fp32 columns (rows
// from wrow0, B-columns n0 + bcol[j] + 0..31) go through the wave's 16 KB of
// LDS at wl, in two halves of 32 columns, so that the global stores are
// 16 bytes per lane; NaN instead when the wave lost a split part.
// Accumulator r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32 of
// its 32x32 tile.
__device__ __forceinline__ void store_down_tile(const Args& a, const f32x16_t (&acc)[4][2],
                                                unsigned char* smem, int wave, int lane, int wrow0,
                                                int row_end, int n0, const int (&bcol)[2],
                                                bool lost) {
  const int lrow = lane & 31, lq = lane >> 5, N = a.N;
  unsigned char* wl = smem + wave * (128 * 128);
  float* Y = static_cast<float*>(a.out);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * i + 8 * (r >> 2) + 4 * lq + (r & 3);
        *reinterpret_cast<float*>(wl + m * 128 + lrow * 4) =
            lost ? __builtin_nanf("") : acc[i][j][r];
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + lane, m = idx >> 3, ch = idx & 7;
      const int grow = wrow0 + m, n = n0 + bcol[j] + 4 * ch;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wl + m * 128 + ch * 16);
      if (grow < row_end && n < N) *reinterpret_cast<u32x4_t*>(Y + (size_t)grow * N + n) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next half overwrites
  }
}

}  // namespace
}  // namespace moe

// Internal launchers of libmoe (host side). Each enqueues kernels on the
// given stream and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Rows per M-tile of the grouped GEMMs (both projections, bf16 and MXFP4
// weights).
constexpr int kBM = 256;
// Tokens per dispatch chunk (one workgroup of the count and rank kernels).
constexpr int kChunk = 256;

inline int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Upper bound of the number of M-tiles: every kept row in a full tile plus
// one partial tile per expert.
inline int max_mtiles(const moe_cfg& c) { return ceil_div((long long)c.T * c.top_k, kBM) + c.E; }
// int32 entries of the tile map: [0] = regular M-tiles, [1] = wide M-tiles
// (-1: off), then (expert, row0) pairs of the regular, then the wide M-tiles.
inline size_t tilemap_ints(const moe_cfg& c) { return 2 + 2 * (size_t)max_mtiles(c); }
// The grouped GEMMs split the tiles of their last round along K: one slot
// of 256 x 256 fp32 partial sums per split part (at most 32 per XCD), and
// one ready flag per slot in each of two banks (gate/up, then down), both
// zeroed by the tile-map kernel.
constexpr int kSplitSlots = 256;
constexpr size_t kSplitSlotBytes = 256 * 256 * 4;
constexpr size_t kSplitFlagBytes = 2 * kSplitSlots * 4;
// Default polls of a split part's ready flag before its consumer gives up
// (each poll sleeps about 128 cycles: about a second in all).
constexpr int kSplitWaitDefault = 1 << 24;
inline bool gemm_splits(const moe_cfg& c) { return c.act_dtype == MOE_BF16; }
inline size_t split_bytes(const moe_cfg& c) {
  return gemm_splits(c) ? kSplitFlagBytes + kSplitSlots * kSplitSlotBytes : 0;
}
inline int num_chunks(const moe_cfg& c) { return ceil_div(c.T, kChunk); }

hipError_t launch_router(const moe_cfg& c, const void* x, const float* W_r, const float* bias,
                         int32_t* idx, float* w, float* logits, hipStream_t s);

// int32 entries of the fixed device scratch of moe_dispatch_noalloc (1 MiB)
constexpr size_t kDispatchScratchInts = 1 << 18;
// Device address of the current device's dispatch scratch (resolved on the
// first call on each device).
hipError_t dispatch_scratch(int32_t** out);

// Screened router (route_fast.hip): MFMA estimates of the logits with a
// rigorous error bound pick each token's candidate experts, and only their
// exact fp32 chains are run; the indices and weights equal the exact
// router's. Applies with bf16 activations, at least kScreenMinE experts and
// any gating except softmax without renormalisation (whose weights need
// every expert's exact logit). At 128 experts (8192 tokens, k = 8) it takes
// 0.20 ms against the exact router's 0.25 ms.
constexpr int kScreenMinE = 128;
bool router_screen_applies(const moe_cfg& c);
size_t router_screen_ws_bytes(const moe_cfg& c);
hipError_t launch_router_screened(const moe_cfg& c, const void* x, const float* W_r,
                                  const float* bias, int32_t* idx, float* w, void* ws,
                                  hipStream_t s);

// chunk_ws: int32 [E][num_chunks]
hipError_t launch_dispatch(const moe_cfg& c, const int32_t* idx, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* slot_pos, int32_t* perm, void* x_perm,
                           int32_t* chunk_ws, hipStream_t s);

// Builds the tile map (tilemap_ints(c) int32, M-tiles of kBM rows; with
// `wide`, an expert's last M-tile of at most kBM / 2 rows becomes a wide
// tile of 128 rows x 512 B-columns, which the MXFP4-weight GEMMs, with bf16
// or MXFP8 activations, run)
// from device offsets; also zeroes both banks of split flags
// (2 kSplitSlots int32) when `flags` is not null.
hipError_t launch_tilemap(const moe_cfg& c, const int32_t* offsets, int32_t* tilemap,
                          int32_t* flags, bool wide, hipStream_t s);

// bf16 activations: grouped MFMA GEMMs over the tile map. A dense launch
// (tilemap == nullptr) treats rows [0, rows) as one segment of expert 0.
struct GemmProblem {
  const void* A;           // [rows][K] bf16 (MXFP8: e4m3 codes), or [gather_rows][K] when gathered
  const uint8_t* SA;       // MXFP8 A only: e8m0 scales, grouped [ceil(K/512)][A rows][16]
  const int32_t* gather;   // nullptr, or the A row of each routed row (perm_token)
  int gather_rows;
  const int32_t* tilemap;  // nullptr: dense
  const int32_t* offsets;  // segment ends (offsets[e+1]); unused when dense
  int rows;                // dense row count / grid bound
  int max_tiles;           // M-tiles in the grid
  int K, N;
  int E;
  const void* B0;          // gate (SwiGLU) or down; [E][K][N] bf16 or MXFP4 codes [E][K/32][N][16]
  const void* B1;          // up (SwiGLU), else nullptr
  const uint8_t* S0;       // MXFP4 scales [E][K/32][N]
  const uint8_t* S1;
  int mxfp4;
  float clamp;
  void* out;               // SwiGLU: H bf16 [rows][N] (MXFP8 A: codes [rows][N] then
                           // grouped scales [ceil(N/512)][rows][16]); down: fp32 [rows][N]
  float* split_ws;         // kSplitSlots partial-sum slots, or nullptr: no split
  int32_t* split_flags;    // kSplitSlots flags, zero before the launch
  int split_wait;          // polls of a flag before a split tile stores NaN
};
hipError_t launch_gemm_swiglu(const GemmProblem& p, hipStream_t s);
hipError_t launch_gemm_down(const GemmProblem& p, hipStream_t s);

// MXFP4 weights with MXFP8 activations: rows of bf16 -> MXFP8 (codes
// [rows][K], scales [rows][K/32]), and the grouped GEMM on the scaled MFMA
// (gemm_a8.hip).
// (grouped: scales [ceil(K/512)][rows][16], the layout the GEMM reads; else [rows][K/32])
hipError_t launch_quant_mxfp8(const void* x, long long rows, int K, uint8_t* codes, uint8_t* scales,
                              bool grouped, hipStream_t s);
hipError_t launch_gemm_a8(const GemmProblem& p, bool swiglu, hipStream_t s);

// fp32 activations and weights: the grouped GEMM on the fp32 MFMA.
hipError_t launch_ffn_f32_gate_up(const moe_cfg& c, const float* x_perm, const int32_t* offsets,
                                  const float* Wg, const float* Wu, float* H, hipStream_t s);
hipError_t launch_ffn_f32_down(const moe_cfg& c, const float* H, const int32_t* offsets,
                               const float* Wd, float* y_perm, hipStream_t s);

hipError_t launch_combine(const moe_cfg& c, const float* y_perm, const int32_t* slot_pos,
                          const float* topk_w, const float* y_shared, void* y, hipStream_t s);

}  // namespace moe

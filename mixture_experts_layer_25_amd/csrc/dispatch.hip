// Dispatch: group (token, slot) pairs by expert in token order, apply the
// capacity, and copy each kept pair's x row into its expert's segment.
//
// "moe f&b compute flow" (Echo's blog), Dispatch: tokens go to the input
// buffer of the experts the router picked. "ops-transformer MoE operator on
// Ascend NPU": MoEForward step 3 gathers each expert's tokens; pitfall 1
// caps each expert at `capacity` tokens and drops the overflow.
//
// The rank of pair (t, j) routed to e is the number of pairs before it in
// (token, slot) order that are routed to e, so segments keep token order and
// the drops are the latest tokens. Four launches, all integer work except
// the row copy, all deterministic:
//   count: per 256-token chunk, per-expert histogram (LDS integer atomics;
//          counts do not depend on their order) -> chunk_ws[e][chunk];
//   scan:  one wave per expert, exclusive scan over chunks -> the chunk's
//          base rank, and the expert's total count;
//   rank:  per chunk, kept counts -> offsets (every workgroup rescans the
//          E counts; E <= 1024), then each pair's rank = chunk base + earlier
//          waves' counts + earlier pairs in the wave (per-expert lane masks
//          in LDS) -> slot_pos, perm_token;
//   copy:  one wave per token reads the row once (16-byte vectors) and
//          writes it to each kept slot. With MXFP8 activation operands
//          (MOE_MXFP4_A8) the wave quantises the row once instead and writes
//          the codes to each kept slot's row, the scales in the grouped
//          layout of the A8 GEMM after the codes.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "mxfp8.h"

namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, int T,
                                                             int E, int k, int nchunks,
                                                             int32_t* __restrict__ chunk_ws) {
  __shared__ int hist[kMaxE];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t = chunk * kChunk + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_ws[(size_t)e * nchunks + chunk] = hist[e];
}

__global__ __launch_bounds__(256) void dispatch_scan_kernel(int E, int nchunks,
                                                            int32_t* __restrict__ chunk_ws,
                                                            int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int32_t* row = chunk_ws + (size_t)e * nchunks;
  int running = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < nchunks ? row[c] : 0;
    const int incl = wave_inclusive_scan(v);
    if (c < nchunks) row[c] = running + incl - v;
    running += __shfl(incl, 63, 64);
  }
  if (lane == 0) counts[e] = running;
}

__global__ __launch_bounds__(256) void dispatch_rank_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ chunk_ws, int T, int E, int k, int capacity, int nchunks,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_pos, int32_t* __restrict__ perm) {
  __shared__ int off_sh[kMaxE + 1];
  __shared__ int wh[4][kMaxE];
  __shared__ int wave_tot[4];
  __shared__ int ev_sh[256][kMaxK + 1];
  __shared__ unsigned long long lanes_of[4][kMaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = blockIdx.x;

  // kept counts -> exclusive scan over experts (4 experts per thread)
  int kept[4];
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    int c = e < E ? counts[e] : 0;
    if (capacity > 0 && c > capacity) c = capacity;
    kept[q] = c;
    local += c;
  }
  const int incl = wave_inclusive_scan(local);
  if (lane == 63) wave_tot[wave] = incl;
  for (int e = tid; e < E; e += 256) {
    wh[0][e] = 0;
    wh[1][e] = 0;
    wh[2][e] = 0;
    wh[3][e] = 0;
    lanes_of[0][e] = 0ull;
    lanes_of[1][e] = 0ull;
    lanes_of[2][e] = 0ull;
    lanes_of[3][e] = 0ull;
  }
  __syncthreads();
  int base = incl - local;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < E) off_sh[e] = base;
    base += kept[q];
  }
  if (tid == 255) off_sh[E] = base;  // total kept (thread 255 covers e >= E - 1)

  // this token's pairs (e = -1: none) and the per-wave histograms
  const int t = chunk * kChunk + tid;
  const bool valid_t = t < T;
  int ev[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    int e = -1;
    if (j < k && valid_t) {
      e = idx[(size_t)t * k + j];
      if (e < 0 || e >= E) e = -1;
    }
    ev[j] = e;
    ev_sh[tid][j] = e;
    if (e >= 0) atomicAdd(&wh[wave][e], 1);
  }
  __syncthreads();
  if (chunk == 0) {
    for (int e = tid; e <= E; e += 256) offsets[e] = off_sh[e];
  }

  // Pairs of earlier tokens of this wave with the same expert, column by
  // column: every lane sets its bit in the mask of its column-jj expert,
  // then each pair counts the set bits of lanes below it in the mask of its
  // own expert, and the lanes clear what they set. (A wave's LDS
  // instructions run in program order.)
  const uint64_t below = (1ull << lane) - 1ull;
  int r[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) r[j] = 0;
  for (int jj = 0; jj < k; ++jj) {
    const int col = ev_sh[tid][jj];
    if (col >= 0)
      __hip_atomic_fetch_or(reinterpret_cast<unsigned*>(&lanes_of[wave][col]) + (lane >> 5),
                            1u << (lane & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k && ev[j] >= 0) r[j] += __popcll(lanes_of[wave][ev[j]] & below);
    if (col >= 0) lanes_of[wave][col] = 0ull;
  }
  if (!valid_t) return;

#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= k) continue;
    const int e = ev[j];
    int slot = -1;
    if (e >= 0) {
      int rank = chunk_ws[(size_t)e * nchunks + chunk] + r[j];
      for (int w = 0; w < wave; ++w) rank += wh[w][e];
      // earlier slots of this token
#pragma unroll
      for (int jj = 0; jj < kMaxK; ++jj)
        if (jj < j) rank += (ev[jj] == e);
      if (capacity <= 0 || rank < capacity) {
        slot = off_sh[e] + rank;
        perm[slot] = t;
      }
    }
    slot_pos[(size_t)t * k + j] = slot;
  }
}

__global__ __launch_bounds__(256) void dispatch_copy_kernel(const uint4* __restrict__ x,
                                                            const int32_t* __restrict__ slot_pos,
                                                            int T, int k, int nvec,
                                                            uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int pos[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) pos[j] = j < k ? slot_pos[(size_t)t * k + j] : -1;
  const uint4* src = x + (size_t)t * nvec;
  for (int v = lane; v < nvec; v += 64) {
    const uint4 val = src[v];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (pos[j] >= 0) x_perm[(size_t)pos[j] * nvec + v] = val;
  }
}

__global__ __launch_bounds__(256) void dispatch_copy_mxfp8_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ slot_pos, int T, int k, int D,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int pos[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) pos[j] = j < k ? slot_pos[(size_t)t * k + j] : -1;
  const long long rows = (long long)T * k;
  const int KB = D / 32;
  for (int b = lane; b < KB; b += 64) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * D + 32 * b);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = src[i];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[8 * i + 2 * c] = __uint_as_float(ww[c] << 16);
        v[8 * i + 2 * c + 1] = __uint_as_float(ww[c] & 0xFFFF0000u);
      }
    }
    uint32_t q[8];
    const uint32_t s = mxfp8_block(v, q);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (pos[j] < 0) continue;
      uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)pos[j] * D + 32 * b);
      dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
      dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
      scales[grouped_scale(pos[j], b, rows)] = (uint8_t)s;
    }
  }
}

// T = 0: no pair to dispatch; the counts and offsets of the empty layer
// (a kernel, not a memset, so that the call stays capturable into a graph)
__global__ __launch_bounds__(256) void dispatch_empty_kernel(int E, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets) {
  for (int e = blockIdx.x * 256 + threadIdx.x; e <= E; e += gridDim.x * 256) {
    if (counts && e < E) counts[e] = 0;
    if (offsets) offsets[e] = 0;
  }
}

}  // namespace

hipError_t launch_dispatch_empty(const moe_cfg& c, int32_t* counts, int32_t* offsets,
                                 hipStream_t s) {
  if (!counts && !offsets) return hipSuccess;
  dispatch_empty_kernel<<<ceil_div(c.E + 1, 256), 256, 0, s>>>(c.E, counts, offsets);
  return hipGetLastError();
}

// Scratch of the no-allocation dispatch (moe_dispatch_noalloc): the
// per-chunk expert counts, int32 [E][ceil(T/256)], at most
// kDispatchScratchInts. The count kernel writes every entry it uses, so
// nothing needs clearing between calls. Every call on a device shares that
// device's copy; calls that overlap on one device race.
static __device__ __align__(256) int32_t scratch[kDispatchScratchInts];

hipError_t dispatch_scratch(int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    // the device address of this device's copy; the host-side name of the
    // array is not a device address
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t launch_dispatch(const moe_cfg& c, const int32_t* idx, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* slot_pos, int32_t* perm, void* x_perm,
                           int32_t* chunk_ws, hipStream_t s) {
  const int nchunks = num_chunks(c);
  dispatch_count_kernel<<<nchunks, 256, 0, s>>>(idx, c.T, c.E, c.top_k, nchunks, chunk_ws);
  dispatch_scan_kernel<<<ceil_div(c.E, 4), 256, 0, s>>>(c.E, nchunks, chunk_ws, counts);
  dispatch_rank_kernel<<<nchunks, 256, 0, s>>>(idx, counts, chunk_ws, c.T, c.E, c.top_k,
                                               c.capacity, nchunks, offsets, slot_pos, perm);
  if (!x_perm) return hipGetLastError();  // the caller gathers rows through perm
  if (c.w_dtype == MOE_MXFP4_A8) {
    uint8_t* q = static_cast<uint8_t*>(x_perm);
    dispatch_copy_mxfp8_kernel<<<ceil_div(c.T, 4), 256, 0, s>>>(
        static_cast<const uint16_t*>(x), slot_pos, c.T, c.top_k, c.D, q,
        q + (size_t)c.T * c.top_k * c.D);
    return hipGetLastError();
  }
  const size_t row_bytes = (size_t)c.D * (c.act_dtype == MOE_BF16 ? 2 : 4);
  dispatch_copy_kernel<<<ceil_div(c.T, 4), 256, 0, s>>>(
      static_cast<const uint4*>(x), slot_pos, c.T, c.top_k, static_cast<int>(row_bytes / 16),
      static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe

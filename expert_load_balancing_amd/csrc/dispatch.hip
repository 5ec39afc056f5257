// Counting-sort dispatch of the flat assignments j = t * K + slot by expert.
//
// The pages define no dispatch; what is computed is the plain stable counting sort:
// bucket e holds the flat positions routed to expert e in ascending order, offsets[e] is
// the bucket start, and inv is the inverse permutation.  Positions come from an
// expert-major, tile-ordered exclusive scan of per-tile histograms plus a stable rank
// inside the tile, never from the order in which atomics happen to land, so the result is
// bit-identical run to run.
//
//  1. hist:     one workgroup per tile of E entries (E chosen so there are at most 256
//               tiles): LDS histogram -> ws[e][tile].
//  2. tilescan: one wave per expert: ws[e][tile] <- sum of hist[e][tile'] for tile' < tile,
//               and the expert's total.
//  3. scatter:  one workgroup per tile.  Each block scans the 256 expert totals itself (a few
//               hundred cycles) to get the bucket starts, then walks its tile in chunks of
//               256 entries in flat order: a wave finds the lanes that hold the same expert
//               with 8 ballots (one per bit of e) and ranks them by lane; waves of a chunk are
//               ranked through LDS counters.
// Workspace: ws [n_experts][n_tiles] int32, then totals [n_experts] int32.
#include "device_common.hpp"
#include "elb_kernels.h"

namespace elb {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxExperts = 256;
constexpr int kMaxTiles = 256;

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void dispatch_hist_kernel(const int32_t* __restrict__ idx, int64_t total,
                                                                 int64_t tile_entries, int n_experts, int n_tiles,
                                                                 int32_t* __restrict__ ws) {
  __shared__ int hist[kMaxExperts];
  hist[threadIdx.x] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * tile_entries;
  const int64_t hi = lo + tile_entries < total ? lo + tile_entries : total;
  for (int64_t j = lo + threadIdx.x; j < hi; j += kThreads) {
    const int e = idx[j];
    if ((unsigned)e < (unsigned)n_experts) atomicAdd(&hist[e], 1);  // out-of-range ids are dropped
  }
  __syncthreads();
  if ((int)threadIdx.x < n_experts) ws[(int64_t)threadIdx.x * n_tiles + blockIdx.x] = hist[threadIdx.x];
}

__global__ __launch_bounds__(64) void dispatch_tilescan_kernel(int32_t* __restrict__ ws, int n_tiles,
                                                               int32_t* __restrict__ totals) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t* row = ws + (int64_t)e * n_tiles;
  int v[kMaxTiles / 64];
#pragma unroll
  for (int c = 0; c < kMaxTiles / 64; ++c) {
    const int t = c * 64 + lane;
    v[c] = t < n_tiles ? row[t] : 0;
  }
  int carry = 0;
#pragma unroll
  for (int c = 0; c < kMaxTiles / 64; ++c) {
    const int t = c * 64 + lane;
    const int incl = wave_inclusive_scan(v[c]);
    if (t < n_tiles) row[t] = carry + incl - v[c];
    carry += __shfl(incl, 63);
  }
  if (lane == 0) totals[e] = carry;
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(const int32_t* __restrict__ idx, int64_t total,
                                                                    int64_t tile_entries, int n_experts, int n_tiles,
                                                                    const int32_t* __restrict__ ws,
                                                                    const int32_t* __restrict__ totals,
                                                                    int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ perm,
                                                                    int32_t* __restrict__ inv) {
  __shared__ int base[kMaxExperts];
  __shared__ int wave_sum[kThreads / 64];
  __shared__ int wave_cnt[kThreads / 64][kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Bucket starts: exclusive scan of the expert totals, then this tile's own offset.
  const int tot = tid < n_experts ? totals[tid] : 0;
  const int incl = wave_inclusive_scan(tot);
  if (lane == 63) wave_sum[wave] = incl;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) wave_cnt[w][tid] = 0;
  __syncthreads();
  int start = incl - tot;
  for (int w = 0; w < wave; ++w) start += wave_sum[w];
  if (tid < n_experts) {
    base[tid] = start + ws[(int64_t)tid * n_tiles + blockIdx.x];
    if (blockIdx.x == 0) offsets[tid] = start;
  }
  if (blockIdx.x == 0 && tid == 0) {
    int all = 0;
    for (int w = 0; w < kThreads / 64; ++w) all += wave_sum[w];
    offsets[n_experts] = all;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t lo = (int64_t)blockIdx.x * tile_entries;
  const int64_t hi = lo + tile_entries < total ? lo + tile_entries : total;
  for (int64_t c0 = lo; c0 < hi; c0 += kThreads) {
    const int64_t j = c0 + tid;
    const int raw = j < hi ? idx[j] : -1;
    const bool valid = (unsigned)raw < (unsigned)n_experts;  // out-of-range ids are dropped
    const int e = valid ? raw : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t m = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    const int cnt = __popcll(peers);
    if (valid && rank == cnt - 1) wave_cnt[wave][e] = cnt;  // the last peer in lane order
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wave_cnt[w][e];
      perm[pos] = (int32_t)j;
      if (inv != nullptr) inv[j] = pos;
    }
    __syncthreads();
    if (tid < n_experts) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        add += wave_cnt[w][tid];
        wave_cnt[w][tid] = 0;
      }
      base[tid] += add;
    }
    __syncthreads();
  }
}

}  // namespace

int64_t dispatch_tile_entries(int64_t total) {
  // At most kMaxTiles tiles, never fewer than 1024 entries per tile.
  int64_t t = 1024;
  while (t * kMaxTiles < total) t <<= 1;
  return t;
}

size_t dispatch_workspace_bytes(int64_t total, int n_experts) {
  if (total <= 0) return 0;
  const int64_t te = dispatch_tile_entries(total);
  const int64_t n_tiles = (total + te - 1) / te;
  return (size_t)(n_tiles * n_experts + n_experts) * sizeof(int32_t);
}

hipError_t launch_dispatch(const int32_t* idx, int64_t total, int n_experts, void* workspace, int32_t* offsets,
                           int32_t* perm, int32_t* inv, hipStream_t stream) {
  if (total == 0) return launch_fill_i32(offsets, n_experts + 1, 0, stream);
  const int64_t te = dispatch_tile_entries(total);
  const int n_tiles = (int)((total + te - 1) / te);
  int32_t* ws = static_cast<int32_t*>(workspace);
  int32_t* totals = ws + (int64_t)n_tiles * n_experts;
  hipError_t err = launch(dispatch_hist_kernel, dim3(n_tiles), dim3(kThreads), 0, stream, idx, total, te,
                          n_experts, n_tiles, ws);
  if (err != hipSuccess) return err;
  err = launch(dispatch_tilescan_kernel, dim3(n_experts), dim3(64), 0, stream, ws, n_tiles, totals);
  if (err != hipSuccess) return err;
  return launch(dispatch_scatter_kernel, dim3(n_tiles), dim3(kThreads), 0, stream, idx, total, te, n_experts,
                n_tiles, (const int32_t*)ws, (const int32_t*)totals, offsets, perm, inv);
}

}  // namespace elb

// Counting-sort dispatch of the flat assignments j = t * K + slot by expert.
//
// The pages define no dispatch; what is computed is the plain stable counting sort:
// bucket e holds the flat positions routed to expert e in ascending order, offsets[e] is
// the bucket start, and inv is the inverse permutation.  Positions come from an
// expert-major, tile-ordered exclusive scan of per-tile loads plus a stable rank inside the
// tile, never from the order in which atomics happen to land, so the result is
// bit-identical run to run.
//
// A tile is 256 tokens, all K slots of each: 256 K consecutive flat entries.  Workspace:
//   loads  [n_experts][stride] int32: entries of tile b routed to expert e, then (after the
//          scan) the number of such entries in tiles before b;
//   totals [n_experts] int32.
//  1. loads:   one workgroup per tile, LDS histogram.  Skipped when the MFMA router kernel
//              already stored its own tile histogram in the table.
//  2. scan:    one wave per expert scans its row in place and writes the expert's total (and,
//              in a routed step, adds it into the step's expert loads: the router kernel then
//              leaves `counts` alone, which spares 256 contended global atomics per tile).
//  3. scatter: one workgroup per tile, one pass.  With a bias update requested, one more
//              workgroup runs it (balance_wave.hpp): the update reads only `counts`, which are
//              final once the router kernel is done, and its few microseconds of dependent
//              memory round trips hide behind the scatter's (the scan is shorter).  Each block scans the expert totals itself
//              (a few hundred cycles) for the bucket starts.  Entry c * 256 + tid of the tile
//              goes to thread tid; each 64-entry run ("virtual wave" v = c * 4 + wave, in
//              ascending j) ranks its lanes by expert with 8 ballots (one per bit of e), the
//              last lane of each expert stores the run's count, and one in-place scan per
//              expert over the runs turns those counts into run offsets.
#include "balance_wave.hpp"
#include "device_common.hpp"
#include "elb_kernels.h"

#include <mutex>

// The dispatch workspace of elb_router_dispatch_noalloc, for callers that cannot allocate: one
// copy per GPU, held until the process ends.  Host code never passes this name to a kernel (in
// host code it is a host-side stand-in, not the device address): dispatch_scratch() looks up
// each device's own address once, with that device current, and the launches use that.
static __device__ __align__(256) unsigned char scratch[elb::kDispatchScratchBytes];

namespace elb {
namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];  // device address of `scratch` per device ordinal, set on first use

constexpr int kThreads = kDispatchTile;  // one thread per token (per entry of a chunk)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxExperts = 256;

using i32x4 = int __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void dispatch_loads_kernel(const int32_t* __restrict__ idx, int64_t total,
                                                                  int k, int n_experts, int64_t stride,
                                                                  int32_t* __restrict__ loads) {
  __shared__ int hist[kMaxExperts];
  hist[threadIdx.x] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * kDispatchTile * k;
  const int64_t hi = lo + (int64_t)kDispatchTile * k < total ? lo + (int64_t)kDispatchTile * k : total;
  for (int64_t j = lo + threadIdx.x; j < hi; j += kThreads) {
    const int e = idx[j];
    if ((unsigned)e < (unsigned)n_experts) atomicAdd(&hist[e], 1);  // out-of-range ids are dropped
  }
  __syncthreads();
  if ((int)threadIdx.x < n_experts) loads[(int64_t)threadIdx.x * stride + blockIdx.x] = hist[threadIdx.x];
}

// Block e < n_experts scans row e.
__global__ __launch_bounds__(64) void dispatch_scan_kernel(int32_t* __restrict__ loads, int64_t n_tiles,
                                                           int64_t stride, int n_experts,
                                                           int32_t* __restrict__ totals,
                                                           int32_t* __restrict__ counts, int accumulate) {
  const int lane = threadIdx.x;
  int32_t* const row = loads + (int64_t)blockIdx.x * stride;
  int carry = 0;
  for (int64_t c0 = 0; c0 < n_tiles; c0 += 256) {
    const int64_t t0 = c0 + 4 * lane;  // stride % 4 == 0: t0 < stride covers t0 .. t0 + 3
    i32x4 v = {0, 0, 0, 0};
    if (t0 < stride) v = *reinterpret_cast<const i32x4*>(row + t0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (t0 + q >= n_tiles) v[q] = 0;  // padding columns hold stale workspace
    const int local = v[0] + v[1] + v[2] + v[3];
    const int incl = wave_inclusive_scan(local);
    const int excl = carry + incl - local;
    if (t0 < stride)
      *reinterpret_cast<i32x4*>(row + t0) = i32x4{excl, excl + v[0], excl + v[0] + v[1], excl + v[0] + v[1] + v[2]};
    carry += __shfl(incl, 63);
  }
  if (lane == 0) {
    totals[blockIdx.x] = carry;
    if (counts != nullptr) counts[blockIdx.x] = (accumulate ? counts[blockIdx.x] : 0) + carry;
  }
}

template <int K>
__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(const int32_t* __restrict__ idx, int64_t total,
                                                                    int n_experts, int64_t stride,
                                                                    const int32_t* __restrict__ loads,
                                                                    const int32_t* __restrict__ totals,
                                                                    int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ perm,
                                                                    int32_t* __restrict__ inv, BalanceArgs update) {
  if ((int64_t)blockIdx.x == (total + kDispatchTile * K - 1) / (kDispatchTile * K)) {
    // The block after the last tile (launched only with an update): the bias update, one wave.
    if (threadIdx.x < 64) balance_wave(update);
    return;
  }
  __shared__ int wsum[kWaves];
  __shared__ int vcnt[K * kWaves][kMaxExperts];  // per virtual wave: count, then start
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t lo = (int64_t)blockIdx.x * (kDispatchTile * K);

  int e[K];
#pragma unroll
  for (int c = 0; c < K; ++c) {
    const int64_t j = lo + c * kThreads + tid;
    const int raw = j < total ? idx[j] : -1;
    e[c] = (unsigned)raw < (unsigned)n_experts ? raw : -1;  // out-of-range ids are dropped
  }
  const int tot = tid < n_experts ? totals[tid] : 0;
  const int before = tid < n_experts ? loads[(int64_t)tid * stride + blockIdx.x] : 0;
#pragma unroll
  for (int v = 0; v < K * kWaves; ++v) vcnt[v][tid] = 0;

  // Bucket start of expert tid: exclusive scan of the totals.
  const int incl = wave_inclusive_scan(tot);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int start = incl - tot;
  for (int w = 0; w < wave; ++w) start += wsum[w];
  if (blockIdx.x == 0) {
    if (tid < n_experts) offsets[tid] = start;
    if (tid == 0) offsets[n_experts] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }

  // Rank inside each 64-entry run: lanes below with the same expert.
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int rank[K];
#pragma unroll
  for (int c = 0; c < K; ++c) {
    const bool valid = e[c] >= 0;
    const int key = valid ? e[c] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t m = __ballot((key >> b) & 1);
      peers &= ((key >> b) & 1) ? m : ~m;
    }
    rank[c] = __popcll(peers & lt_mask);
    const int cnt = __popcll(peers);
    if (valid && rank[c] == cnt - 1) vcnt[c * kWaves + wave][key] = cnt;  // the last peer in lane order
  }
  __syncthreads();
  // Run offsets of expert tid: its bucket start, plus earlier tiles, plus earlier runs.
  if (tid < n_experts) {
    int run = start + before;
#pragma unroll
    for (int v = 0; v < K * kWaves; ++v) {
      const int x = vcnt[v][tid];
      vcnt[v][tid] = run;
      run += x;
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < K; ++c) {
    if (e[c] >= 0) {
      const int64_t j = lo + c * kThreads + tid;
      const int pos = vcnt[c * kWaves + wave][e[c]] + rank[c];
      perm[pos] = (int32_t)j;
      if (inv != nullptr) inv[j] = pos;
    }
  }
}

template <int K>
hipError_t launch_scatter(const int32_t* idx, int64_t total, int n_experts, const DispatchGeom& g,
                          const int32_t* loads, const int32_t* totals, int32_t* offsets, int32_t* perm, int32_t* inv,
                          const BalanceArgs* update, hipStream_t stream, hipEvent_t ev_stop) {
  const BalanceArgs none{};
  return launch_timed(dispatch_scatter_kernel<K>, dim3((unsigned)(g.n_tiles + (update != nullptr ? 1 : 0))),
                      dim3(kThreads), 0, stream, nullptr, ev_stop, idx, total, n_experts, g.stride, loads, totals,
                      offsets, perm, inv, update != nullptr ? *update : none);
}

}  // namespace

hipError_t dispatch_scratch(hipStream_t stream, void** ptr) {
  hipDevice_t dev = 0;
  hipError_t err = hipStreamGetDevice(stream, &dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    int cur = 0;
    if ((err = hipGetDevice(&cur)) != hipSuccess) return err;
    if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_addr[dev] = p;
  }
  *ptr = scratch_addr[dev];
  return hipSuccess;
}

DispatchGeom dispatch_geometry(int64_t T) {
  DispatchGeom g;
  g.n_tiles = (T + kDispatchTile - 1) / kDispatchTile;
  g.stride = (g.n_tiles + 3) / 4 * 4;
  return g;
}

size_t dispatch_workspace_bytes(int64_t T, int n_experts) {
  if (T <= 0) return 0;
  const DispatchGeom g = dispatch_geometry(T);
  return (size_t)(g.stride * n_experts + n_experts) * sizeof(int32_t);
}

hipError_t launch_dispatch(const int32_t* idx, int64_t T, int k, int n_experts, void* workspace, bool loads_ready,
                           int32_t* counts, bool accumulate, const BalanceArgs* update, int32_t* offsets,
                           int32_t* perm, int32_t* inv, hipStream_t stream, hipEvent_t ev_stop) {
  if (T == 0) {
    hipError_t err = launch_fill_i32(offsets, n_experts + 1, 0, stream);
    if (err == hipSuccess && counts != nullptr && !accumulate) err = launch_fill_i32(counts, n_experts, 0, stream);
    if (err != hipSuccess) return err;
    if (update != nullptr) return launch_balance(*update, stream, ev_stop);
    return ev_stop != nullptr ? launch_mark(ev_stop, stream) : hipSuccess;
  }
  const DispatchGeom g = dispatch_geometry(T);
  const int64_t total = T * k;
  int32_t* loads = static_cast<int32_t*>(workspace);
  int32_t* totals = loads + g.stride * n_experts;
  hipError_t err = hipSuccess;
  if (!loads_ready) {
    err = launch(dispatch_loads_kernel, dim3((unsigned)g.n_tiles), dim3(kThreads), 0, stream, idx, total, k,
                 n_experts, g.stride, loads);
    if (err != hipSuccess) return err;
  }
  err = launch(dispatch_scan_kernel, dim3((unsigned)n_experts), dim3(64), 0, stream, loads, g.n_tiles, g.stride,
               n_experts, totals, counts, accumulate ? 1 : 0);
  if (err != hipSuccess) return err;
  const int32_t* cl = loads;
  const int32_t* ct = totals;
  switch (k) {
    case 1: return launch_scatter<1>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
    case 2: return launch_scatter<2>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
    case 3: return launch_scatter<3>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
    case 4: return launch_scatter<4>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
    case 5: return launch_scatter<5>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
    case 6: return launch_scatter<6>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
    case 7: return launch_scatter<7>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
    default: return launch_scatter<8>(idx, total, n_experts, g, cl, ct, offsets, perm, inv, update, stream, ev_stop);
  }
}

}  // namespace elb

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
//          scan) kScanned | the number of such entries in tiles before b;
//   totals [n_experts] int32: kScanned | the expert's total once scanned, reset to 0 by
//          whichever kernel fills the table.
//  1. loads: one workgroup per tile, LDS histogram.  Skipped when the MFMA router kernel
//     already stored its own tile histogram in the table (and reset the totals).
//  2. one launch with three kinds of workgroup, in this block order:
//     scan    block e < n_experts scans row e in place and writes the expert's total (and, in a
//             routed step without an update, sets or adds it into the step's expert loads: the
//             router kernel then leaves `counts` alone, which spares 256 contended global
//             atomics per tile).  Every scanned entry and total carries the flag bit kScanned
//             (all of them are below 2^31), so each one shows by itself whether it is final;
//     update  with a bias update requested, one block: its wave polls the totals the same way
//             as the scatter blocks below, forms the step's loads (adding the earlier ones with
//             ELB_ACCUMULATE_COUNTS), stores them in `counts` unless ELB_CLEAR_COUNTS zeroes them,
//             and runs the update on them (balance_wave.hpp);
//     scatter one block per tile (the tiles of each XCD contiguous).  It ranks its entries first
//             (independent of the scan): entry c * 256 + tid of the tile goes to thread tid;
//             each 64-entry run ("virtual wave" v = c * 4 + wave, in ascending j) ranks its lanes
//             by expert with 8 ballots (one per bit of e), and the last lane of each expert
//             stores the run's count.  Then each
//             thread polls just the two words it needs, its expert's total and the entry of this
//             tile, until both carry the flag (a value is published by the one store that writes
//             it: no counter, no store-completion wait).  Each block scans the expert totals
//             itself (a few hundred cycles) for the bucket starts, and one in-place scan per
//             expert over the runs turns the run counts into run offsets.
//     Only blocks after the scan blocks ever wait, and scan blocks never wait: blocks are
//     dispatched in index order, so every waited-for block has been dispatched and finishes.  The
//     wait is also bounded (about a second), so no fault elsewhere can turn it into a hang.
//     Visibility across the XCDs' separate L2 caches: the scan's results are written and read
//     with coherent accesses that go past the XCD's L2 (agent-scope atomic loads and stores, and
//     16-byte stores with the same coherence bit).
//     A count of finished rows with a release / acquire pair around it would also work, but the
//     release and acquire write back and invalidate whole L2 caches, once per block, and a
//     counter that every block polls while the scan blocks add to it holds those adds up: that
//     form made this launch slower than the separate scan kernel it replaces.
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

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (balance_wave.hpp): within each
// row of 16 by shifts of 1, 2, 4 and 8 lanes, then each row's total into the rows after it.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp::mov<dpp::kShr1>(v);
  v += dpp::mov<dpp::kShr2>(v);
  v += dpp::mov<dpp::kShr4>(v);
  v += dpp::mov<dpp::kShr8>(v);
  v += dpp::mov<dpp::kBcast15, 0xA>(v);  // rows 1 and 3 add the total of rows 0 and 2
  v += dpp::mov<dpp::kBcast31, 0xC>(v);  // rows 2 and 3 add the total of rows 0-1
  return v;
}

__global__ __launch_bounds__(kThreads) void dispatch_loads_kernel(const int32_t* __restrict__ idx, int64_t total,
                                                                  int k, int n_experts, int64_t stride,
                                                                  int32_t* __restrict__ loads) {
  __shared__ int hist[kMaxExperts];
  hist[threadIdx.x] = 0;
  // Filling the table also resets the totals the scan will flag.
  if (blockIdx.x == 0 && (int)threadIdx.x < n_experts) loads[stride * n_experts + threadIdx.x] = 0;
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

constexpr int kSpinLimit = 1 << 22;  // polls of one word, 512 cycles apart: about a second
constexpr int kScanned = int(0x80000000u);  // flag bit of a scanned table entry or total

// Scan block: row e of the loads table, in chunks of 4 entries per thread.
__device__ __forceinline__ void scan_row(int e, int32_t* __restrict__ loads, int64_t n_tiles, int64_t stride,
                                         int32_t* __restrict__ totals, int32_t* __restrict__ counts, int accumulate) {
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* const row = loads + (int64_t)e * stride;
  auto put = [](int32_t* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  // A thread's four scanned entries leave in one 16-byte store that carries the same coherence
  // bit (sc1) an agent-scope atomic store does, so whole lines are written through rather than
  // four partial ones (-0.8 us per launch at 1024 tiles); each entry carries its own flag, so a
  // reader sees each of them either stale or final.
  const __amdgpu_buffer_rsrc_t rrow =
      __builtin_amdgcn_make_buffer_rsrc(row, (short)0, (int)(stride * 4), 0x00020000);
  constexpr int kCoherent = 16;  // sc1
  int carry = 0;
  for (int64_t c0 = 0; c0 < n_tiles; c0 += 4 * kThreads) {
    const int64_t t0 = c0 + 4 * tid;  // stride % 4 == 0: t0 < stride covers t0 .. t0 + 3
    i32x4 v = {0, 0, 0, 0};
    if (t0 < stride) v = *reinterpret_cast<const i32x4*>(row + t0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (t0 + q >= n_tiles) v[q] = 0;  // padding columns hold stale workspace
    const int local = v[0] + v[1] + v[2] + v[3];
    const int incl = wave_inclusive_scan(local);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      before += w < wave ? wsum[w] : 0;
      chunk += wsum[w];
    }
    const int excl = carry + before + incl - local;
    if (t0 < stride) {
      const i32x4 o = {kScanned | excl, kScanned | (excl + v[0]), kScanned | (excl + v[0] + v[1]),
                       kScanned | (excl + v[0] + v[1] + v[2])};
      __builtin_amdgcn_raw_buffer_store_b128(o, rrow, (int)(t0 * 4), 0, kCoherent);
    }
    carry += chunk;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (tid == 0) {
    put(totals + e, kScanned | carry);
    if (counts != nullptr) counts[e] = (accumulate ? counts[e] : 0) + carry;
  }
}

// A scanned word: its first (coherent, agent-scope atomic) load is issued with the others the
// caller needs, then finish() polls it (~0.25 us apart) until it carries kScanned.
__device__ __forceinline__ int load_scanned(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int finish_scanned(const int32_t* p, int v) {
  for (int spins = 0; (v & kScanned) == 0 && spins < kSpinLimit; ++spins) {
    __builtin_amdgcn_s_sleep(8);
    v = load_scanned(p);
  }
  return v & ~kScanned;
}

template <int K>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(const int32_t* __restrict__ idx, int64_t total,
                                                            int n_experts, int64_t n_tiles, int64_t stride,
                                                            int32_t* __restrict__ loads,
                                                            int32_t* __restrict__ totals,
                                                            int32_t* __restrict__ counts, int accumulate,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ inv, BalanceArgs update) {
  if ((int)blockIdx.x < n_experts) {
    // With an update, the update block sets the counts (it must store them before it clears them).
    scan_row((int)blockIdx.x, loads, n_tiles, stride, totals, update.counts != nullptr ? nullptr : counts, accumulate);
    return;
  }
  // With an update, the block right after the scan blocks runs it: dispatched ahead of the tile
  // blocks, it starts waiting for the totals as soon as the scans do (placed after the tile
  // blocks it started ~0.5-1 us later at 1024 tiles).
  const bool has_update = update.counts != nullptr;
  if (has_update && (int)blockIdx.x == n_experts) {
    // The bias update, one wave.
    if (threadIdx.x < 64) {
      BalanceIn in;
      balance_load_bm(update, in);  // issued before the wait
      int t[kBalancePer];
#pragma unroll
      for (int r = 0; r < kBalancePer; ++r) {
        const int e = (int)threadIdx.x + 64 * r;
        t[r] = e < n_experts ? load_scanned(totals + e) : kScanned;
        in.c[r] = e < n_experts && accumulate ? update.counts[e] : 0;
      }
#pragma unroll
      for (int r = 0; r < kBalancePer; ++r) {
        const int e = (int)threadIdx.x + 64 * r;
        in.c[r] += finish_scanned(totals + e, t[r]);
        if (e < n_experts && !update.clear) update.counts[e] = in.c[r];
      }
      balance_apply(update, in);
    }
    return;
  }
  // Tile blocks: padded to a multiple of 8, and those that land on one XCD (blocks go to the 8
  // XCDs in turn) take one contiguous range of tiles.  Neighbouring tiles write neighbouring
  // pieces (about K entries each) of every expert's bucket, so the partial lines of perm meet in
  // one L2 and go to memory whole, instead of piecewise from every XCD.
  const int64_t n_pad = (n_tiles + 7) / 8 * 8;
  const int64_t tb = (int64_t)blockIdx.x - n_experts - (has_update ? 1 : 0);
  const int64_t tile = (tb % 8) * (n_pad / 8) + tb / 8;
  if (tile >= n_tiles) return;
  __shared__ int wsum[kWaves];
  __shared__ int vcnt[K * kWaves][kMaxExperts];  // per virtual wave: count, then start
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t lo = tile * (kDispatchTile * K);

  int e[K];
#pragma unroll
  for (int c = 0; c < K; ++c) {
    const int64_t j = lo + c * kThreads + tid;
    const int raw = j < total ? idx[j] : -1;
    e[c] = (unsigned)raw < (unsigned)n_experts ? raw : -1;  // out-of-range ids are dropped
  }
#pragma unroll
  for (int v = 0; v < K * kWaves; ++v) vcnt[v][tid] = 0;
  __syncthreads();

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

  // The tile's offsets need the scan: totals and this tile's column of the scanned table.
  const int32_t* const at = loads + (int64_t)tid * stride + tile;
  int tot = 0, before = 0;
  if (tid < n_experts) {
    tot = load_scanned(totals + tid);
    before = load_scanned(at);
    tot = finish_scanned(totals + tid, tot);
    before = finish_scanned(at, before);
  }

  // Bucket start of expert tid: exclusive scan of the totals.
  const int incl = wave_inclusive_scan(tot);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int start = incl - tot;
  for (int w = 0; w < wave; ++w) start += wsum[w];
  if (tile == 0) {
    if (tid < n_experts) offsets[tid] = start;
    if (tid == 0) offsets[n_experts] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }
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
      // Always in range once the scan has been seen; only a wait that ran out (kSpinLimit)
      // could leave pos outside [0, total), and then the store is dropped, never misplaced.
      if ((uint32_t)pos >= (uint32_t)total) continue;
      perm[pos] = (int32_t)j;
      if (inv != nullptr) inv[j] = pos;
    }
  }
}

template <int K>
hipError_t launch_dispatch_k(const int32_t* idx, int64_t total, int n_experts, const DispatchGeom& g, int32_t* loads,
                             int32_t* totals, int32_t* counts, bool accumulate, int32_t* offsets,
                             int32_t* perm, int32_t* inv, const BalanceArgs* update, hipStream_t stream,
                             hipEvent_t ev_stop) {
  const BalanceArgs none{};
  const int64_t blocks = n_experts + (g.n_tiles + 7) / 8 * 8 + (update != nullptr ? 1 : 0);
  return launch_timed(dispatch_kernel<K>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, nullptr, ev_stop, idx,
                      total, n_experts, g.n_tiles, g.stride, loads, totals, counts, accumulate ? 1 : 0, offsets,
                      perm, inv, update != nullptr ? *update : none);
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
  if (!loads_ready) {
    const hipError_t err = launch(dispatch_loads_kernel, dim3((unsigned)g.n_tiles), dim3(kThreads), 0, stream, idx,
                                  total, k, n_experts, g.stride, loads);
    if (err != hipSuccess) return err;
  }
  switch (k) {
#define ELB_DISPATCH_K(KK) \
  case KK:                 \
    return launch_dispatch_k<KK>(idx, total, n_experts, g, loads, totals, counts, accumulate, offsets, perm, inv, \
                                 update, stream, ev_stop);
    ELB_DISPATCH_K(1)
    ELB_DISPATCH_K(2)
    ELB_DISPATCH_K(3)
    ELB_DISPATCH_K(4)
    ELB_DISPATCH_K(5)
    ELB_DISPATCH_K(6)
    ELB_DISPATCH_K(7)
#undef ELB_DISPATCH_K
    default:
      return launch_dispatch_k<8>(idx, total, n_experts, g, loads, totals, counts, accumulate, offsets, perm,
                                  inv, update, stream, ev_stop);
  }
}

}  // namespace elb

// Shape-generic router forward: fp32 or bf16 inputs, any n_experts <= 256, any K <= 8, any
// 16-byte-aligned row length.  This kernel carries the fp32 inputs (whose logits must stay
// fp32-exact) and every shape the MFMA kernel does not take; it favours plain, obviously
// correct code over speed.
//
// Per token t and expert i (Arcee Trinity Large Technical Report, section 2.3; hotdry blog
// post on Trinity Large MoE routing, section on sigmoid routing and Top-K; "SMEBU Load
// Balancing" study note, "How it works", eq. (17)):
//   z = u_t . e_i (fp32 FMA, ascending k), s = 1 / (1 + exp(-z)), q = s + b_i;
//   the K largest q are chosen one at a time (ties to the lower index), gates come from s.
//
// Layout: a workgroup of 256 threads handles 8 tokens at a time, thread i owning expert i (with
// at most 64 or 128 experts, the waves split the 8 tokens between them, each thread then owning
// expert i mod 64 or 128).  The 8 token rows are staged through LDS in chunks of 256 elements;
// each thread streams its own weight row.  Selection runs one token per wave-pass with a
// shuffle arg-max.
#include "device_common.hpp"
#include "elb_kernels.h"

#include "../../include/elb.h"

namespace elb {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 8;     // tokens per group
constexpr int kChunk = 256; // row elements staged per pass

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// 32 consecutive row elements as fp32, read as 16-byte vectors (p is 16-byte aligned: rows are,
// and the offset is a multiple of 32 elements), all issued before any is used.
constexpr int kVec = 32;
__device__ __forceinline__ void load_vec(const float* p, float (&v)[kVec]) {
  float4 q[kVec / 4];
#pragma unroll
  for (int i = 0; i < kVec / 4; ++i) q[i] = reinterpret_cast<const float4*>(p)[i];
#pragma unroll
  for (int i = 0; i < kVec / 4; ++i) {
    v[4 * i] = q[i].x;
    v[4 * i + 1] = q[i].y;
    v[4 * i + 2] = q[i].z;
    v[4 * i + 3] = q[i].w;
  }
}
__device__ __forceinline__ void load_vec(const uint16_t* p, float (&v)[kVec]) {
  uint4 q[kVec / 8];
#pragma unroll
  for (int i = 0; i < kVec / 8; ++i) q[i] = reinterpret_cast<const uint4*>(p)[i];
#pragma unroll
  for (int i = 0; i < kVec / 8; ++i) {
    const uint32_t u[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[8 * i + 2 * c] = __uint_as_float(u[c] << 16);
      v[8 * i + 2 * c + 1] = __uint_as_float(u[c] & 0xFFFF0000u);
    }
  }
}

// S: token subsets.  With at most 64 (128) experts, the waves split each group's 8 tokens four
// (two) ways: thread tid owns expert tid % (256 / S) for tokens tid / (256 / S) + S i, so that no
// thread multiplies more than 8 / S rows while most of the workgroup would otherwise idle.
template <typename Tin, int S>
__global__ __launch_bounds__(kThreads) void router_generic_kernel(const Tin* __restrict__ x, const Tin* __restrict__ w,
                                                                  const float* __restrict__ bias, int64_t T, int d,
                                                                  int n_experts, int K, int normalize,
                                                                  int32_t* __restrict__ idx_out,
                                                                  float* __restrict__ gates_out,
                                                                  int32_t* __restrict__ counts,
                                                                  float* __restrict__ logits, float* __restrict__ lse) {
  __shared__ float xs[kTok][kChunk];
  __shared__ float zs[kTok][256];
  __shared__ float ss[kTok][256];
  __shared__ float qs[kTok][256];
  __shared__ int hist[256];
  static_assert(kTok * kChunk % kThreads == 0 && kTok % S == 0, "tile shape");
  constexpr int kSlots = kThreads / S;  // experts per token subset
  constexpr int kMine = kTok / S;       // tokens per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ex = tid % kSlots;  // this thread's expert
  const int sub = tid / kSlots; // and token subset (wave-uniform)
  const bool live = ex < n_experts;
  const float b = live ? bias[ex] : 0.0f;
  hist[tid] = 0;

  const int64_t n_groups = (T + kTok - 1) / kTok;
  for (int64_t g = blockIdx.x; g < n_groups; g += gridDim.x) {
    const int64_t t0 = g * kTok;
    float z[kMine];  // token sub + S i
#pragma unroll
    for (int i = 0; i < kMine; ++i) z[i] = 0.0f;
    for (int k0 = 0; k0 < d; k0 += kChunk) {
      const int kn = d - k0 < kChunk ? d - k0 : kChunk;
      // All eight loads of this thread are issued before the first is stored (a loop that
      // stores each element as it arrives waits out one memory latency per element).
      float xv[kTok * kChunk / kThreads];
#pragma unroll
      for (int q = 0; q < kTok * kChunk / kThreads; ++q) {
        const int i = tid + q * kThreads;
        const int j = i / kChunk, kk = i % kChunk;
        xv[q] = (t0 + j < T && kk < kn) ? load_elem(x, (t0 + j) * (int64_t)d + k0 + kk) : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kTok * kChunk / kThreads; ++q) {
        const int i = tid + q * kThreads;
        xs[i / kChunk][i % kChunk] = xv[q];
      }
      __syncthreads();
      if (live) {
        // The thread's weight row, 32 elements per pass read ahead as vectors (a scalar load per
        // element would expose every load's latency), multiplied in ascending k.
        const Tin* wr = w + (int64_t)ex * d + k0;
        int kk = 0;
        for (; kk + kVec <= kn; kk += kVec) {
          float wv[kVec];
          load_vec(wr + kk, wv);
#pragma unroll
          for (int u = 0; u < kVec; ++u)
#pragma unroll
            for (int i = 0; i < kMine; ++i) z[i] = fmaf(xs[sub + S * i][kk + u], wv[u], z[i]);
        }
        for (; kk < kn; ++kk) {
          const float wv = load_elem(wr, kk);
#pragma unroll
          for (int i = 0; i < kMine; ++i) z[i] = fmaf(xs[sub + S * i][kk], wv, z[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int j = sub + S * i;
      const float s = 1.0f / (1.0f + expf(-z[i]));
      zs[j][ex] = z[i];
      ss[j][ex] = s;
      qs[j][ex] = live ? s + b : -__builtin_inff();
      if (logits != nullptr && live && t0 + j < T) logits[(t0 + j) * n_experts + ex] = z[i];
    }
    __syncthreads();

    // Selection: wave `wave` handles tokens wave, wave + 4; lane l holds experts l + 64 c.
    for (int j = wave; j < kTok; j += kThreads / 64) {
      const int64_t t = t0 + j;
      if (t >= T) continue;
      float qv[4];
      int taken = 0;  // bit c: expert lane + 64 c already chosen
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        qv[c] = e < n_experts ? qs[j][e] : -__builtin_inff();
      }
      float ssum = 0.0f;
      int chosen[8];
      float sval[8];
      for (int r = 0; r < K; ++r) {
        float bq = -__builtin_inff();
        int be = 0x7fffffff;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = lane + 64 * c;
          if (!((taken >> c) & 1) && e < n_experts && (qv[c] > bq || (qv[c] == bq && e < be))) {
            bq = qv[c];
            be = e;
          }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          const float oq = __shfl_xor(bq, off);
          const int oe = __shfl_xor(be, off);
          if (oq > bq || (oq == bq && oe < be)) {
            bq = oq;
            be = oe;
          }
        }
        if (be >= n_experts) be = 0;  // only reachable with NaN scores; keeps every index in range
        if ((be & 63) == lane) taken |= 1 << (be >> 6);
        chosen[r] = be;
        sval[r] = ss[j][be];
        ssum += sval[r];
      }
      if (lane == 0) {
        for (int r = 0; r < K; ++r) {
          idx_out[t * K + r] = chosen[r];
          gates_out[t * K + r] = normalize ? sval[r] / ssum : sval[r];
          atomicAdd(&hist[chosen[r]], 1);
        }
      }
      if (lse != nullptr) {
        float m = -__builtin_inff();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = lane + 64 * c;
          if (e < n_experts) m = fmaxf(m, zs[j][e]);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = lane + 64 * c;
          if (e < n_experts) acc += expf(zs[j][e] - m);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) lse[t] = m + logf(acc);
      }
    }
  }
  __syncthreads();
  if (tid < n_experts && counts != nullptr && hist[tid] != 0) atomicAdd(&counts[tid], hist[tid]);
}

template <typename Tin>
hipError_t launch_s(const RouterArgs& a, int subsets, int grid, int normalize, hipStream_t stream) {
  auto kernel = subsets == 4 ? router_generic_kernel<Tin, 4>
                             : subsets == 2 ? router_generic_kernel<Tin, 2> : router_generic_kernel<Tin, 1>;
  return launch_timed(kernel, dim3(grid), dim3(kThreads), 0, stream, nullptr, a.ev_stop, (const Tin*)a.x,
                      (const Tin*)a.w, a.bias, a.T, a.d, a.n_experts, a.k, normalize, a.idx, a.gates, a.counts,
                      a.logits, a.lse);
}

}  // namespace

hipError_t launch_router_generic(const RouterArgs& a, hipStream_t stream) {
  const int64_t n_groups = (a.T + kTok - 1) / kTok;
  const int grid = (int)(n_groups < 2048 ? n_groups : 2048);
  const int normalize = (a.flags & ELB_GATES_RAW) ? 0 : 1;
  const int subsets = a.n_experts <= 64 ? 4 : a.n_experts <= 128 ? 2 : 1;
  if (a.dtype == ELB_F32) return launch_s<float>(a, subsets, grid, normalize, stream);
  return launch_s<uint16_t>(a, subsets, grid, normalize, stream);
}

}  // namespace elb

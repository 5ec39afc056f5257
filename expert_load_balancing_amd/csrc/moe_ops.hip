// Expert-side data movement around the router: token rows to expert-contiguous rows, and the
// gated combine of expert outputs back to token order.
//
// The gating scores weight the routed experts' outputs and the results are summed per token
// (Arcee Trinity Large Technical Report, section 2.3 "Mixture-of-Experts").  Between the two,
// each expert's tokens form one contiguous block: row p of the expert-contiguous buffer holds
// the token of flat assignment perm[p], i.e. assignment (t, j) sits at row inv[t * K + j] (the
// dispatch permutation of dispatch.hip).
//
// Both kernels are HBM streams with no reuse, so the design is about bytes, not math:
//  * permute scatters BY TOKEN: each token row is read once and written to its K rows, so the
//    tokens cost T * row_bytes of reads instead of K * T (a gather by expert row would re-read
//    every token K times, from HBM, since its K copies are far apart in the buffer);
//  * combine gathers by token: one wave per token reads its K expert rows and writes y once;
//  * one wave owns one token row at a time; its lanes move 16 bytes each per step, rows are
//    walked in steps of 1 KiB with several steps in flight.  The grid is capped (kMaxBlocks)
//    and the waves stride over the tokens, so every T the API accepts launches (a grid of one
//    wave per token would pass the 32-bit work-item count of a dispatch at T = 2^26);
//  * everything is read or written exactly once, so all global traffic is non-temporal.
#include "../../include/elb.h"
#include "device_common.hpp"
#include "elb_kernels.h"

namespace elb {
namespace {

using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr int kWavesPerBlock = 4;
constexpr int kUnrollRow = 4;  // 16-byte chunks in flight per lane
constexpr int64_t kMaxBlocks = int64_t(1) << 20;  // 4 Mi waves, far more than the GPU holds at once

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// xp[inv[t*K + j]] = x[t] for every j.  chunks = row_bytes / 16.
__global__ __launch_bounds__(64 * kWavesPerBlock) void permute_rows_kernel(const u32x4* __restrict__ x, int64_t T,
                                                                           int64_t chunks, int k,
                                                                           const int32_t* __restrict__ inv,
                                                                           u32x4* __restrict__ xp) {
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); t < T;
       t += (int64_t)gridDim.x * kWavesPerBlock) {
    int64_t dst[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = j < k ? (int64_t)inv[t * k + j] * chunks : 0;
    const u32x4* src = x + t * chunks;
    for (int64_t c0 = 0; c0 < chunks; c0 += 64 * kUnrollRow) {
      u32x4 v[kUnrollRow];
#pragma unroll
      for (int u = 0; u < kUnrollRow; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < chunks) v[u] = load_nt(src + c);
      }
#pragma unroll
      for (int u = 0; u < kUnrollRow; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < chunks) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < k) store_nt(xp + dst[j] + c, v[u]);
        }
      }
    }
  }
}

__device__ __forceinline__ void widen8(u32x4 v, float (&f)[8]) {  // 8 bf16 -> fp32, exact
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(v[q] << 16);
    f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  // Round to nearest, ties to even (inputs are finite).
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// y[t] = sum_j g[t, j] * eo[inv[t*K + j]], fp32 in slot order.  IN_BF16: 8 elements per 16-byte
// chunk, else 4.  OUT_BF16: y stored as bf16 (round to nearest even), else fp32.
template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(64 * kWavesPerBlock) void combine_kernel(const u32x4* __restrict__ eo, int64_t T,
                                                                      int64_t chunks, int k,
                                                                      const int32_t* __restrict__ inv,
                                                                      const float* __restrict__ gates,
                                                                      void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); t < T;
       t += (int64_t)gridDim.x * kWavesPerBlock) {
    constexpr int kPer = IN_BF16 ? 8 : 4;  // elements per chunk
    int64_t src[8];
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      src[j] = j < k ? (int64_t)inv[t * k + j] * chunks : 0;
      g[j] = j < k ? gates[t * k + j] : 0.0f;
    }
    for (int64_t c0 = 0; c0 < chunks; c0 += 64 * 2) {
      float acc[2][kPer];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[u][e] = 0.0f;
      u32x4 v[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t c = c0 + u * 64 + lane;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < k && c < chunks) v[u][j] = load_nt(eo + src[j] + c);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c >= chunks) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j >= k) break;
          float f[kPer];
          if constexpr (IN_BF16) {
            widen8(v[u][j], f);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[u][j][e]);
          }
#pragma unroll
          for (int e = 0; e < kPer; ++e) acc[u][e] = __builtin_fmaf(g[j], f[e], acc[u][e]);
        }
        const int64_t e0 = c * kPer;  // first element of this chunk in the row
        if constexpr (OUT_BF16) {
          uint32_t* yo = static_cast<uint32_t*>(y) + (t * chunks * kPer + e0) / 2;
          if constexpr (kPer == 8) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              o[q] = f32_to_bf16_rne(acc[u][2 * q]) | (f32_to_bf16_rne(acc[u][2 * q + 1]) << 16);
            store_nt(reinterpret_cast<u32x4*>(yo), o);
          } else {
            using u32x2 = unsigned int __attribute__((ext_vector_type(2)));
            u32x2 o;
            o[0] = f32_to_bf16_rne(acc[u][0]) | (f32_to_bf16_rne(acc[u][1]) << 16);
            o[1] = f32_to_bf16_rne(acc[u][2]) | (f32_to_bf16_rne(acc[u][3]) << 16);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(yo));
          }
        } else {
          float* yo = static_cast<float*>(y) + t * chunks * kPer + e0;
#pragma unroll
          for (int q = 0; q < kPer / 4; ++q) {
            const f32x4 o{acc[u][4 * q], acc[u][4 * q + 1], acc[u][4 * q + 2], acc[u][4 * q + 3]};
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(yo) + q);
          }
        }
      }
    }
  }
}

dim3 token_grid(int64_t T) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  return dim3((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks));
}

}  // namespace

hipError_t launch_permute_rows(const void* x, int64_t T, int64_t row_bytes, int k, const int32_t* inv, void* xp,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  return launch(permute_rows_kernel, token_grid(T), dim3(64 * kWavesPerBlock), 0, stream,
                static_cast<const u32x4*>(x), T, row_bytes / 16, k, inv, static_cast<u32x4*>(xp));
}

hipError_t launch_combine(const void* eo, int in_dtype, int64_t T, int d, int k, const int32_t* inv,
                          const float* gates, void* y, int out_dtype, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t chunks = in_dtype == ELB_BF16 ? d / 8 : d / 4;
  const u32x4* e = static_cast<const u32x4*>(eo);
  const dim3 grid = token_grid(T), block(64 * kWavesPerBlock);
  if (in_dtype == ELB_BF16)
    return out_dtype == ELB_BF16 ? launch(combine_kernel<true, true>, grid, block, 0, stream, e, T, chunks, k, inv, gates, y)
                                 : launch(combine_kernel<true, false>, grid, block, 0, stream, e, T, chunks, k, inv, gates, y);
  return out_dtype == ELB_BF16 ? launch(combine_kernel<false, true>, grid, block, 0, stream, e, T, chunks, k, inv, gates, y)
                               : launch(combine_kernel<false, false>, grid, block, 0, stream, e, T, chunks, k, inv, gates, y);
}

}  // namespace elb

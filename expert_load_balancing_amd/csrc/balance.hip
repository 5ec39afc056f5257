// Expert-bias update / MaxVio launches (the arithmetic and its citations live in
// balance_wave.hpp, which the dispatch scatter also runs as an extra workgroup when a routed
// step asks for the update), and the router z-loss reduction.
#include "balance_wave.hpp"

namespace elb {
namespace {

// One workgroup (one wave) per MoE layer; layer l's rows of counts, b, m, delta_b are
// [l * n, (l + 1) * n) and its MaxVio pair is maxvio[2 l], maxvio[2 l + 1].  Layers share
// nothing: each has its own loads, bias and momentum ("SMEBU Load Balancing", "How it works":
// the update is stated per router).
__global__ __launch_bounds__(64) void balance_layers_kernel(BalanceArgs a) {
  const int64_t off = (int64_t)blockIdx.x * a.n;
  BalanceArgs l = a;
  l.counts += off;
  if (l.bias != nullptr) l.bias += off;
  if (l.momentum != nullptr) l.momentum += off;
  if (l.delta_b != nullptr) l.delta_b += off;
  if (l.maxvio != nullptr) l.maxvio += 2 * (int64_t)blockIdx.x;
  balance_wave(l);
}

// Router z-loss from per-token log-sum-exps: mean_t lse_t^2 (talk summary "Arcee Halts 400B
// Blackwell Model Collapse With Dynamic Router Biases", section "Precision Fallbacks, Loss
// Stabilization, and MaxVio as Data Telemetry": L_z = log^2 sum e^x).  One workgroup; each
// thread adds its strided share in float64 in index order, then a butterfly per wave and the
// waves in order: the same bits every run.
constexpr int kZThreads = 1024;
__global__ __launch_bounds__(kZThreads) void zloss_kernel(const float* __restrict__ lse, int64_t T,
                                                          float* __restrict__ out) {
  __shared__ double part[kZThreads / 64];
  double acc = 0.0;
  // Eight loads in flight per thread, then the adds in index order (the same order, and so the
  // same bits, as one element at a time).
  int64_t i = threadIdx.x;
  for (; i + 7 * kZThreads < T; i += 8 * kZThreads) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = lse[i + q * kZThreads];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += (double)v[q] * (double)v[q];
  }
  for (; i < T; i += kZThreads) {
    const double v = lse[i];
    acc += v * v;
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kZThreads / 64; ++w) s += part[w];
    out[0] = T > 0 ? (float)(s / (double)T) : 0.0f;
  }
}

}  // namespace

hipError_t launch_balance_layers(const BalanceArgs& a, int n_layers, hipStream_t stream, hipEvent_t ev_stop) {
  return launch_timed(balance_layers_kernel, dim3((unsigned)n_layers), dim3(64), 0, stream, nullptr, ev_stop, a);
}

hipError_t launch_balance(const BalanceArgs& a, hipStream_t stream, hipEvent_t ev_stop) {
  return launch_balance_layers(a, 1, stream, ev_stop);
}

hipError_t launch_zloss(const float* lse, int64_t T, float* out, hipStream_t stream, hipEvent_t ev_stop) {
  return launch_timed(zloss_kernel, dim3(1), dim3(kZThreads), 0, stream, nullptr, ev_stop, lse, T, out);
}

}  // namespace elb

// Expert-bias update and MaxVio: one workgroup, one expert per thread slot.
//
// SMEBU ("SMEBU Load Balancing" study note, "How it works", eq. (23)-(28)):
//   v_i = (nbar - n_i) / nbar, vt_i = tanh(kappa v_i), db_i = lambda vt_i,
//   db_i -= mean(db), m_i = beta m_i + (1 - beta) db_i, b_i += m_i.
// Sign step of Trinity Nano/Mini (same note, eq. (20)-(22)): b_i += gamma sign(nbar - n_i),
//   then b is re-centred to zero mean (the re-centre of the updated b).
// Linear: SMEBU with vt_i = v_i (the unclamped update the note contrasts SMEBU with).
// MaxVio: max n / min n (talk summary "Arcee Halts 400B Blackwell Model Collapse With Dynamic
//   Router Biases", section "The MaxVio Metric and the Day-4 Crisis") and (max n - nbar) / nbar.
//
// The update is latency-bound (N_r = 256 values); what matters is that it is exact where it
// can be and deterministic everywhere:
//  * sums of loads are int64, so nbar and the signs nbar - n_i are exact;
//  * v_i = (S - N n_i) / S is one rounding of an exact integer ratio (S = sum n);
//  * float means use a fixed-order tree, so repeated runs give identical bits.
#include "device_common.hpp"
#include "elb_kernels.h"

namespace elb {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 4;  // experts per thread: up to 1024 experts

template <typename T, typename Op>
__device__ T block_reduce(T v, T* scratch, Op op) {
  // Fixed-order tree over the 256 thread values: deterministic.
  scratch[threadIdx.x] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) scratch[threadIdx.x] = op(scratch[threadIdx.x], scratch[threadIdx.x + s]);
    __syncthreads();
  }
  T r = scratch[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void balance_kernel(const int32_t* __restrict__ counts, int n, int mode,
                                                           float lambda, float beta, float kappa, float gamma,
                                                           float* __restrict__ bias, float* __restrict__ momentum,
                                                           float* __restrict__ delta_b, float* __restrict__ maxvio) {
  __shared__ long long si[kThreads];
  __shared__ float sf[kThreads];
  const int tid = threadIdx.x;

  long long c[kPer];
  long long lsum = 0, lmax = LLONG_MIN, lmin = LLONG_MAX;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * kThreads;
    c[r] = e < n ? (long long)counts[e] : 0;
    if (e < n) {
      lsum += c[r];
      lmax = c[r] > lmax ? c[r] : lmax;
      lmin = c[r] < lmin ? c[r] : lmin;
    }
  }
  const long long S = block_reduce<long long>(lsum, si, [](long long a, long long b) { return a + b; });
  const long long nmax = block_reduce<long long>(lmax, si, [](long long a, long long b) { return a > b ? a : b; });
  const long long nmin = block_reduce<long long>(lmin, si, [](long long a, long long b) { return a < b ? a : b; });

  if (maxvio != nullptr && tid == 0) {
    if (S == 0) {
      maxvio[0] = __builtin_nanf("");
      maxvio[1] = __builtin_nanf("");
    } else {
      maxvio[0] = nmin == 0 ? __builtin_inff() : float(double(nmax) / double(nmin));
      maxvio[1] = float(double((long long)n * nmax - S) / double(S));
    }
  }
  if (mode < 0) return;  // MaxVio only

  if (S == 0) {  // no routed tokens: the step is skipped
    if (delta_b != nullptr) {
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int e = tid + r * kThreads;
        if (e < n) delta_b[e] = 0.0f;
      }
    }
    return;
  }

  const float fS = float(S);
  float db[kPer];
  if (mode == 1) {  // sign step, then re-centre the updated bias
    float nb[kPer];
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int e = tid + r * kThreads;
      const long long diff = S - (long long)n * c[r];  // sign(nbar - n_e) = sign(S - N n_e)
      db[r] = diff > 0 ? gamma : (diff < 0 ? -gamma : 0.0f);
      nb[r] = e < n ? bias[e] + db[r] : 0.0f;
      part += nb[r];
    }
    const float mean = block_reduce<float>(part, sf, [](float a, float b) { return a + b; }) / float(n);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int e = tid + r * kThreads;
      if (e < n) {
        bias[e] = nb[r] - mean;
        if (delta_b != nullptr) delta_b[e] = db[r];
      }
    }
    return;
  }

  // SMEBU (mode 0) or linear (mode 2).
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * kThreads;
    const float v = float(S - (long long)n * c[r]) / fS;  // (nbar - n_e) / nbar
    const float vt = mode == 0 ? tanhf(kappa * v) : v;
    db[r] = e < n ? lambda * vt : 0.0f;
    part += db[r];
  }
  const float mean = block_reduce<float>(part, sf, [](float a, float b) { return a + b; }) / float(n);
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = tid + r * kThreads;
    if (e < n) {
      const float d = db[r] - mean;
      const float m = beta * momentum[e] + (1.0f - beta) * d;
      momentum[e] = m;
      bias[e] = bias[e] + m;
      if (delta_b != nullptr) delta_b[e] = d;
    }
  }
}

}  // namespace

hipError_t launch_balance(const int32_t* counts, int n_experts, int mode, float lambda, float beta, float kappa,
                          float gamma, float* bias, float* momentum, float* delta_b, float* maxvio,
                          hipStream_t stream) {
  return launch(balance_kernel, dim3(1), dim3(kThreads), 0, stream, counts, n_experts, mode, lambda, beta, kappa,
                gamma, bias, momentum, delta_b, maxvio);
}

}  // namespace elb

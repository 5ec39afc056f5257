// Expert-bias update and MaxVio computed by ONE wavefront (64 lanes, up to 1024 experts).
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
// The update is latency-bound (a few hundred values), so it runs in one wave with no LDS and
// no barrier: every reduction is a butterfly of lane shuffles.  It is exact where it can be
// and deterministic everywhere:
//  * sums of loads are int64, so nbar and the signs nbar - n_i are exact;
//  * v_i = (S - N n_i) / S is one rounding of an exact integer ratio (S = sum n);
//  * float sums add each lane's experts in a fixed order, then butterfly: a + b is
//    commutative, so every lane ends with the same bits, run after run.
#pragma once

#include "../../include/elb.h"
#include "device_common.hpp"
#include "elb_kernels.h"

namespace elb {

constexpr int kBalancePer = 16;  // experts per lane: 64 * 16 = 1024

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
  return v;
}

// What one lane holds of the update's inputs: its experts lane + 64 r.
struct BalanceIn {
  int c[kBalancePer];
  float b0[kBalancePer], m0[kBalancePer];
};

// Bias and momentum of the lane's experts (what the mode needs of them).
__device__ __forceinline__ void balance_load_bm(const BalanceArgs& a, BalanceIn& in) {
  const int lane = threadIdx.x & 63;
  const bool need_b = a.mode >= 0;
  const bool need_m = a.mode >= 0 && a.mode != ELB_MODE_SIGN;
#pragma unroll
  for (int r = 0; r < kBalancePer; ++r) {
    const int e = lane + 64 * r;
    in.b0[r] = need_b && e < a.n ? a.bias[e] : 0.0f;
    in.m0[r] = need_m && e < a.n ? a.momentum[e] : 0.0f;
  }
}

__device__ __forceinline__ void balance_apply(const BalanceArgs& a, const BalanceIn& in);

// Runs on the 64 lanes of the calling wave (lane = threadIdx.x & 63).
__device__ __forceinline__ void balance_wave(const BalanceArgs& a) {
  const int lane = threadIdx.x & 63;
  // Every load is issued up front: one memory round trip instead of one per dependent step.
  BalanceIn in;
#pragma unroll
  for (int r = 0; r < kBalancePer; ++r) {
    const int e = lane + 64 * r;
    in.c[r] = e < a.n ? a.counts[e] : 0;
  }
  balance_load_bm(a, in);
  balance_apply(a, in);
}

// The update from the lane's inputs; with a.clear, zeroes the lane's entries of a.counts.
__device__ __forceinline__ void balance_apply(const BalanceArgs& a, const BalanceIn& in) {
  const int lane = threadIdx.x & 63;
  const int n = a.n;
  const int* const c = in.c;
  const float* const b0 = in.b0;
  const float* const m0 = in.m0;
  long long lsum = 0;
  int lmax = -2147483647 - 1, lmin = 2147483647;
#pragma unroll
  for (int r = 0; r < kBalancePer; ++r) {
    if (lane + 64 * r < n) {
      lsum += c[r];
      lmax = max(lmax, c[r]);
      lmin = min(lmin, c[r]);
    }
  }
  if (a.clear) {  // each lane clears exactly its own entries
#pragma unroll
    for (int r = 0; r < kBalancePer; ++r) {
      const int e = lane + 64 * r;
      if (e < n) a.counts[e] = 0;
    }
  }
  const long long S = wave_sum(lsum);
  const int nmax = wave_max(lmax);
  const int nmin = wave_min(lmin);

  if (a.maxvio != nullptr && lane == 0) {
    if (S == 0) {
      a.maxvio[0] = __builtin_nanf("");
      a.maxvio[1] = __builtin_nanf("");
    } else {
      a.maxvio[0] = nmin == 0 ? __builtin_inff() : float(double(nmax) / double(nmin));
      a.maxvio[1] = float(double((long long)n * nmax - S) / double(S));
    }
  }
  if (a.mode < 0) return;  // MaxVio only

  if (S == 0) {  // no routed tokens: the step is skipped
    if (a.delta_b != nullptr) {
#pragma unroll
      for (int r = 0; r < kBalancePer; ++r) {
        const int e = lane + 64 * r;
        if (e < n) a.delta_b[e] = 0.0f;
      }
    }
    return;
  }

  float db[kBalancePer];
  if (a.mode == ELB_MODE_SIGN) {  // sign step, then re-centre the updated bias
    float nb[kBalancePer];
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < kBalancePer; ++r) {
      const int e = lane + 64 * r;
      const long long diff = S - (long long)n * c[r];  // sign(nbar - n_e) = sign(S - N n_e)
      db[r] = diff > 0 ? a.gamma : (diff < 0 ? -a.gamma : 0.0f);
      nb[r] = e < n ? b0[r] + db[r] : 0.0f;
      part += nb[r];
    }
    const float mean = wave_sum(part) / float(n);
#pragma unroll
    for (int r = 0; r < kBalancePer; ++r) {
      const int e = lane + 64 * r;
      if (e < n) {
        a.bias[e] = nb[r] - mean;
        if (a.delta_b != nullptr) a.delta_b[e] = db[r];
      }
    }
    return;
  }

  // SMEBU or linear.
  const float fS = float(S);
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < kBalancePer; ++r) {
    db[r] = 0.0f;
    if (lane + 64 * r < n) {  // skipped whole-wave for the unused slots
      const float v = float(S - (long long)n * c[r]) / fS;  // (nbar - n_e) / nbar
      const float vt = a.mode == ELB_MODE_SMEBU ? tanhf(a.kappa * v) : v;
      db[r] = a.lambda * vt;
    }
    part += db[r];
  }
  const float mean = wave_sum(part) / float(n);
#pragma unroll
  for (int r = 0; r < kBalancePer; ++r) {
    const int e = lane + 64 * r;
    if (e < n) {
      const float d = db[r] - mean;
      const float m = a.beta * m0[r] + (1.0f - a.beta) * d;
      a.momentum[e] = m;
      a.bias[e] = b0[r] + m;
      if (a.delta_b != nullptr) a.delta_b[e] = d;
    }
  }
}

}  // namespace elb

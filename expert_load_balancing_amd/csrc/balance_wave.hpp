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

// Cross-lane steps through the vector ALU's data-parallel primitives (DPP): each is a register
// move with a lane pattern, a few cycles, where a shuffle (ds_bpermute) is a round trip through
// the LDS crossbar and waits for it at every step of a reduction.
namespace dpp {
constexpr int kXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]: lane i <- i ^ 1
constexpr int kXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]: lane i <- i ^ 2
constexpr int kHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int kMirror = 0x140;      // lane i <- 15 - i within each row of 16 lanes
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;  // lane i <- i - n in its row, else 0
constexpr int kBcast15 = 0x142;     // lane 15 of each row to the whole next row (rows picked by the mask)
constexpr int kBcast31 = 0x143;     // lane 31 to rows 2 and 3 (picked by the mask)

// The value of the lane CTRL names; 0 in lanes whose source is out of the row, or whose row
// ROW_MASK leaves out.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int mov(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float mov(float v) {
  return __builtin_bit_cast(float, mov<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL, typename T>
__device__ __forceinline__ T mov64(T v) {  // 8-byte values, as two 4-byte moves
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned long long lo = (unsigned)mov<CTRL>((int)(unsigned)u);
  const unsigned long long hi = (unsigned)mov<CTRL>((int)(unsigned)(u >> 32));
  return __builtin_bit_cast(T, lo | (hi << 32));
}
template <int CTRL> __device__ __forceinline__ long long mov(long long v) { return mov64<CTRL>(v); }
template <int CTRL> __device__ __forceinline__ double mov(double v) { return mov64<CTRL>(v); }

__device__ __forceinline__ int lane_value(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
template <typename T>
__device__ __forceinline__ T lane_value64(T v, int lane) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned long long lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, lane);
  const unsigned long long hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), lane);
  return __builtin_bit_cast(T, lo | (hi << 32));
}
__device__ __forceinline__ long long lane_value(long long v, int lane) { return lane_value64(v, lane); }
__device__ __forceinline__ double lane_value(double v, int lane) { return lane_value64(v, lane); }

// op over the 64 lanes, the same bits in every lane: pairs within each quad, quads within each
// 8 lanes, those within each row of 16 (every step combines two equal-sized groups, and each
// lane of a pair applies the commutative op to the same two operands), then the four rows in a
// fixed order from scalar reads.
template <typename T, typename Op>
__device__ __forceinline__ T reduce(T v, Op op) {
  v = op(v, mov<kXor1>(v));
  v = op(v, mov<kXor2>(v));
  v = op(v, mov<kHalfMirror>(v));
  v = op(v, mov<kMirror>(v));
  return op(op(lane_value(v, 0), lane_value(v, 16)), op(lane_value(v, 32), lane_value(v, 48)));
}
}  // namespace dpp

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return dpp::reduce(v, [](T a, T b) { return a + b; });
}

__device__ __forceinline__ int wave_max(int v) {
  return dpp::reduce(v, [](int a, int b) { return max(a, b); });
}

__device__ __forceinline__ int wave_min(int v) {
  return dpp::reduce(v, [](int a, int b) { return min(a, b); });
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

// Fused router forward for bf16 inputs on CDNA4 matrix cores (gfx950).
//
// What it computes, per token t and routed expert i (Arcee Trinity Large Technical Report,
// section 2.3 "Mixture-of-Experts"; hotdry blog post on Trinity Large MoE routing, section on
// sigmoid routing and Top-K; "SMEBU Load Balancing" study note, "How it works", eq. (17)):
//   z_{t,i} = u_t . e_i          bf16 x bf16 products, fp32 accumulation (MFMA)
//   s_{t,i} = sigmoid(z_{t,i})   fp32
//   the K experts with the largest s + b_i (ties to the lower index), listed in descending
//   order; gates are s of the chosen experts (normalised over the K, or raw); the bias never
//   reaches the gates; per-expert loads n_i are counted on the way.
// No logit is written to memory unless the caller asks for the debug copy.
//
// Work decomposition
//   One workgroup (8 waves, two per SIMD) owns a tile of 256 tokens x all 256 experts and
//   keeps the 256x256 fp32 logit tile in registers: each wave pair shares 64 tokens, and each
//   wave of the pair holds 128 of the experts (8 accumulators of 32x32).  Batches of at most
//   128 x 256 tokens (one 256-token tile per CU would leave CUs idle) take 128-token tiles
//   instead: each wave pair 32 tokens.  Two waves per SIMD let one wave's LDS reads and
//   selection run under the other's MFMAs.
//   The contraction is written transposed, Z^T = W . X^T, so that the 32x32 MFMA output puts
//   one token per lane column: a lane ends up holding 64 of its wave's 128 logits of each of
//   its tokens, and the other 64 sit in lane ^ 32.  Top-K needs only a small LDS exchange: a
//   register-local selection over 64 values, one cross-lane merge, then the K best of the
//   partner wave through LDS.
//
// Memory pipeline: the product runs on the shared streaming tile of mfma_tile.hpp with
//   A = the router weights (L2-resident, cached) and B = the tile's tokens (read once from HBM,
//   non-temporal): d is consumed in stages of 64 elements through a DMA ring in LDS.
//
// Epilogue (per lane, per token): s = 1 / (1 + 2^(-z log2 e)) with the hardware exp2/rcp;
//   the selection key is the fp32 bit pattern of s + b' with its low 8 bits replaced by an
//   index, where b' = b + (1 - min b) >= 1 keeps every key a positive float, so float max and
//   med3 order keys exactly like (s + b, -index).  Inside a lane the index is the lane-local
//   slot (ascending with the expert id); the K survivors are re-keyed with 255 - expert before
//   the cross-lane merge.  Keeping 24 bits of s + b' resolves differences down to
//   2^-15 (1 + max b - min b); closer calls go to the lower index.  Insertion into a sorted
//   top-K list is one max plus K-1 med3.  The chosen experts' exact scores come back through
//   LDS for the gates.  Loads: LDS histogram, one global atomic per expert per workgroup.
#include "device_common.hpp"
#include "elb_kernels.h"
#include "mfma_tile.hpp"

#include "../../include/elb.h"

namespace elb {
namespace {

using namespace tile;  // the streaming product and its constants

constexpr int kExp = kRowsA;              // experts per tile (padded)
constexpr int kTile = kRowsB;             // tokens per workgroup of the full tile (NB = 2)
constexpr int kCus = 256;                 // compute units of the MI355X
constexpr float kLog2e = 1.4426950408889634f;

// Sorted (descending) top-K insertion: the new j-th largest is med3(old (j-1)-th, old j-th, x).
template <int K>
__device__ __forceinline__ void topk_insert(float (&top)[K], float x) {
#pragma unroll
  for (int j = K - 1; j > 0; --j) top[j] = __builtin_amdgcn_fmed3f(top[j - 1], top[j], x);
  top[0] = fmaxf(top[0], x);
}

__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Epilogue of the 8-wave tile.  Wave w holds experts 128 eh .. + 127 (eh = w % 2) of
// tokens 32 NB tq .. (tq = w / 2); a lane holds 64 of them for its token, lane ^ 32 the other 64.
// Per 32-token block: every wave selects its K best (same keys as the 4-wave epilogue, a
// lane-local slot in the low bits, re-keyed with 255 - expert before the merges), parks its
// scores, and leaves its K keys (and, with EXTRA, its log-sum-exp partial) in LDS; after a
// barrier one wave of each pair (eh = block parity) merges the partner's K keys and writes the
// token's indices, gates and histogram counts.  b' (the shifted bias) is in ws1[0..1 KiB), the
// histogram in ws1[1..2 KiB).
template <int K, bool FULL, bool EXTRA, int NB>
__device__ __forceinline__ void epilogue_split(const f32x16 (&acc)[kMB / 2][NB], int tid, int wave, int lane,
                                               int64_t row0, int64_t T, int n_experts, int normalize, float bshift,
                                               unsigned char* xs0, unsigned char* xs1, unsigned char* xs2,
                                               unsigned char* ws0, unsigned char* ws1, int32_t* __restrict__ idx_out,
                                               float* __restrict__ gates_out, float* __restrict__ logits,
                                               float* __restrict__ lse) {
  constexpr int kMBw = kMB / 2;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int eh = wave & 1, tq = wave >> 1;
  float* const bprime = reinterpret_cast<float*>(ws1);
  int* const hist = reinterpret_cast<int*>(ws1 + 1024);
  float* const xkey = reinterpret_cast<float*>(ws1 + 2048);                   // [8 waves][32 tokens][8]
  float2* const xlse = reinterpret_cast<float2*>(ws1 + 2048 + 8 * 32 * 8 * 4);  // [8 waves][32 tokens]
  if (tid < kExp) {
    bprime[tid] = tid < n_experts ? bshift : 0.0f;
    hist[tid] = 0;
  }
  // Parks: wave v's scores in the 16 KiB half (v & 1) of slot v / 2, [16 groups][64 lanes][4].
  auto park_of = [&](int v) {
    unsigned char* const sl = (v >> 1) == 0 ? xs0 : (v >> 1) == 1 ? xs1 : (v >> 1) == 2 ? xs2 : ws0;
    return reinterpret_cast<float*>(sl + (v & 1) * 16384);
  };
  float* const park = park_of(wave);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  bare_barrier();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t t = row0 + tq * (32 * NB) + nb * 32 + l32;
    float top[K];
#pragma unroll
    for (int j = 0; j < K; ++j) top[j] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < kMBw; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e0 = 128 * eh + mb * 32 + g * 8 + 4 * h;
        const f32x4 bp = *reinterpret_cast<const f32x4*>(bprime + e0);
        f32x4 sv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = sigmoid_fast(acc[mb][nb][g * 4 + r]);
          sv[r] = sc;
          const uint32_t slot_id = (uint32_t)(63 - (mb * 16 + g * 4 + r));  // lane-local, ascending expert
          const float key = __uint_as_float((__float_as_uint(sc + bp[r]) & 0xFFFFFF00u) | slot_id);
          topk_insert<K>(top, FULL || e0 + r < n_experts ? key : 0.0f);
        }
        *reinterpret_cast<f32x4*>(park + ((mb * 4 + g) * 64 + lane) * 4) = sv;
      }
    }
    // Re-key with the global expert id, merge with lane ^ 32 (the wave's other 64 experts).
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t bits = __float_as_uint(top[j]);
      const int ls = 63 - (int)(bits & 0x3Fu);
      const int e = 128 * eh + (((ls >> 2) << 3) | (h << 2) | (ls & 3));
      top[j] = __uint_as_float((bits & 0xFFFFFF00u) | (uint32_t)(255 - e));
    }
    float other[K];
#pragma unroll
    for (int j = 0; j < K; ++j) other[j] = __shfl_xor(top[j], 32);
#pragma unroll
    for (int j = 0; j < K; ++j) topk_insert<K>(top, other[j]);
    if (h == 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) xkey[(wave * 32 + l32) * 8 + j] = top[j];
    }
    float m = -__builtin_inff(), sum = 0.0f;
    if constexpr (EXTRA) {
      if (logits != nullptr && t < T) {
#pragma unroll
        for (int mb = 0; mb < kMBw; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ee = 128 * eh + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (ee < n_experts) logits[t * n_experts + ee] = acc[mb][nb][r];
          }
      }
      if (lse != nullptr) {
        // This wave's partial over its 128 experts (the lane's 64 merged with lane ^ 32's).
#pragma unroll
        for (int mb = 0; mb < kMBw; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ee = 128 * eh + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (ee < n_experts) m = fmaxf(m, acc[mb][nb][r]);
          }
#pragma unroll
        for (int mb = 0; mb < kMBw; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ee = 128 * eh + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (ee < n_experts) sum += __builtin_amdgcn_exp2f((acc[mb][nb][r] - m) * kLog2e);
          }
        const float m2 = __shfl_xor(m, 32);
        const float sum2 = __shfl_xor(sum, 32);
        const float mm = fmaxf(m, m2);
        // An empty half (every expert past n_experts) has m = -inf and contributes nothing.
        sum = (m == mm ? sum : sum * __builtin_amdgcn_exp2f((m - mm) * kLog2e)) +
              (m2 == mm ? sum2 : sum2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e));
        m = mm;
        if (h == 0) xlse[wave * 32 + l32] = float2{m, sum};
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    bare_barrier();  // parks, keys and partials of every wave are visible
    if (eh == (nb & 1)) {
      const int partner = wave ^ 1;
#pragma unroll
      for (int j = 0; j < K; ++j) topk_insert<K>(top, xkey[(partner * 32 + l32) * 8 + j]);
      if (t < T) {
        int e[K];
        float sg[K];
        float ssum = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
          e[j] = 255 - (int)(__float_as_uint(top[j]) & 0xFFu);
          const int el = e[j] & 127;
          const float* const pk = park_of(2 * tq + (e[j] >> 7));
          sg[j] = pk[(((el >> 5) * 4 + ((el & 31) >> 3)) * 64 + l32 + 32 * ((el >> 2) & 1)) * 4 + (el & 3)];
          ssum += sg[j];
        }
        if (h == 0) {
          if constexpr (K == 4) {
            *reinterpret_cast<i32x4*>(idx_out + t * 4) = i32x4{e[0], e[1], e[2], e[3]};
          } else {
#pragma unroll
            for (int j = 0; j < K; ++j) idx_out[t * K + j] = e[j];
          }
#pragma unroll
          for (int j = 0; j < K; ++j) atomicAdd(&hist[e[j]], 1);
        } else {
          const float inv = normalize ? 1.0f / ssum : 1.0f;
          if constexpr (K == 4) {
            *reinterpret_cast<f32x4*>(gates_out + t * 4) = f32x4{sg[0] * inv, sg[1] * inv, sg[2] * inv, sg[3] * inv};
          } else {
#pragma unroll
            for (int j = 0; j < K; ++j) gates_out[t * K + j] = sg[j] * inv;
          }
        }
        if constexpr (EXTRA) {
          if (lse != nullptr && h == 0) {
            const float2 o = xlse[partner * 32 + l32];
            const float mm = fmaxf(m, o.x);
            const float tot = (m == mm ? sum : sum * __builtin_amdgcn_exp2f((m - mm) * kLog2e)) +
                              (o.x == mm ? o.y : o.y * __builtin_amdgcn_exp2f((o.x - mm) * kLog2e));
            lse[t] = mm + __logf(tot);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    bare_barrier();  // the parks and keys are read before the next block overwrites them
  }
}

// NB: 32-token blocks per wave pair (tile of 128 NB tokens).  8 waves, two per SIMD: each pair
// shares a token range, and each wave of it holds 128 of the 256 experts.
template <int K, bool FULL, bool EXTRA, int NB, int TG>
__global__ __launch_bounds__(TG * 128) __attribute__((amdgpu_waves_per_eu(2, 2))) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias, int64_t T, int d,
    int n_experts, int normalize, int32_t* __restrict__ idx_out, float* __restrict__ gates_out,
    int32_t* __restrict__ counts, float* __restrict__ logits, float* __restrict__ lse,
    int32_t* __restrict__ tile_loads, int64_t loads_stride) {
  // The five ring slots are the whole LDS; the epilogue reuses them once the ring drains.
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[kSlot], xs1[kSlot], xs2[kSlot];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[kSlot], ws1[kSlot];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps LDS bases in SGPRs
  constexpr int kTok = TG * 32 * NB;  // tokens per workgroup
  const int64_t row0 = (int64_t)blockIdx.x * kTok;
  const int rows = (int)(T - row0 < kTok ? T - row0 : kTok);

  // Bias loads go first: a load issued behind the DMA prologue would have to wait for it.
  // Each wave reads all of b (4 values per lane) to form min b without any LDS.
  float bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bq[c] = lane + 64 * c < n_experts ? bias[lane + 64 * c] : __builtin_inff();

  // ---- operand streams: start the DMA ring (A = weights, B = this tile's tokens) ----
  const uint32_t row_bytes = (uint32_t)d * 2u;
  Stream<kAuxCached, kAuxStream, RowsK, RowsK, NB, 2, TG == kWaves, TG> st;
  st.init(w, (uint32_t)n_experts * row_bytes, row_bytes, x + row0 * d, (uint32_t)rows * row_bytes, row_bytes,
          d / kBK, wave, lane, Slots{xs0, xs1, xs2, ws0, ws1});
  st.prologue();

  // ---- shifted bias b' = b + (1 - min b) >= 1, so every selection key is a positive float ----
  float mn = fminf(fminf(bq[0], bq[1]), fminf(bq[2], bq[3]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mn = fminf(mn, __shfl_xor(mn, off));
  const float shift = 1.0f - mn;  // identical in every wave: min is exact
  const float bv = tid < n_experts ? bias[tid] : 0.0f;

  f32x16 acc[kMB / 2][NB];
  st.run(acc, wave, lane);
  epilogue_split<K, FULL, EXTRA, NB>(acc, tid, wave, lane, row0, T, n_experts, normalize, bv + shift, xs0, xs1, xs2,
                                     ws0, ws1, idx_out, gates_out, logits, lse);

  int* const hist = reinterpret_cast<int*>(ws1 + 1024);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  bare_barrier();
  if (tid < n_experts) {
    const int n = hist[tid];
    if (n != 0) atomicAdd(&counts[tid], n);
    // This tile's loads for the dispatch scan (the full tile is the dispatch tile; the launcher
    // passes no table with the half tile).
    if (NB == kNB && tile_loads != nullptr) tile_loads[(int64_t)tid * loads_stride + blockIdx.x] = n;
  }
}

template <int K, bool FULL, int NB, int TG>
hipError_t launch_kfn(const RouterArgs& a, hipStream_t stream) {
  const int normalize = (a.flags & ELB_GATES_RAW) ? 0 : 1;
  constexpr int kTok = TG * 32 * NB;
  const dim3 grid((unsigned)((a.T + kTok - 1) / kTok));
  int32_t* const loads = NB == kNB ? a.tile_loads : nullptr;
  if (a.logits != nullptr || a.lse != nullptr)
    return launch_timed(router_mfma_kernel<K, FULL, true, NB, TG>, grid, dim3(TG * 128), 0, stream, nullptr, a.ev_stop,
                        (const uint16_t*)a.x, (const uint16_t*)a.w, a.bias, a.T, a.d, a.n_experts, normalize, a.idx,
                        a.gates, a.counts, a.logits, a.lse, loads, a.loads_stride);
  return launch_timed(router_mfma_kernel<K, FULL, false, NB, TG>, grid, dim3(TG * 128), 0, stream, nullptr, a.ev_stop,
                      (const uint16_t*)a.x, (const uint16_t*)a.w, a.bias, a.T, a.d, a.n_experts, normalize, a.idx,
                      a.gates, a.counts, a.logits, a.lse, loads, a.loads_stride);
}

template <int K, bool FULL>
hipError_t launch_kf(const RouterArgs& a, hipStream_t stream) {
  if (router_mfma_full_tile(a.T)) return launch_kfn<K, FULL, kNB, kWaves>(a, stream);
  // Half-size batches: 128-token tiles; below that 64-token tiles, so every CU still gets one.
  return a.T > (int64_t)(kTile / 4) * kCus ? launch_kfn<K, FULL, 1, kWaves>(a, stream)
                                           : launch_kfn<K, FULL, 1, 2>(a, stream);
}

template <int K>
hipError_t launch_k(const RouterArgs& a, hipStream_t stream) {
  return a.n_experts == kExp ? launch_kf<K, true>(a, stream) : launch_kf<K, false>(a, stream);
}

}  // namespace

static_assert(kTile == kDispatchTile, "the router's full tile must be the dispatch tile");

bool router_mfma_full_tile(int64_t T) { return T > (int64_t)(kTile / 2) * kCus; }

bool router_mfma_applies(const RouterArgs& a) {
  return a.dtype == ELB_BF16 && a.d % kBK == 0 && a.n_experts <= kExp && a.k >= 1 && a.k <= 8 &&
         (int64_t)a.d * 2 * kTile < (int64_t(1) << 30);
}

hipError_t launch_router_mfma(const RouterArgs& a, hipStream_t stream) {
  switch (a.k) {
    case 1: return launch_k<1>(a, stream);
    case 2: return launch_k<2>(a, stream);
    case 3: return launch_k<3>(a, stream);
    case 4: return launch_k<4>(a, stream);
    case 5: return launch_k<5>(a, stream);
    case 6: return launch_k<6>(a, stream);
    case 7: return launch_k<7>(a, stream);
    default: return launch_k<8>(a, stream);
  }
}

}  // namespace elb

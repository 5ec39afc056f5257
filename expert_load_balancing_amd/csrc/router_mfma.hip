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
//   instead: each wave pair 32 tokens; batches of at most 64 x 256 take 64-token tiles, where
//   waves 0-3 hold the product (two pairs of 32 tokens) and waves 4-7 only issue the DMAs.  Two
//   waves per SIMD let one wave's LDS reads and selection run under the other's MFMAs.
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
//   the selection key is an unsigned integer: a fixed-point code of v = s + b - min b in its
//   high 23 bits and an index in its low 8 bits, so integer max and med3 order keys exactly
//   like (s + b, -index).  The code is formed with one fma: with 2^E <= 1 + max b - min b <
//   2^(E+1) and scale = 2^(22-E), fl(s * scale + (b - min b) * scale + 2^23 + 1) lies in
//   [2^23, 2^24], where a float's mantissa bits are the integer itself; shifting the bit
//   pattern left by 8 drops the exponent and leaves the code, >= 1 (the code of an absent
//   expert is 0).  Codes resolve s + b to 2^(E-22): 2.4e-7 for a bias spread below 1,
//   under 1e-3 for any spread below 8191; closer calls go to the lower index.  Inside a lane
//   the index is the lane-local slot (ascending with the expert id); the K survivors are
//   re-keyed with 255 - expert before the cross-lane merge.  Insertion into a sorted top-K
//   list is one max plus K-1 med3.  The chosen experts' exact scores come back through LDS
//   for the gates.  Loads: LDS histogram, one global atomic per expert per workgroup.
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

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return __builtin_elementwise_max(a, b); }
// Median of three (one v_med3_u32).
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return umax(__builtin_elementwise_min(a, b), __builtin_elementwise_min(umax(a, b), c));
}

// Sorted (descending) top-K insertion: the new j-th largest is med3(old (j-1)-th, old j-th, x).
template <int K>
__device__ __forceinline__ void topk_insert(uint32_t (&top)[K], uint32_t x) {
#pragma unroll
  for (int j = K - 1; j > 0; --j) top[j] = umed3(top[j - 1], top[j], x);
  top[0] = umax(top[0], x);
}

// Selection scaling from the bias range (identical in every workgroup: min and max are exact).
// With 2^E <= 1 + (max b - min b) < 2^(E+1): scale = 2^(22-E), so that s * scale + (b - min b) *
// scale < 2^23 + 1 for every s in [0, 1].
__device__ __forceinline__ float key_scale(float bmin, float bmax) {
  const int E = (int)((__float_as_uint(1.0f + (bmax - bmin)) >> 23) & 0xFF) - 127;
  return __uint_as_float((uint32_t)(127 + 22 - E) << 23);
}

// Per-expert addend of the key fma: (b - min b) * scale + 2^23 + 1.
__device__ __forceinline__ float key_bias(float b, float bmin, float scale) {
  return (b - bmin) * scale + 8388609.0f;
}

// Key of score s (fixed-point code of s + b - min b, see the file header) with index bits id.
__device__ __forceinline__ uint32_t sel_key(float s, float scale, float kb, uint32_t id) {
  return (__float_as_uint(__builtin_fmaf(s, scale, kb)) << 8) | id;
}

__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Epilogue of the 8-wave tile.  Wave w holds experts 128 eh .. + 127 (eh = w % 2) of
// tokens 32 NB tq .. (tq = w / 2); a lane holds 64 of them for its token, lane ^ 32 the other 64.
// Per 32-token block: every wave selects its K best (keys as described at the top, a
// lane-local slot in the low bits, re-keyed with 255 - expert before the merges), parks its
// scores, and leaves its K keys (and, with EXTRA, its log-sum-exp partial) in LDS; after a
// barrier one wave of each pair (eh = block parity) merges the partner's K keys and writes the
// token's indices, gates and histogram counts.  The key addends (key_bias) are in scratch[0..1 KiB),
// the histogram in scratch[1..2 KiB), the exchanged keys and log-sum-exp partials after them
// (12 KiB in all); each wave parks its scores in its own 16 KiB region park[wave].
// The pointers carry the LDS address space, so that every access through them stays an LDS
// instruction (a generic pointer would make them flat accesses, which also count as vector
// memory operations and wait behind the DMAs in flight).
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
__device__ __forceinline__ lds_u8* to_lds(unsigned char* p) { return (lds_u8*)p; }

// This wave's park, the two parks of its wave pair (waves 2 tq and 2 tq + 1: the gate lookup
// reads one of them per expert half), and the scratch region.  All wave-uniform.
struct Parks {
  lds_u8* mine;
  lds_u8* pair[2];
  lds_u8* scratch;
};

// The per-wave park regions of a tile (8 of 16 KiB), chosen with wave-uniform selects.
__device__ __forceinline__ unsigned char* park_region(int v, unsigned char* p0, unsigned char* p1,
                                                      unsigned char* p2, unsigned char* p3, unsigned char* p4,
                                                      unsigned char* p5, unsigned char* p6, unsigned char* p7) {
  return v == 0 ? p0 : v == 1 ? p1 : v == 2 ? p2 : v == 3 ? p3 : v == 4 ? p4 : v == 5 ? p5 : v == 6 ? p6 : p7;
}

__device__ __forceinline__ Parks make_parks(int wave, unsigned char* scratch, unsigned char* p0, unsigned char* p1,
                                            unsigned char* p2, unsigned char* p3, unsigned char* p4,
                                            unsigned char* p5, unsigned char* p6, unsigned char* p7) {
  Parks k;
  k.mine = to_lds(park_region(wave, p0, p1, p2, p3, p4, p5, p6, p7));
  k.pair[0] = to_lds(park_region(wave & ~1, p0, p1, p2, p3, p4, p5, p6, p7));
  k.pair[1] = to_lds(park_region(wave | 1, p0, p1, p2, p3, p4, p5, p6, p7));
  k.scratch = to_lds(scratch);
  return k;
}

template <int K, bool FULL, bool EXTRA, int NB>
__device__ __forceinline__ void epilogue_split(const f32x16 (&acc)[kMB / 2][NB], int tid, int wave, int lane,
                                               int64_t row0, int64_t T, int n_experts, int normalize, float kbias, float kscale,
                                               const Parks& pk_lds, int32_t* __restrict__ idx_out,
                                               float* __restrict__ gates_out, float* __restrict__ logits,
                                               float* __restrict__ lse) {
  constexpr int kMBw = kMB / 2;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int eh = wave & 1, tq = wave >> 1;
  lds_u8* const scr = pk_lds.scratch;
  typedef __attribute__((address_space(3))) int lds_i32;
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  typedef __attribute__((address_space(3))) f32x4 lds_f4;
  lds_f32* const kb_lds = (lds_f32*)scr;
  lds_i32* const hist = (lds_i32*)(scr + 1024);
  lds_u32* const xkey = (lds_u32*)(scr + 2048);                   // [8 waves][32 tokens][8]
  lds_f32* const xlse = (lds_f32*)(scr + 2048 + 8 * 32 * 8 * 4);  // [8 waves][32 tokens][2]
  if (tid < kExp) {
    kb_lds[tid] = tid < n_experts ? kbias : 0.0f;
    hist[tid] = 0;
  }
  // Parks: wave v's scores in its region, [16 groups][64 lanes][4].
  lds_f32* const park = (lds_f32*)pk_lds.mine;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  bare_barrier();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t t = row0 + tq * (32 * NB) + nb * 32 + l32;
    uint32_t top[K];
#pragma unroll
    for (int j = 0; j < K; ++j) top[j] = 0u;
#pragma unroll
    for (int mb = 0; mb < kMBw; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e0 = 128 * eh + mb * 32 + g * 8 + 4 * h;
        const f32x4 kb = *(const lds_f4*)(kb_lds + e0);
        f32x4 sv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = sigmoid_fast(acc[mb][nb][g * 4 + r]);
          sv[r] = sc;
          const uint32_t slot_id = (uint32_t)(63 - (mb * 16 + g * 4 + r));  // lane-local, ascending expert
          const uint32_t key = sel_key(sc, kscale, kb[r], slot_id);
          topk_insert<K>(top, FULL || e0 + r < n_experts ? key : 0u);
        }
        *(lds_f4*)(park + ((mb * 4 + g) * 64 + lane) * 4) = sv;
      }
    }
    // Re-key with the global expert id, merge with lane ^ 32 (the wave's other 64 experts).
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t bits = top[j];
      const int ls = 63 - (int)(bits & 0x3Fu);
      const int e = 128 * eh + (((ls >> 2) << 3) | (h << 2) | (ls & 3));
      top[j] = (bits & 0xFFFFFF00u) | (uint32_t)(255 - e);
    }
    uint32_t other[K];
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
        if (h == 0) {
          xlse[(wave * 32 + l32) * 2] = m;
          xlse[(wave * 32 + l32) * 2 + 1] = sum;
        }
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
          e[j] = 255 - (int)(top[j] & 0xFFu);
          const int el = e[j] & 127;
          const lds_f32* const pk = (const lds_f32*)((e[j] >> 7) ? pk_lds.pair[1] : pk_lds.pair[0]);
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
          for (int j = 0; j < K; ++j) __hip_atomic_fetch_add(&hist[e[j]], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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
            const float2 o{xlse[(partner * 32 + l32) * 2], xlse[(partner * 32 + l32) * 2 + 1]};
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

// The ring slots fill the LDS; the epilogue reuses them once the ring drains.  The full tile
// (NB = 2): tokens 3 x 32 KiB, weights 2 x 32 KiB.  The smaller tiles have shorter stages and
// take deeper rings: 128 tokens 4 x 16 KiB + 3 x 32 KiB, 64 tokens 4 x 8 KiB + 4 x 32 KiB.  Each
// kernel branch below declares exactly the slots its Ring names (checked at compile time: a
// slot left out would be a null LDS address).
template <int NB, int TG>
struct Ring {
  static constexpr int NXR = NB == kNB ? kNX : 4;
  static constexpr int NWR = NB == kNB ? kNW : (TG == kWaves ? 3 : 4);
};

// NB: 32-token blocks per wave pair (tile of 128 NB tokens).  8 waves, two per SIMD: each pair
// shares a token range, and each wave of it holds 128 of the 256 experts.
template <int K, bool FULL, bool EXTRA, int NB, int TG>
__device__ __forceinline__ void router_body(Slots slots, Parks pk,
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias, int64_t T, int d,
    int n_experts, int normalize, int32_t* __restrict__ idx_out, float* __restrict__ gates_out,
    int32_t* __restrict__ counts, float* __restrict__ logits, float* __restrict__ lse,
    int32_t* __restrict__ tile_loads, int64_t loads_stride) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps LDS bases in SGPRs
  constexpr int kTok = TG * 32 * NB;  // tokens per workgroup
  const int64_t row0 = (int64_t)blockIdx.x * kTok;
  const int rows = (int)(T - row0 < kTok ? T - row0 : kTok);

  // Bias loads go first: a load issued behind the DMA prologue would have to wait for it.
  // Each wave reads all of b (4 values per lane) to form min b and max b without any LDS.
  float bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bq[c] = lane + 64 * c < n_experts ? bias[lane + 64 * c] : __builtin_nanf("");
  const float braw = tid < n_experts ? bias[tid] : 0.0f;

  // ---- operand streams: start the DMA ring (A = weights, B = this tile's tokens) ----
  const uint32_t row_bytes = (uint32_t)d * 2u;
  Stream<kAuxCached, kAuxStream, RowsK, RowsK, NB, 2, true, TG, Ring<NB, TG>::NXR, Ring<NB, TG>::NWR> st;
  st.init(w, (uint32_t)n_experts * row_bytes, row_bytes, x + row0 * d, (uint32_t)rows * row_bytes, row_bytes,
          d / kBK, wave, lane, slots);
  // Rows a multiple of 4 KiB apart: every workgroup's rows share their low 12 address bits, so
  // workgroups in step would all read the same columns at once, which concentrates the traffic on
  // a few memory channels (the token stream alone ran at 5.4 instead of 7 TB/s at d = 4096).
  // Each workgroup starts its k loop at another stage instead.
  if (row_bytes % 4096u == 0) st.rot = (int)(blockIdx.x % (uint32_t)(d / kBK));
  st.prologue();

  f32x16 acc[kMB / 2][NB];
  st.run(acc, wave, lane);

  // ---- selection key scaling from min b and max b (fminf / fmaxf skip the NaN padding) ----
  // Only the epilogue needs it: done after the main loop, so that no wait for the bias loads
  // drains the DMA prologue (the loads were issued first and landed long ago).
  float mn = fminf(fminf(bq[0], bq[1]), fminf(bq[2], bq[3]));
  float mx = fmaxf(fmaxf(bq[0], bq[1]), fmaxf(bq[2], bq[3]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  const float kscale = key_scale(mn, mx);  // identical in every wave: min and max are exact
  const float kbias = tid < n_experts ? key_bias(braw, mn, kscale) : 0.0f;
  if (TG == kWaves || wave < kWaves) {
    epilogue_split<K, FULL, EXTRA, NB>(acc, tid, wave, lane, row0, T, n_experts, normalize, kbias, kscale, pk,
                                       idx_out, gates_out, logits, lse);
  } else {
    // The DMA-only waves of the 64-token tile hold no scores: they pass the epilogue's barriers.
#pragma unroll
    for (int i = 0; i < 1 + 2 * NB; ++i) bare_barrier();
  }

  __attribute__((address_space(3))) int* const hist = (__attribute__((address_space(3))) int*)(pk.scratch + 1024);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  bare_barrier();
  if (tid < n_experts) {
    const int n = hist[tid];
    // No counts in a routed step with dispatch: the dispatch scan sums the tile loads into them.
    if (counts != nullptr && n != 0) atomicAdd(&counts[tid], n);
    // This tile's loads for the dispatch scan (the full tile is the dispatch tile; the launcher
    // passes no table with the half tile).
    if (NB == kNB && tile_loads != nullptr) tile_loads[(int64_t)tid * loads_stride + blockIdx.x] = n;
  }
  // Filling the table also resets the totals the dispatch scan will flag.
  if (NB == kNB && tile_loads != nullptr && blockIdx.x == 0 && tid < n_experts)
    tile_loads[loads_stride * n_experts + tid] = 0;
}

template <int K, bool FULL, bool EXTRA, int NB, int TG>
__global__ __launch_bounds__(kWaves * 128) __attribute__((amdgpu_waves_per_eu(2, 2))) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias, int64_t T, int d,
    int n_experts, int normalize, int32_t* __restrict__ idx_out, float* __restrict__ gates_out,
    int32_t* __restrict__ counts, float* __restrict__ logits, float* __restrict__ lse,
    int32_t* __restrict__ tile_loads, int64_t loads_stride) {
  // Each tile declares its own ring slots (distinct arrays: the compiler tracks which DMA fills
  // which slot), then the score parks (16 KiB per wave) and the epilogue's scratch in slots the
  // drained ring leaves.
  constexpr int XS = 32 * TG * NB * kRowB;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (NB == kNB) {
    static_assert(Ring<NB, TG>::NXR == 3 && Ring<NB, TG>::NWR == 2, "the slots declared here");
    __shared__ __attribute__((aligned(1024))) unsigned char xs0[XS], xs1[XS], xs2[XS], ws0[kSlot], ws1[kSlot];
    router_body<K, FULL, EXTRA, NB, TG>(
        Slots{xs0, xs1, xs2, ws0, ws1},
        make_parks(wave, ws1, xs0, xs0 + 16384, xs1, xs1 + 16384, xs2, xs2 + 16384, ws0, ws0 + 16384), x, w, bias, T, d,
        n_experts, normalize, idx_out, gates_out, counts, logits, lse, tile_loads, loads_stride);
  } else if constexpr (TG == kWaves) {
    static_assert(Ring<NB, TG>::NXR == 4 && Ring<NB, TG>::NWR == 3, "the slots declared here");
    __shared__ __attribute__((aligned(1024))) unsigned char xs0[XS], xs1[XS], xs2[XS], xs3[XS];
    __shared__ __attribute__((aligned(1024))) unsigned char ws0[kSlot], ws1[kSlot], ws2[kSlot];
    router_body<K, FULL, EXTRA, NB, TG>(
        Slots{xs0, xs1, xs2, ws0, ws1, xs3, ws2},
        make_parks(wave, xs2, ws0, ws0 + 16384, ws1, ws1 + 16384, ws2, ws2 + 16384, xs0, xs1), x, w, bias, T, d,
        n_experts, normalize, idx_out, gates_out, counts, logits, lse, tile_loads, loads_stride);
  } else {
    static_assert(Ring<NB, TG>::NXR == 4 && Ring<NB, TG>::NWR == 4, "the slots declared here");
    __shared__ __attribute__((aligned(1024))) unsigned char xs0[XS], xs1[XS], xs2[XS], xs3[XS];
    __shared__ __attribute__((aligned(1024))) unsigned char ws0[kSlot], ws1[kSlot], ws2[kSlot], ws3[kSlot];
    router_body<K, FULL, EXTRA, NB, TG>(
        Slots{xs0, xs1, xs2, ws0, ws1, xs3, ws2, ws3},
        make_parks(wave, ws2, ws0, ws0 + 16384, ws1, ws1 + 16384, ws0, ws0, ws0, ws0), x, w, bias, T, d,
        n_experts, normalize, idx_out, gates_out, counts, logits, lse, tile_loads, loads_stride);
  }
}

template <int K, bool FULL, int NB, int TG>
hipError_t launch_kfn(const RouterArgs& a, hipStream_t stream) {
  const int normalize = (a.flags & ELB_GATES_RAW) ? 0 : 1;
  constexpr int kTok = TG * 32 * NB;
  const dim3 grid((unsigned)((a.T + kTok - 1) / kTok));
  int32_t* const loads = NB == kNB ? a.tile_loads : nullptr;
  if (a.logits != nullptr || a.lse != nullptr)
    return launch_timed(router_mfma_kernel<K, FULL, true, NB, TG>, grid, dim3(kWaves * 128), 0, stream, nullptr, a.ev_stop,
                        (const uint16_t*)a.x, (const uint16_t*)a.w, a.bias, a.T, a.d, a.n_experts, normalize, a.idx,
                        a.gates, a.counts, a.logits, a.lse, loads, a.loads_stride);
  return launch_timed(router_mfma_kernel<K, FULL, false, NB, TG>, grid, dim3(kWaves * 128), 0, stream, nullptr, a.ev_stop,
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

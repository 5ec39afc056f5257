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
//   One workgroup (4 waves, one per SIMD) owns a tile of 256 tokens x all 256 experts and
//   keeps the 256x256 fp32 logit tile in registers (each wave: 256 experts x 64 tokens = 16
//   accumulators of 32x32).  The contraction is written transposed, Z^T = W . X^T, so that the
//   32x32 MFMA output puts one token per lane column: a lane ends up holding 128 of the 256
//   logits of each of its tokens, and the other 128 sit in lane ^ 32.  Top-K therefore needs
//   no LDS round trip: a register-local selection over 128 values, then one cross-lane merge.
//
// Memory pipeline (per 64-element slice of d, "stage"):
//   global -> VGPR (16-byte buffer loads, 8 consecutive lanes read one 128-byte row segment,
//   so every HBM line is fully used; rows past T or past N_r come back as zeros from the
//   buffer range check) -> LDS (two stages, rows XOR-swizzled in 16-byte chunks so both the
//   stores and the MFMA operand reads are bank-conflict free) -> MFMA operands.
//   The loads for stage k+2 are issued right after stage k+1 is written to LDS, so they fly
//   during the 64 MFMAs of stage k+1; barriers fence LDS only (see lds_barrier).
//
// Epilogue (per lane, per token): s = 1 / (1 + 2^(-z log2 e)) with the hardware exp2/rcp;
//   the selection key is the fp32 bit pattern of s + b' with its low 8 bits replaced by
//   255 - i, where b' = b + (1 - min b) >= 1 keeps every key a positive float, so float
//   max / med3 order keys exactly like (s + b, -i).  Keeping 24 bits of s + b' resolves
//   differences down to 2^-15 (1 + max b - min b); closer calls fall to the lower index.
//   Insertion into a sorted top-K list is one max plus K-1 med3.  The chosen experts' exact
//   scores come back through LDS for the gates.  Loads: LDS histogram, one global atomic per
//   expert per workgroup.
#include "device_common.hpp"
#include "elb_kernels.h"

#include "../../include/elb.h"

namespace elb {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kExp = 256;                        // experts per tile (padded)
constexpr int kMB = kExp / 32;                   // 32-row MFMA blocks of experts
constexpr int kTokWave = 64;                     // tokens per wave
constexpr int kNB = kTokWave / 32;               // 32-column MFMA blocks of tokens
constexpr int kTile = kWaves * kTokWave;         // tokens per workgroup
constexpr int kBK = 64;                          // d elements per stage
constexpr int kRowB = kBK * 2;                   // bytes of one row per stage
constexpr int kWBytes = kExp * kRowB;            // 32 KiB
constexpr int kXBytes = kTile * kRowB;           // 32 KiB
constexpr int kStage = kWBytes + kXBytes;        // 64 KiB
constexpr int kLoads = kWBytes / (kThreads * 16);  // 16-byte loads per thread per tensor
constexpr int kRowsPerLoad = kThreads / 8;       // rows covered by one load instruction (32)
constexpr float kLog2e = 1.4426950408889634f;

static_assert(kLoads * kRowsPerLoad == kExp && kXBytes == kWBytes, "load mapping");
static_assert(kWaves * 32768 <= 2 * kStage, "per-wave score slices must fit in the stage buffers");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer: stride 0, range checked against `bytes`; out-of-range loads return zeros.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}

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

template <int K, bool EXTRA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias, int64_t T, int d,
    int n_experts, int normalize, int32_t* __restrict__ idx_out, float* __restrict__ gates_out,
    int32_t* __restrict__ counts, float* __restrict__ logits, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];
  __shared__ __attribute__((aligned(16))) float bprime[kExp];
  __shared__ int hist[kExp];
  __shared__ float wave_min[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int64_t row0 = (int64_t)blockIdx.x * kTile;
  const int rows = (int)(T - row0 < kTile ? T - row0 : kTile);

  // ---- shifted bias b' = b + (1 - min b) >= 1, so every selection key is a positive float ----
  const float bv = tid < n_experts ? bias[tid] : __builtin_inff();
  float mn = bv;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mn = fminf(mn, __shfl_xor(mn, off));
  if (lane == 0) wave_min[wave] = mn;
  hist[tid] = 0;
  lds_barrier();
  const float shift = 1.0f - fminf(fminf(wave_min[0], wave_min[1]), fminf(wave_min[2], wave_min[3]));
  bprime[tid] = tid < n_experts ? bv + shift : 0.0f;  // visible after the first main-loop barrier

  // ---- operand streams ----
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + row0 * d, (uint32_t)rows * row_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)n_experts * row_bytes);
  const int lrow = tid >> 3;  // row within a 32-row group
  const int lc = tid & 7;     // 16-byte chunk within the 128-byte row segment
  const uint32_t goff = (uint32_t)lrow * row_bytes + (uint32_t)lc * 16u;
  const uint32_t gstep = (uint32_t)kRowsPerLoad * row_bytes;
  const uint32_t soff = (uint32_t)lrow * kRowB + (uint32_t)((lc ^ (lrow & 7)) << 4);
  constexpr uint32_t sstep = kRowsPerLoad * kRowB;  // 4 KiB

  u32x4 rw[kLoads], rx[kLoads];
  auto gload = [&](int kb) {
    const uint32_t ko = (uint32_t)kb * kRowB;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) rw[i] = load16(wr, goff + i * gstep + ko);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) rx[i] = load16(xr, goff + i * gstep + ko);
  };
  auto swrite = [&](int buf) {
    unsigned char* base = smem + buf * kStage + soff;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) *reinterpret_cast<u32x4*>(base + i * sstep) = rw[i];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) *reinterpret_cast<u32x4*>(base + kWBytes + i * sstep) = rx[i];
  };

  // Operand read offsets: row r = l32 (+32 per block), chunk 2s + h of the row segment.
  uint32_t fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = (uint32_t)l32 * kRowB + (uint32_t)((((2 * s + h) ^ (l32 & 7))) << 4);
  const uint32_t xo = kWBytes + (uint32_t)wave * (kTokWave * kRowB);

  f32x16 acc[kMB][kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  const int nkb = d / kBK;
  gload(0);
  swrite(0);
  if (nkb > 1) gload(1);
  lds_barrier();
  for (int kb = 0; kb < nkb; ++kb) {
    const unsigned char* sb = smem + (kb & 1) * kStage;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[kMB], b[kNB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) a[mb] = *reinterpret_cast<const bf16x8*>(sb + fo[s] + mb * (32 * kRowB));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) b[nb] = *reinterpret_cast<const bf16x8*>(sb + xo + fo[s] + nb * (32 * kRowB));
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
    }
    if (kb + 1 < nkb) {
      swrite((kb + 1) & 1);
      if (kb + 2 < nkb) gload(kb + 2);
    }
    lds_barrier();
  }

  // ---- epilogue ----
  // Output layout of a 32x32 MFMA block (rows = experts, columns = tokens): lane column
  // l32 is the token; accumulator r holds expert row 8 (r / 4) + 4 h + (r % 4).
  // The stage buffers are free now (every wave passed the last barrier); each wave parks
  // its scores in its own 32 KiB slice: [32 row groups][64 lanes][4 floats].
  float* sbuf = reinterpret_cast<float*>(smem + wave * 32768);
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int64_t t = row0 + wave * kTokWave + nb * 32 + l32;
    float top[K];
#pragma unroll
    for (int j = 0; j < K; ++j) top[j] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e0 = mb * 32 + g * 8 + 4 * h;
        const f32x4 bp = *reinterpret_cast<const f32x4*>(bprime + e0);
        f32x4 sv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = sigmoid_fast(acc[mb][nb][g * 4 + r]);
          sv[r] = s;
          const uint32_t bits = (__float_as_uint(s + bp[r]) & 0xFFFFFF00u) | (uint32_t)(255 - (e0 + r));
          topk_insert<K>(top, e0 + r < n_experts ? __uint_as_float(bits) : 0.0f);
        }
        *reinterpret_cast<f32x4*>(sbuf + ((mb * 4 + g) * 64 + lane) * 4) = sv;
      }
    }
    // Merge with lane ^ 32, which holds the other 128 experts of the same token.
    float other[K];
#pragma unroll
    for (int j = 0; j < K; ++j) other[j] = __shfl_xor(top[j], 32);
#pragma unroll
    for (int j = 0; j < K; ++j) topk_insert<K>(top, other[j]);
    wave_lds_sync();

    if (t < T) {
      int e[K];
      float sg[K];
      float ssum = 0.0f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        e[j] = 255 - (int)(__float_as_uint(top[j]) & 0xFFu);
        const int src_lane = l32 + 32 * ((e[j] >> 2) & 1);
        sg[j] = sbuf[((e[j] >> 3) * 64 + src_lane) * 4 + (e[j] & 3)];
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
    }

    if constexpr (EXTRA) {
      if (logits != nullptr && t < T) {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (e < n_experts) logits[t * n_experts + e] = acc[mb][nb][r];
          }
      }
      if (lse != nullptr) {
        float m = -__builtin_inff();
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (e < n_experts) m = fmaxf(m, acc[mb][nb][r]);
          }
        float sum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (e < n_experts) sum += __builtin_amdgcn_exp2f((acc[mb][nb][r] - m) * kLog2e);
          }
        const float m2 = __shfl_xor(m, 32);
        const float sum2 = __shfl_xor(sum, 32);
        const float mm = fmaxf(m, m2);
        const float tot = sum * __builtin_amdgcn_exp2f((m - mm) * kLog2e) + sum2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e);
        if (h == 0 && t < T) lse[t] = mm + __logf(tot);
      }
    }
  }

  lds_barrier();
  if (tid < n_experts && hist[tid] != 0) atomicAdd(&counts[tid], hist[tid]);
}

template <int K>
hipError_t launch_k(const RouterArgs& a, hipStream_t stream) {
  const int normalize = (a.flags & ELB_GATES_RAW) ? 0 : 1;
  const dim3 grid((unsigned)((a.T + kTile - 1) / kTile));
  if (a.logits != nullptr || a.lse != nullptr)
    return launch(router_mfma_kernel<K, true>, grid, dim3(kThreads), 0, stream, (const uint16_t*)a.x,
                  (const uint16_t*)a.w, a.bias, a.T, a.d, a.n_experts, normalize, a.idx, a.gates, a.counts,
                  a.logits, a.lse);
  return launch(router_mfma_kernel<K, false>, grid, dim3(kThreads), 0, stream, (const uint16_t*)a.x,
                (const uint16_t*)a.w, a.bias, a.T, a.d, a.n_experts, normalize, a.idx, a.gates, a.counts,
                a.logits, a.lse);
}

}  // namespace

bool router_mfma_applies(const RouterArgs& a) {
  return a.dtype == ELB_BF16 && a.d % kBK == 0 && a.n_experts <= kExp && a.k >= 1 && a.k <= 8 &&
         (int64_t)a.d * 2 * kExp < (1ll << 31);
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

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
// Memory pipeline: d is consumed in stages of 64 elements (128 bytes of every row: every
//   tile row costs HBM one full line per visit; 64-byte visits stream markedly slower because
//   all workgroups touch 256 rows 2*d bytes apart at once).  Rows go from HBM (tokens) or L2
//   (router weights) straight into LDS with buffer-to-LDS DMA loads, which need no registers:
//   the token stream runs 2 stages ahead in a ring of 3 LDS slots, the weight stream 1 stage
//   ahead in a ring of 2 (weights come from L2, well within one stage).  The five 32 KiB slots
//   fill the 160 KiB LDS.  Rows past T or past N_r fall outside the buffer range and arrive as
//   zeros.  Every wave waits for its own DMAs with an explicit vmcnt budget, then one barrier
//   per stage publishes the slot to all waves and frees the slot the next DMA overwrites.
//   Barriers carry no memory fence: a fence on LDS would wait for every DMA in flight and
//   drain the prefetch.  Near the end, out-of-range dummy DMAs keep the vmcnt budget uniform;
//   they move no HBM bytes.  Within a slot, the eight 16-byte chunks of row r sit at
//   chunk ^ ((r >> 1) & 7), which keeps the MFMA operand reads (16 rows x 16 bytes per LDS
//   cycle over 64 banks) free of bank conflicts.
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

#include "../../include/elb.h"

namespace elb {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kExp = 256;                 // experts per tile (padded)
constexpr int kMB = kExp / 32;            // 32-row MFMA blocks of experts
constexpr int kTokWave = 64;              // tokens per wave
constexpr int kNB = kTokWave / 32;        // 32-column MFMA blocks of tokens
constexpr int kTile = kWaves * kTokWave;  // tokens per workgroup
constexpr int kBK = 64;                   // d elements per stage
constexpr int kRowB = kBK * 2;            // bytes of one row per stage
constexpr int kSlot = 256 * kRowB;        // one stage of 256 rows: 32 KiB
constexpr int kNX = 3, kPX = 2;           // token ring: slots, stages in flight
constexpr int kNW = 2, kPW = 1;           // weight ring
constexpr int kUnroll = 6;                // lcm(kNX, kNW): slots are compile-time constants
constexpr int kKSteps = kBK / 16;         // MFMA k-steps per stage
// The compiler tracks at most 8 distinct LDS DMA targets when it decides which DMAs an LDS
// read must wait for; with more slots it would fall back to waiting for all of them.
static_assert(kNX + kNW <= 8, "at most 8 DMA target slots");
static_assert((kNX + kNW) * kSlot <= 160 * 1024, "LDS");
constexpr int kDma = kSlot / (kWaves * 1024);  // DMA instructions per wave per slot (1 KiB each)
constexpr float kLog2e = 1.4426950408889634f;

static_assert(kNX == kPX + 1 && kNW == kPW + 1 && kUnroll % kNX == 0 && kUnroll % kNW == 0, "ring shape");
static_assert(kPX >= kPW, "the vmcnt budget below assumes the token stream runs further ahead");
// VMEM instructions a wave issues after the DMAs of stage j's weights, when it must have stage j:
// the token DMAs of the same iteration, then (kPW - 1) full iterations.
constexpr int kVmBudget = kDma + 2 * kDma * (kPW - 1);

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 63 & 15 | (3 << 14) | (7 << 4);  // lgkmcnt(0) only

__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer: stride 0, range checked against `bytes`; out-of-range loads return zeros.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

#define ELB_AS3(p) ((__attribute__((address_space(3))) void*)(p))

// Cache policy of the DMAs: the token rows are read exactly once, so they go non-temporal
// (nt): streaming them through the caches with normal allocation costs the L2-resident router
// weights their place and the whole memory pipeline ~20% of its rate.
constexpr int kAuxTokens = 2;   // nt
constexpr int kAuxWeights = 0;  // default: keep the weights cached

// One wave's share of one slot: kDma 1-KiB DMA instructions (8 rows each).  A dummy DMA (past
// the last stage) keeps the vmcnt budget uniform: it goes through `none`, a descriptor with an
// empty range, so it reads zeros and moves no bytes.  The choice is a scalar select of the
// descriptor; the row offsets stay in their own registers.  (Selecting the offset per DMA
// instead put a VALU write to one shared register before every DMA, which stalls behind the
// previous DMA's operand read whenever the vector memory queue is full, and with it every
// MFMA queued behind.)
template <int AUX>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, __amdgpu_buffer_rsrc_t none,
                                         unsigned char* wave_base, const uint32_t (&vo)[kDma], uint32_t soff,
                                         bool real) {
  const __amdgpu_buffer_rsrc_t use = real ? r : none;
#pragma unroll
  for (int i = 0; i < kDma; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(use, ELB_AS3(wave_base + i * 1024), 16, vo[i], (int)soff, 0, AUX);
}

// LDS position of 16-byte chunk c of a 128-byte row segment r.  The LDS serves 16 lanes x 16
// bytes per cycle from 64 banks; an MFMA operand read has 16 consecutive rows read the same
// chunk, and XOR-ing the chunk with bits 1..3 of the row spreads those 16 reads over the
// whole 256-byte bank window (rows r and r + 1 already sit in different 128-byte halves).
__device__ __forceinline__ constexpr int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

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

template <int K, bool FULL, bool EXTRA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias, int64_t T, int d,
    int n_experts, int normalize, int32_t* __restrict__ idx_out, float* __restrict__ gates_out,
    int32_t* __restrict__ counts, float* __restrict__ logits, float* __restrict__ lse,
    int32_t* __restrict__ tile_loads, int64_t loads_stride) {
  // The five ring slots are the whole LDS; the epilogue reuses them once the ring drains.
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[kSlot], xs1[kSlot], xs2[kSlot];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[kSlot], ws1[kSlot];
  auto xslot = [&](int i) -> unsigned char* { return i == 0 ? xs0 : i == 1 ? xs1 : xs2; };
  auto wslot = [&](int i) -> unsigned char* { return i == 0 ? ws0 : ws1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps LDS bases in SGPRs
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int64_t row0 = (int64_t)blockIdx.x * kTile;
  const int rows = (int)(T - row0 < kTile ? T - row0 : kTile);
  const int nkb = d / kBK;

  // Bias loads go first: a load issued behind the DMA prologue would have to wait for it.
  // Each wave reads all of b (4 values per lane) to form min b without any LDS.
  float bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bq[c] = lane + 64 * c < n_experts ? bias[lane + 64 * c] : __builtin_inff();

  // ---- operand streams: start the DMA ring ----
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + row0 * d, (uint32_t)rows * row_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)n_experts * row_bytes);
  const __amdgpu_buffer_rsrc_t none = make_rsrc(w, 0u);
  // DMA lane mapping: instruction i of wave `wave` fills rows wave*64 + 8 i + lane/8; lane
  // position p = lane & 7 in the row receives the global chunk stored there, swz(row, p)
  // (the swizzle is its own inverse).
  uint32_t vo[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int r = wave * 64 + 8 * i + (lane >> 3);
    vo[i] = (uint32_t)r * row_bytes + (uint32_t)(swz(r, lane & 7) << 4);
  }
  const uint32_t wave_off = (uint32_t)wave * (64 * kRowB);
  // Prologue: stages 0..kPX-1 of the tokens and 0..kPW-1 of the weights, issued in the same
  // order the steady state uses (weights first, then tokens, per virtual iteration).
#pragma unroll
  for (int vi = -kPX; vi < 0; ++vi) {
    if (vi + kPW >= 0) dma_rows<kAuxWeights>(wr, none, wslot((vi + kPW) % kNW) + wave_off, vo, (uint32_t)(vi + kPW) * kRowB, vi + kPW < nkb);
    dma_rows<kAuxTokens>(xr, none, xslot((vi + kPX) % kNX) + wave_off, vo, (uint32_t)(vi + kPX) * kRowB, vi + kPX < nkb);
  }

  // ---- shifted bias b' = b + (1 - min b) >= 1, so every selection key is a positive float ----
  float mn = fminf(fminf(bq[0], bq[1]), fminf(bq[2], bq[3]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mn = fminf(mn, __shfl_xor(mn, off));
  const float shift = 1.0f - mn;  // identical in every wave: min is exact
  const float bv = tid < n_experts ? bias[tid] : 0.0f;

  // Operand reads: row r = l32 (+32 per block), chunk 2s + h of the 128-byte row segment.
  uint32_t fo[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) fo[s] = (uint32_t)l32 * kRowB + (uint32_t)(swz(l32, 2 * s + h) << 4);
  const uint32_t xo = (uint32_t)wave * (kTokWave * kRowB);

  f32x16 acc[kMB][kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // nkb >= 1 always (d >= kBK): a do-while tells the compiler so, and spares it a second,
  // never-run copy of the 256 zero accumulators held across the loop.
  int j0 = 0;
  do {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = j0 + u;
      if (j >= nkb) break;
      // Own DMAs of stage j are done; after the barrier everyone's are, and every wave has
      // finished reading stage j - 1, whose slots the DMAs below overwrite.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kVmBudget) & ~(15 << 8));  // and lgkmcnt(0)
      bare_barrier();
      // Weight DMAs at the head of the stage (they must precede this stage's token DMAs for
      // the vmcnt budget); the token DMAs are spread over the MFMA stream below, so that a
      // DMA waiting for room in the vector memory pipeline only delays MFMAs already queued.
      dma_rows<kAuxWeights>(wr, none, wslot((u + kPW) % kNW) + wave_off, vo, (uint32_t)(j + kPW) * kRowB, j + kPW < nkb);
      __builtin_amdgcn_sched_barrier(0);
      dma_rows<kAuxTokens>(xr, none, xslot((u + kPX) % kNX) + wave_off, vo, (uint32_t)(j + kPX) * kRowB, j + kPX < nkb);
      const unsigned char* ws = wslot(u % kNW);
      const unsigned char* xsb = xslot(u % kNX) + xo;
      // Operand fragments are double-buffered: the 10 LDS reads of k-step s + 1 go out before
      // the 16 MFMAs of k-step s, so their latency hides behind 512 MFMA cycles (one wave per
      // SIMD has no other wave to hide it).
      bf16x8 a[2][kMB], b[2][kNB];
      auto fetch = [&](int buf, int s) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          b[buf][nb] = *reinterpret_cast<const bf16x8*>(xsb + fo[s] + nb * (32 * kRowB));
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
          a[buf][mb] = *reinterpret_cast<const bf16x8*>(ws + fo[s] + mb * (32 * kRowB));
      };
      fetch(0, 0);
      fetch(1, 1);
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        if (s >= 1 && s + 1 < kKSteps) fetch((s + 1) & 1, s + 1);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][mb], b[s & 1][nb], acc[mb][nb], 0, 0, 0);
      }
      // Issue order for the scheduler: reads of steps 0 and 1; then per step its MFMAs with
      // kDma / kKSteps token DMAs slotted between them, and the reads of step s + 2.
      static_assert(kDma % kKSteps == 0 && (kMB * kNB) % (kDma / kKSteps) == 0, "DMA interleave");
      constexpr int kDmaPerStep = kDma / kKSteps;
      constexpr int kMfmaPerDma = kMB * kNB / kDmaPerStep;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (kMB + kNB), 0);  // DS reads, steps 0 and 1
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
#pragma unroll
        for (int q = 0; q < kDmaPerStep; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerDma, 0);  // MFMAs, step s
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);            // one token DMA
        }
        if (s + 2 < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, kMB + kNB, 0);  // DS reads, step s + 2
      }
    }
    j0 += kUnroll;
  } while (j0 < nkb);

  // ---- epilogue ----
  // Drain the trailing dummy DMAs (they write the slots reused below) and let every wave
  // finish its last operand reads; then slot ws1 holds b' and the load histogram, and each
  // wave parks its scores in a slot of its own: [32 row groups][64 lanes][4 floats].
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & ~(15 << 8));
  bare_barrier();
  float* const bprime = reinterpret_cast<float*>(ws1);
  int* const hist = reinterpret_cast<int*>(ws1 + 1024);
  bprime[tid] = tid < n_experts ? bv + shift : 0.0f;
  hist[tid] = 0;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  bare_barrier();
  float* const park = reinterpret_cast<float*>(wave == 0 ? xs0 : wave == 1 ? xs1 : wave == 2 ? xs2 : ws0);
  // Output layout of a 32x32 MFMA block (rows = experts, columns = tokens): lane column l32 is
  // the token; accumulator r holds expert row 8 (r / 4) + 4 h + (r % 4).
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
          const uint32_t slot_id = (uint32_t)(127 - (mb * 16 + g * 4 + r));  // lane-local, ascending expert
          const float key = __uint_as_float((__float_as_uint(s + bp[r]) & 0xFFFFFF00u) | slot_id);
          topk_insert<K>(top, FULL || e0 + r < n_experts ? key : 0.0f);
        }
        *reinterpret_cast<f32x4*>(park + ((mb * 4 + g) * 64 + lane) * 4) = sv;
      }
    }
    // Re-key the survivors with the global expert id, then merge with lane ^ 32, which holds
    // the other 128 experts of the same token.
    int e[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t bits = __float_as_uint(top[j]);
      const int ls = 127 - (int)(bits & 0x7Fu);
      e[j] = ((ls >> 2) << 3) | (h << 2) | (ls & 3);
      top[j] = __uint_as_float((bits & 0xFFFFFF00u) | (uint32_t)(255 - e[j]));
    }
    float other[K];
#pragma unroll
    for (int j = 0; j < K; ++j) other[j] = __shfl_xor(top[j], 32);
#pragma unroll
    for (int j = 0; j < K; ++j) topk_insert<K>(top, other[j]);
    wave_lds_sync();

    if (t < T) {
      float sg[K];
      float ssum = 0.0f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        e[j] = 255 - (int)(__float_as_uint(top[j]) & 0xFFu);
        const int src_lane = l32 + 32 * ((e[j] >> 2) & 1);
        sg[j] = park[((e[j] >> 3) * 64 + src_lane) * 4 + (e[j] & 3)];
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
            const int ee = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (ee < n_experts) logits[t * n_experts + ee] = acc[mb][nb][r];
          }
      }
      if (lse != nullptr) {
        float m = -__builtin_inff();
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ee = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (ee < n_experts) m = fmaxf(m, acc[mb][nb][r]);
          }
        float sum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ee = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (ee < n_experts) sum += __builtin_amdgcn_exp2f((acc[mb][nb][r] - m) * kLog2e);
          }
        const float m2 = __shfl_xor(m, 32);
        const float sum2 = __shfl_xor(sum, 32);
        const float mm = fmaxf(m, m2);
        const float tot =
            sum * __builtin_amdgcn_exp2f((m - mm) * kLog2e) + sum2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e);
        if (h == 0 && t < T) lse[t] = mm + __logf(tot);
      }
    }
  }

  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  bare_barrier();
  if (tid < n_experts) {
    const int n = hist[tid];
    if (n != 0) atomicAdd(&counts[tid], n);
    // This tile's loads for the dispatch scan (the workgroup is the dispatch tile).
    if (tile_loads != nullptr) tile_loads[(int64_t)tid * loads_stride + blockIdx.x] = n;
  }
}

template <int K, bool FULL>
hipError_t launch_kf(const RouterArgs& a, hipStream_t stream) {
  const int normalize = (a.flags & ELB_GATES_RAW) ? 0 : 1;
  const dim3 grid((unsigned)((a.T + kTile - 1) / kTile));
  if (a.logits != nullptr || a.lse != nullptr)
    return launch(router_mfma_kernel<K, FULL, true>, grid, dim3(kThreads), 0, stream, (const uint16_t*)a.x,
                  (const uint16_t*)a.w, a.bias, a.T, a.d, a.n_experts, normalize, a.idx, a.gates, a.counts,
                  a.logits, a.lse, a.tile_loads, a.loads_stride);
  return launch(router_mfma_kernel<K, FULL, false>, grid, dim3(kThreads), 0, stream, (const uint16_t*)a.x,
                (const uint16_t*)a.w, a.bias, a.T, a.d, a.n_experts, normalize, a.idx, a.gates, a.counts,
                a.logits, a.lse, a.tile_loads, a.loads_stride);
}

template <int K>
hipError_t launch_k(const RouterArgs& a, hipStream_t stream) {
  return a.n_experts == kExp ? launch_kf<K, true>(a, stream) : launch_kf<K, false>(a, stream);
}

}  // namespace

static_assert(kTile == kDispatchTile, "the router tile must be the dispatch tile");

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

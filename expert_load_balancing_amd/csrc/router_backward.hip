// Router backward on CDNA4 matrix cores: gradients of a loss through the gates and the router
// z-loss, with respect to the logits, the tokens and the router weights.
//
// The pages give no backward; this is the chain rule through the forward of router_mfma.hip,
// at the forward's own selection (Top-K is piecewise constant, and the bias b, used only inside
// Top-K, gets no gradient: it is a buffer moved by the balancer, "SMEBU Load Balancing", "How it
// works").  For the loss L = sum_{t,j} G[t,j] g[t,j] + c mean_t lse_t^2, token t, chosen experts
// i_j with s_j = sigmoid(z_{t,i_j}) and S = sum_j s_j:
//   normalised gates (g_j = s_j / S):  dL/ds_j = (G_j - sum_m G_m g_m) / S;   raw: dL/ds_j = G_j
//   dL/dz_{t,i_j} = dL/ds_j s_j (1 - s_j)
//   every expert i: dL/dz_{t,i} += (2 c / T) lse_t softmax(z_t)_i     (the z-loss)
//   dL/dX = dZ W,  dL/dW = dZ^T X.
// The gate weighting of the routed outputs is the Arcee Trinity Large Technical Report,
// section 2.3; the z-loss is the talk summary "Arcee Halts 400B Blackwell Model Collapse...",
// section "Precision Fallbacks, Loss Stabilization, and MaxVio as Data Telemetry".
//
// Launches (all bf16 operands, fp32 accumulation; no transposed copies anywhere):
//  1. grad_kernel, one workgroup per 256-token tile:
//     a. the forward's streaming product recomputes the tile's logits in registers;
//     b. the epilogue parks them in LDS, forms dL/dz for each token from them, the forward's
//        topk_idx and the upstream gate gradients, rounds it to bf16 into MFMA operand
//        fragments held in registers, and stores it token-major (dZ [T][256], for dW);
//     c. dX = dZ W for the tile: W streams through LDS 64 columns at a time and is read back
//        transposed (k = experts is W's row index), against the dZ fragments in registers; the
//        fp32 result leaves through an LDS stage as whole 256-byte row segments.
//  2. dw_kernel: dW = dZ^T X contracts over tokens with both operands k-major (dZ and X
//     token-major, read back transposed), split over token ranges into fp32 partials.
//  3. reduce_partials_kernel: dW = the partials summed in range order.
// dL/dz is rounded to bf16 before the two products (the usual training precision); the fp32
// accumulation and the rounding are the only departures from exact arithmetic.
#include "../../include/elb.h"
#include "device_common.hpp"
#include "elb_kernels.h"
#include "mfma_tile.hpp"

namespace elb {
namespace {

using namespace tile;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCtas = 256;  // compute units: the dW split count aims at one workgroup per CU

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  // Round to nearest, ties to even (values are finite).
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Stores per wave per dX stage (64 tokens x 64 columns, 1 KiB each): 16 in fp32, 8 in bf16.
template <bool DXBF>
constexpr int kDxStores = DXBF ? 8 : 16;
static_assert(kDma + 2 * kDxStores<false> <= 63, "vmcnt budget fits the counter");
constexpr int kDxAhead = 3;  // k-blocks of W fragments read ahead (4 reads each, <= 15 in flight)

// One 256-token tile: dZ [t][256] (bf16, token-major; NULL: not stored) and dX [t][d] (fp32, or
// bf16 rounded to nearest even with DXBF; NULL: not computed).  zc2 = 2 c / T (0: no z-loss).
template <int K, bool FULL, bool DXBF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grad_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int d, int n_experts, int normalize,
    const int32_t* __restrict__ idx, const float* __restrict__ dgates, float zc2, uint16_t* __restrict__ dz,
    void* __restrict__ dx) {
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[kSlot], xs1[kSlot], xs2[kSlot];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[kSlot], ws1[kSlot];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int64_t row0 = (int64_t)blockIdx.x * kRowsB;
  const int rows = (int)(T - row0 < kRowsB ? T - row0 : kRowsB);
  const uint32_t row_bytes = (uint32_t)d * 2u;

  // fr[nb][kb]: the MFMA operand fragment of dL/dz for token block nb (tokens 32 nb + lane % 32
  // of the wave's 64), k-block kb (experts 16 kb .. + 15): element i = expert
  // 16 kb + 8 (i / 4) + 4 h + (i & 3), as bf16 pairs.
  uint32_t fr[kNB][16][4];
  {
    // ---- a. logits of the tile: Z^T = W X^T, token columns per lane ----
    Stream<kAuxCached, kAuxStream> st;
    st.init(w, (uint32_t)n_experts * row_bytes, row_bytes, x + row0 * d, (uint32_t)rows * row_bytes, row_bytes,
            d / kBK, wave, lane, Slots{xs0, xs1, xs2, ws0, ws1});
    st.prologue();
    f32x16 acc[kMB][kNB];
    st.run(acc, wave, lane);

    // Each wave parks its logits in a slot of its own, [32 groups][64 lanes][4 floats]: group
    // q = 4 mb + g holds acc[mb][nb][4 g .. 4 g + 3], experts 32 mb + 8 g + 4 h + 0..3 of the
    // lane's token.  Reading them back from LDS keeps the epilogue's registers free.
    float* const park = reinterpret_cast<float*>(wave == 0 ? xs0 : wave == 1 ? xs1 : wave == 2 ? xs2 : ws0);
    auto own = [&](int q) { return *reinterpret_cast<const f32x4*>(park + (q * 64 + lane) * 4); };
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[mb][nb][4 * g + r];
          *reinterpret_cast<f32x4*>(park + ((mb * 4 + g) * 64 + lane) * 4) = v;
        }
      wave_lds_sync();
      const int64_t t = row0 + wave * kRowsWave + nb * 32 + l32;
      const bool live = t < T;

      // ---- b. dL/dz ----
      // log-sum-exp of the token's logits (the lane's 128, merged with lane ^ 32's).
      float lse = 0.0f;
      if (zc2 != 0.0f) {
        float m = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          const f32x4 v = own(q);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (FULL || (q >> 2) * 32 + 8 * (q & 3) + 4 * h + r < n_experts) m = fmaxf(m, v[r]);
        }
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          const f32x4 v = own(q);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (FULL || (q >> 2) * 32 + 8 * (q & 3) + 4 * h + r < n_experts)
              sum += __builtin_amdgcn_exp2f((v[r] - m) * kLog2e);
        }
        const float m2 = __shfl_xor(m, 32);
        const float sum2 = __shfl_xor(sum, 32);
        const float mm = fmaxf(m, m2);
        lse = mm + __logf(sum * __builtin_amdgcn_exp2f((m - mm) * kLog2e) +
                          sum2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e));
      }
      // dL/dz at the K chosen experts: their logits come from either lane of the pair.
      int e[K];
      float dzs[K];
      {
        float s[K], G[K];
        float S = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
          e[j] = live ? idx[t * K + j] : -1;
          G[j] = live ? dgates[t * K + j] : 0.0f;
          const int ej = e[j] < 0 ? 0 : (e[j] > kRowsA - 1 ? kRowsA - 1 : e[j]);  // stay inside the park
          s[j] = sigmoid_fast(park[((ej >> 3) * 64 + l32 + 32 * ((ej >> 2) & 1)) * 4 + (ej & 3)]);
          S += s[j];
        }
        float Gg = 0.0f;
        const float inv = 1.0f / S;
        if (normalize) {
#pragma unroll
          for (int j = 0; j < K; ++j) Gg += G[j] * (s[j] * inv);
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float ds = normalize ? (G[j] - Gg) * inv : G[j];
          dzs[j] = ds * s[j] * (1.0f - s[j]);
        }
      }
      // Every expert of the lane: z-loss part plus the chosen-expert part; padded experts and
      // tokens past T get 0.  Rounded to bf16 into the fragments; stored token-major.
      const float zl = zc2 * lse;
      uint16_t* const drow = dz + (live ? t : 0) * kRowsA + 4 * h;
#pragma unroll
      for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const f32x4 zv = own(2 * kb + qq);  // experts 16 kb + 8 qq + 4 h + 0..3
          uint32_t b[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ex = 16 * kb + 8 * qq + 4 * h + r;
            float v = 0.0f;
            if (zc2 != 0.0f) v = zl * __builtin_amdgcn_exp2f((zv[r] - lse) * kLog2e);
#pragma unroll
            for (int j = 0; j < K; ++j) v += e[j] == ex ? dzs[j] : 0.0f;
            if (!live || (!FULL && ex >= n_experts)) v = 0.0f;
            b[r] = bf16_rne(v);
          }
          fr[nb][kb][2 * qq] = b[0] | (b[1] << 16);
          fr[nb][kb][2 * qq + 1] = b[2] | (b[3] << 16);
        }
        if (dz != nullptr && live) {
          *reinterpret_cast<uint2*>(drow + 16 * kb) = uint2{fr[nb][kb][0], fr[nb][kb][1]};
          *reinterpret_cast<uint2*>(drow + 16 * kb + 8) = uint2{fr[nb][kb][2], fr[nb][kb][3]};
        }
      }
      wave_lds_sync();  // the park is read before the next block's logits overwrite it
    }
  }
  if (dx == nullptr) return;

  // ---- c. dX = dZ W for the tile's tokens ----
  // Every wave is done with its park and every load and store above has completed, so the
  // slots are free and the vmcnt budgets below start from zero.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & ~(15 << 8));
  bare_barrier();
  // W slots xs0, xs1, ws0 (a ring; stage j + 2 fills while stage j is read): 256 expert rows x
  // 64 columns (128 bytes), rows past n_experts read 0.  Chunks of row r sit at
  // chunk ^ (((r >> 1) & 1) << 2): a transposed read has each group of 32 lanes read 4
  // consecutive rows (two per 256-byte bank window) x 64 bytes, and the swizzle puts rows r and
  // r + 2 in different halves of their window.  Store stage: xs2, 8 KiB a wave.
  //
  // vmcnt budget when stage j's DMAs must have landed: per stage a wave issues 8 DMAs (stage
  // j + 2) and then kSt stores (stage j); behind stage j's DMAs come those of stage 1
  // (j = 0), the DMAs of stage 2 and the stores of stage 0 (j = 1), or the stores of j - 2, the
  // DMAs of j + 1 and the stores of j - 1 (j >= 2).  Stages 0 and 1 are peeled: one loop over
  // three different waits would leave the compiler's own wait analysis with the weakest.
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)n_experts * row_bytes);
  uint32_t vo[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int r = wave * 64 + 8 * i + (lane >> 3);
    vo[i] = (uint32_t)r * row_bytes + (uint32_t)(((lane & 7) ^ (((r >> 1) & 1) << 2)) << 4);
  }
  const uint32_t wave_off = (uint32_t)wave * (64 * kRowB);
  const int nst = d / kBK;
  const __amdgpu_buffer_rsrc_t none = make_rsrc(w, 0u);
  // Stage offsets are forced wave-uniform with readfirstlane: a vector offset would turn every
  // DMA and store into a loop over distinct lane values.
  auto dma = [&](unsigned char* slot, int j) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)j * kRowB);
    dma_rows<kAuxCached, kDma>(wr, none, slot + wave_off, vo, soff, j < nst);
  };
  dma(xs0, 0);
  dma(xs1, 1);
  // Stores go through a descriptor covering the tile's live rows: rows past T are dropped while
  // every store instruction still issues (the vmcnt budget counts them).  They are non-temporal:
  // with normal allocation the dX stream would push W out of L2, where every CU re-reads it.
  constexpr int kEs = DXBF ? 2 : 4;  // bytes per dX element
  constexpr int kSt = kDxStores<DXBF>;
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<unsigned char*>(dx) + row0 * d * kEs, (uint32_t)rows * (uint32_t)d * kEs);
  TrLane tl;
  tl.init(lane);
  const uint32_t ro = tl.row * (uint32_t)kRowB + tl.col;
  const uint32_t sw = ((tl.j >> 1) & 1u) << 6;  // ((row >> 1) & 1) << 2 chunks = 64 bytes
  // Store q: token rows wave*64 + 8 q + lane / 8, 16 bytes at byte 16 (lane % 8) of the row's
  // 128-byte segment (fp32: of one 32-column half; bf16: of the whole 64-column stage).
  const uint32_t so = (uint32_t)(wave * kRowsWave + (lane >> 3)) * (uint32_t)d * kEs + (uint32_t)(lane & 7) * 16u;
  const uint32_t q_stride = 8u * (uint32_t)d * kEs;
  unsigned char* const stg = xs2 + wave * (kSlot / 4);
  // W fragment of k-block kb (experts 16 kb .. + 15), columns 32 cb .. + 31 of the stage.
  auto frag = [&](const unsigned char* sl, int kb, int cb) {
    const unsigned char* p = sl + kb * (16 * kRowB) + ro + (((uint32_t)cb << 6) ^ sw);
    return join_tr(ds_read_tr16(p), ds_read_tr16(p + 8 * kRowB));
  };
  // Stage j: start stage j + 2's DMAs into `nxt`, multiply the W columns in `cur`, store.
  auto stage = [&](int j, const unsigned char* cur, unsigned char* nxt) {
    f32x16 c[2][kNB];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[cb][nb][r] = 0.0f;
    dma(nxt, j + 2);
    // Fragments run kDxAhead k-blocks ahead of the MFMAs that use them: 4 MFMAs (128 cycles) per
    // k-block do not cover an LDS read's latency while four waves share the LDS.
    bf16x8 a[kDxAhead + 1][2];
#pragma unroll
    for (int kb = 0; kb < kDxAhead; ++kb) {
      a[kb][0] = frag(cur, kb, 0);
      a[kb][1] = frag(cur, kb, 1);
    }
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      if (kb + kDxAhead < 16) {
        a[(kb + kDxAhead) % (kDxAhead + 1)][0] = frag(cur, kb + kDxAhead, 0);
        a[(kb + kDxAhead) % (kDxAhead + 1)][1] = frag(cur, kb + kDxAhead, 1);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const i32x4 bv = {(int)fr[nb][kb][0], (int)fr[nb][kb][1], (int)fr[nb][kb][2], (int)fr[nb][kb][3]};
          c[cb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb % (kDxAhead + 1)][cb],
                                                             __builtin_bit_cast(bf16x8, bv), c[cb][nb], 0, 0, 0);
        }
    }
    // Issue order: the reads of the first kDxAhead k-blocks; then per k-block the reads of the one
    // kDxAhead further and its 4 MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * kDxAhead, 0);
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      if (kb + kDxAhead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // Stores go out as whole 128-byte row segments through the wave's 8 KiB LDS stage,
    // [64 tokens][8 chunks of 16 bytes], chunk ch of token row t at ch ^ (t & 7); fp32 takes one
    // 32-column half of the 64 x 64 tile at a time, bf16 the whole tile.  Lane: token
    // 32 nb + l32 of the wave; accumulator 4 g + r: column 32 cb + 8 g + 4 h + r of the stage.
    const uint32_t ssoff = __builtin_amdgcn_readfirstlane((uint32_t)j * (kBK * kEs));
    // Store q: tokens 8 q .. 8 q + 7, 8 lanes (8 chunks) per token row.
    auto flush = [&](uint32_t seg) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int t = 8 * q + (lane >> 3);
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + t * 128 + (((lane & 7) ^ (t & 7)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), xr,
                                               (int)(so + (uint32_t)q * q_stride + seg), (int)ssoff, kAuxStream);
      }
    };
    if constexpr (DXBF) {
      // Chunk of columns 32 cb + 8 g .. + 7 is 4 cb + g; the lane's 4 columns are its half h.
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int t = nb * 32 + l32;
            const uint2 v = {bf16_rne(c[cb][nb][4 * g]) | (bf16_rne(c[cb][nb][4 * g + 1]) << 16),
                             bf16_rne(c[cb][nb][4 * g + 2]) | (bf16_rne(c[cb][nb][4 * g + 3]) << 16)};
            // One integer offset: split into two pointer steps, the compiler lost track of which
            // LDS array the store hits and drained every DMA and store before it.
            *reinterpret_cast<uint2*>(stg + (t * 128 + (((4 * cb + g) ^ (t & 7)) << 4) + 8 * h)) = v;
          }
      flush(0u);
    } else {
      // Chunk of columns 32 cb + 8 g + 4 h .. + 3 within half cb is 2 g + h.
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int t = nb * 32 + l32;
            const f32x4 v = {c[cb][nb][4 * g], c[cb][nb][4 * g + 1], c[cb][nb][4 * g + 2], c[cb][nb][4 * g + 3]};
            *reinterpret_cast<f32x4*>(stg + t * 128 + (((2 * g + h) ^ (t & 7)) << 4)) = v;
          }
        flush((uint32_t)cb * 128u);
      }
    }
  };
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma) & ~(15 << 8));
  bare_barrier();
  stage(0, xs0, ws0);
  if (nst > 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma + kSt) & ~(15 << 8));
    bare_barrier();
    stage(1, xs1, xs0);
  }
  for (int j = 2; j < nst; j += 3) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma + 2 * kSt) & ~(15 << 8));
    bare_barrier();
    stage(j, ws0, xs1);
    if (j + 1 >= nst) break;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma + 2 * kSt) & ~(15 << 8));
    bare_barrier();
    stage(j + 1, xs0, ws0);
    if (j + 2 >= nst) break;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDma + 2 * kSt) & ~(15 << 8));
    bare_barrier();
    stage(j + 2, xs1, xs0);
  }
  // The stores drain before the workgroup ends.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & ~(15 << 8));
}

// Store one wave's blocks of the fp32 product (acc of the streaming product: MBW blocks of 32 A
// rows from row m0, kNB blocks of 32 B rows from column n0) through the wave's own LDS stage, one
// 32-column block at a time ([32 MBW rows][32 columns] fp32), then in 16-byte pieces, 8 rows x
// 128 bytes per store.  Stores m < c_rows, n < c_cols (c_cols % 4 == 0), row stride ldc.
template <int MBW>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[MBW][kNB], float* stage, float* C, int64_t ldc,
                                           int64_t m0, int64_t n0, int64_t c_rows, int64_t c_cols, int lane) {
  const int h = lane >> 5;
  const int l32 = lane & 31;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[(mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * 32 + l32] = acc[mb][nb][r];
    wave_lds_sync();
    const int64_t n = n0 + nb * 32 + (lane & 7) * 4;
#pragma unroll 8
    for (int q = 0; q < 4 * MBW; ++q) {
      const int row = 8 * q + (lane >> 3);
      const int64_t m = m0 + row;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + row * 32 + (lane & 7) * 4);
      if (m < c_rows && n < c_cols) *reinterpret_cast<f32x4*>(C + m * ldc + n) = v;
    }
    wave_lds_sync();  // the stage is read before the next block overwrites it
  }
}

// part[z][m][n0 + n] = sum over tokens t of range z of dZ[t][m] X[t][n0 + n]   (m, n < 256).
// Range z covers 64-token stages [Q z / S, Q (z + 1) / S) (Q = ceil(T / 64), S = splits).  The
// workgroups that share a range run on one XCD (a linear id L runs on XCD L % 8), so its dZ rows
// come from HBM once into that XCD's L2 and serve all n_col column tiles there.  8 waves, two per
// SIMD: wave w holds dW rows 128 (w % 2) .. + 127 of columns 64 (w / 2) .. + 63; waves 4-7 issue
// the DMAs, waves 0-3 only read LDS and multiply.
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void dw_kernel(
    const uint16_t* __restrict__ dz, const uint16_t* __restrict__ x, int64_t T, int d, int64_t Q, int splits,
    int n_col, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[kSlot], xs1[kSlot], xs2[kSlot];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[kSlot], ws1[kSlot];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-grouped order: XCD x holds G / 8 (+1 for x < G % 8) consecutive work items.
  const int G = (int)gridDim.x;
  const int L = (int)blockIdx.x;
  const int xcd = L & 7, slot = L >> 3;
  const int o = xcd * (G >> 3) + (xcd < (G & 7) ? xcd : (G & 7)) + slot;
  const int z = o / n_col, col = o - z * n_col;
  const int64_t s0 = Q * z / splits, s1 = Q * (z + 1) / splits;
  const int64_t t0 = s0 * kBK;
  const int64_t t1 = s1 * kBK < T ? s1 * kBK : T;
  const int64_t n0 = (int64_t)col * kRowsB;
  const uint32_t xrow = (uint32_t)d * 2u;
  Stream<kAuxCached, kAuxStream, KRows, KRows, kNB, 2, true> st;
  st.init(dz + t0 * kRowsA, (uint32_t)(t1 - t0) * (uint32_t)(kRowsA * 2), (uint32_t)(kRowsA * 2), x + t0 * d + n0,
          (uint32_t)((t1 - t0) * xrow - 2 * n0), xrow, (int)(s1 - s0), wave, lane, Slots{xs0, xs1, xs2, ws0, ws1});
  st.prologue();
  f32x16 acc[kMB / 2][kNB];
  st.run(acc, wave, lane);
  // Stage: 16 KiB half (w & 1) of slot w / 2.
  unsigned char* const sl = (wave >> 1) == 0 ? xs0 : (wave >> 1) == 1 ? xs1 : (wave >> 1) == 2 ? xs2 : ws0;
  float* const stage = reinterpret_cast<float*>(sl + (wave & 1) * 16384);
  store_tile<kMB / 2>(acc, stage, part + (int64_t)z * kRowsA * d, d, (wave & 1) * 128, n0 + (wave >> 1) * kRowsWave,
                      kRowsA, d, lane);
}

// out[i] = sum_{s < S} part[s * stride + i], in order s = 0, 1, ... (0 for S = 0); n4 float4s.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float4* __restrict__ part, int S, int64_t stride4,
                                                              int64_t n4, float4* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 a = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < S; ++s) {
      const float4 b = part[s * stride4 + i];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    out[i] = a;
  }
}

template <int K, bool DXBF>
hipError_t launch_grad_kb(const BackwardArgs& a, const BackwardPlan& p, hipStream_t s) {
  const dim3 grid((unsigned)((a.T + kRowsB - 1) / kRowsB));
  const float zc2 = 2.0f * a.zloss_coef / (float)a.T;
  uint16_t* const dz = a.dw != nullptr ? p.dz : nullptr;
  if (a.n_experts == kRowsA)
    return launch(grad_kernel<K, true, DXBF>, grid, dim3(kThreads), 0, s, (const uint16_t*)a.x, (const uint16_t*)a.w,
                  a.T, a.d, a.n_experts, a.normalize, a.idx, a.dgates, zc2, dz, a.dx);
  return launch(grad_kernel<K, false, DXBF>, grid, dim3(kThreads), 0, s, (const uint16_t*)a.x, (const uint16_t*)a.w,
                a.T, a.d, a.n_experts, a.normalize, a.idx, a.dgates, zc2, dz, a.dx);
}

template <int K>
hipError_t launch_grad_k(const BackwardArgs& a, const BackwardPlan& p, hipStream_t s) {
  return a.dx_bf16 ? launch_grad_kb<K, true>(a, p, s) : launch_grad_kb<K, false>(a, p, s);
}

}  // namespace

BackwardPlan backward_plan(int64_t T, int d, void* workspace) {
  BackwardPlan p{};
  p.Q = (T + kBK - 1) / kBK;
  p.n_col = (d + kRowsB - 1) / kRowsB;
  // Token ranges of dW: enough for one workgroup per CU, each range's X rows under 2 GiB (the
  // buffer descriptors' 32-bit range), never more ranges than 64-token stages.
  int64_t S = kCtas / p.n_col > 1 ? kCtas / p.n_col : 1;
  const int64_t need = (T * (int64_t)d + (int64_t(1) << 30) - 1) >> 30;
  if (S < need) S = need;
  if (S > p.Q) S = p.Q;
  p.splits = (int)S;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  unsigned char* base = static_cast<unsigned char*>(workspace);
  size_t off = 0;
  p.dz = reinterpret_cast<uint16_t*>(base + off);
  off += al((size_t)T * kRowsA * 2);
  p.part = reinterpret_cast<float*>(base + off);
  off += al((size_t)p.splits * kRowsA * d * 4);
  p.bytes = off > 0 ? off : 256;
  return p;
}

hipError_t launch_router_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (a.T > 0) {
    switch (a.k) {
      case 1: err = launch_grad_k<1>(a, p, s); break;
      case 2: err = launch_grad_k<2>(a, p, s); break;
      case 3: err = launch_grad_k<3>(a, p, s); break;
      case 4: err = launch_grad_k<4>(a, p, s); break;
      case 5: err = launch_grad_k<5>(a, p, s); break;
      case 6: err = launch_grad_k<6>(a, p, s); break;
      case 7: err = launch_grad_k<7>(a, p, s); break;
      default: err = launch_grad_k<8>(a, p, s); break;
    }
    if (err != hipSuccess) return err;
  }
  if (a.dw == nullptr) return err;
  if (a.T > 0) {
    err = launch(dw_kernel, dim3((unsigned)(p.n_col * p.splits)), dim3(2 * kThreads), 0, s, (const uint16_t*)p.dz,
                 (const uint16_t*)a.x, a.T, a.d, p.Q, p.splits, p.n_col, p.part);
    if (err != hipSuccess) return err;
  }
  const int64_t n4 = (int64_t)a.n_experts * a.d / 4;
  const int64_t blocks = (n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048;
  return launch(reduce_partials_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const float4*)p.part,
                a.T > 0 ? p.splits : 0, (int64_t)kRowsA * a.d / 4, n4, (float4*)a.dw);
}

}  // namespace elb

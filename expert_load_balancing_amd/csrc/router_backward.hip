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
// Launches (all bf16 operands, fp32 accumulation):
//  1. grad_logits: the forward's streaming product recomputes each 256-token tile of logits in
//     registers; the epilogue forms dL/dz from the tile's logits, the forward's topk_idx and the
//     upstream gate gradients, and stores it rounded to bf16 expert-major (dZ^T [256][T_pad]):
//     a lane holds 32 consecutive tokens of one expert row per store.
//  2. transposes (64 x 64 tiles through LDS): dZ^T -> dZ [T_pad][256], W -> W^T [d][256],
//     X -> X^T [d][T_pad], zero-padded, so that both products below contract contiguous rows.
//  3. dX = dZ W as the streaming product with A = dZ (256 tokens), B = W^T (256 columns of d).
//  4. dW = dZ^T X as the streaming product with A = dZ^T (all experts), B = X^T (256 columns of
//     d), split over token chunks into fp32 partials, then summed over the chunks in order.
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

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  // Round to nearest, ties to even (values are finite).
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// dZ^T [256][ld] (bf16) of one 256-token tile.  zc2 = 2 c / T (0: no z-loss term).
template <int K, bool FULL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void grad_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int d, int n_experts, int normalize,
    const int32_t* __restrict__ idx, const float* __restrict__ dgates, float zc2, uint16_t* __restrict__ dzt,
    int64_t ld) {
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
  Stream<kAuxCached, kAuxStream> st;
  st.init(w, (uint32_t)n_experts * row_bytes, x + row0 * d, (uint32_t)rows * row_bytes, row_bytes, d / kBK, wave,
          lane, Slots{xs0, xs1, xs2, ws0, ws1});
  st.prologue();
  f32x16 acc[kMB][kNB];
  st.run(acc, wave, lane);

  // Each wave parks its scores in a slot of its own: [32 row groups][64 lanes][4 floats].
  float* const park = reinterpret_cast<float*>(wave == 0 ? xs0 : wave == 1 ? xs1 : wave == 2 ? xs2 : ws0);
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int64_t t = row0 + wave * kRowsWave + nb * 32 + l32;
    const bool live = t < T;
    // log-sum-exp of the token's logits (the lane's 128, merged with lane ^ 32's).
    float lse = 0.0f;
    if (zc2 != 0.0f) {
      float m = -__builtin_inff();
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (FULL || e < n_experts) m = fmaxf(m, acc[mb][nb][r]);
        }
      float sum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (FULL || e < n_experts) sum += __builtin_amdgcn_exp2f((acc[mb][nb][r] - m) * kLog2e);
        }
      const float m2 = __shfl_xor(m, 32);
      const float sum2 = __shfl_xor(sum, 32);
      const float mm = fmaxf(m, m2);
      lse = mm + __logf(sum * __builtin_amdgcn_exp2f((m - mm) * kLog2e) + sum2 * __builtin_amdgcn_exp2f((m2 - mm) * kLog2e));
    }
    // Scores of the lane's experts, parked so that either lane of the pair can read any of them.
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 sv;
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = sigmoid_fast(acc[mb][nb][g * 4 + r]);
        *reinterpret_cast<f32x4*>(park + ((mb * 4 + g) * 64 + lane) * 4) = sv;
      }
    wave_lds_sync();
    // dL/dz at the K chosen experts.
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
        s[j] = park[((ej >> 3) * 64 + l32 + 32 * ((ej >> 2) & 1)) * 4 + (ej & 3)];
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
    wave_lds_sync();  // every lane has read the park before it is overwritten below
    // dL/dz for each of the lane's experts: z-loss part plus the chosen-expert part; padded
    // experts and tokens past T get 0.  Staged as bf16 in the park, expert-major
    // [256 experts][32 tokens], then written out in 16-byte pieces: 64 bytes per expert row.
    uint16_t* const stage = reinterpret_cast<uint16_t*>(park);
    const float zl = zc2 * lse;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ex = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        float v = 0.0f;
        if (zc2 != 0.0f) v = zl * __builtin_amdgcn_exp2f((acc[mb][nb][r] - lse) * kLog2e);
#pragma unroll
        for (int j = 0; j < K; ++j) v += e[j] == ex ? dzs[j] : 0.0f;
        if (!live || (!FULL && ex >= n_experts)) v = 0.0f;
        stage[ex * 32 + l32] = bf16_rne(v);
      }
    wave_lds_sync();
    // 256 rows x 4 pieces = 1024 pieces, 16 per lane: lane l takes piece q * 64 + l, i.e. row
    // 16 q + l / 4, piece l % 4 (tokens 8 (l % 4) .. + 7 of this block).
    const int64_t t0 = row0 + wave * kRowsWave + nb * 32;
    uint16_t* const out = dzt + (int64_t)(lane >> 2) * ld + t0 + (lane & 3) * 8;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 16 * q + (lane >> 2);
      const uint4 v = *reinterpret_cast<const uint4*>(stage + row * 32 + (lane & 3) * 8);
      *reinterpret_cast<uint4*>(out + (int64_t)(16 * q) * ld) = v;
    }
    wave_lds_sync();  // the stage is read before the next block's scores overwrite it
  }
}

// out[c][r] = in[r][c] for r < R, 0 for R <= r < R_pad; c < C (C % 64 == 0).  64 x 64 tiles.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, int64_t R, int64_t C,
                                                             int64_t ldi, uint16_t* __restrict__ out, int64_t ldo) {
  __shared__ uint16_t tile[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
  // Load: 64 rows x 8 chunks of 8 elements; thread -> (row, chunk), two passes.
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p, rr = q >> 3, ch = q & 7;
    const int64_t r = r0 + rr;
    uint16_t v[8];
    if (r < R) {
      const uint4 u = *reinterpret_cast<const uint4*>(in + r * ldi + c0 + ch * 8);
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = (uint16_t)(uw[i] & 0xFFFF);
        v[2 * i + 1] = (uint16_t)(uw[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[rr][ch * 8 + i] = v[i];
  }
  __syncthreads();
  // Store: 64 output rows (c) x 8 chunks of 8 r values.
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p, cc = q >> 3, ch = q & 7;
    uint32_t uw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) uw[i] = (uint32_t)tile[ch * 8 + 2 * i][cc] | ((uint32_t)tile[ch * 8 + 2 * i + 1][cc] << 16);
    *reinterpret_cast<uint4*>(out + (c0 + cc) * ldo + r0 + ch * 8) = uint4{uw[0], uw[1], uw[2], uw[3]};
  }
}

// C[m][n] (+ z * c_split) = sum over k in chunk z of A[m][k] B[n][k]; A rows m < a_rows, B rows
// n < b_rows (rows past them read 0), rows row_bytes apart; chunk z covers k in
// [z * kc, (z + 1) * kc) (kc = k_stages * 64).  Stores m < c_rows, n < c_cols, row stride ldc.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_nt_kernel(
    const uint16_t* __restrict__ A, int64_t a_rows, const uint16_t* __restrict__ B, int64_t b_rows, int64_t ld,
    int k_stages, float* __restrict__ C, int64_t c_rows, int64_t c_cols, int64_t ldc, int64_t c_split) {
  __shared__ __attribute__((aligned(1024))) unsigned char xs0[kSlot], xs1[kSlot], xs2[kSlot];
  __shared__ __attribute__((aligned(1024))) unsigned char ws0[kSlot], ws1[kSlot];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.x * kRowsA, n0 = (int64_t)blockIdx.y * kRowsB;
  const int64_t k0 = (int64_t)blockIdx.z * k_stages * kBK;
  const int64_t am = a_rows - m0 < kRowsA ? a_rows - m0 : kRowsA;
  const int64_t bn = b_rows - n0 < kRowsB ? b_rows - n0 : kRowsB;
  const uint32_t row_bytes = (uint32_t)(ld * 2);
  const uint32_t span = (uint32_t)(k_stages * kRowB);  // bytes of one row in this chunk
  Stream<kAuxStream, kAuxStream> st;
  st.init(A + m0 * ld + k0, (uint32_t)((am - 1) * row_bytes + span), B + n0 * ld + k0,
          (uint32_t)((bn - 1) * row_bytes + span), row_bytes, k_stages, wave, lane, Slots{xs0, xs1, xs2, ws0, ws1});
  st.prologue();
  f32x16 acc[kMB][kNB];
  st.run(acc, wave, lane);
  // Store the tile through the wave's own (now free) LDS slot, one 32-column block at a time:
  // [256 rows][32 columns] fp32 = 32 KiB, then 16-byte pieces, 8 rows x 128 bytes per store.
  float* const Cz = C + (int64_t)blockIdx.z * c_split;
  float* const stage = reinterpret_cast<float*>(wave == 0 ? xs0 : wave == 1 ? xs1 : wave == 2 ? xs2 : ws0);
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[(mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * 32 + l32] = acc[mb][nb][r];
    wave_lds_sync();
    const int64_t n = n0 + wave * kRowsWave + nb * 32 + (lane & 7) * 4;  // c_cols % 4 == 0: n..n+3 together
#pragma unroll 8
    for (int q = 0; q < 32; ++q) {
      const int row = 8 * q + (lane >> 3);
      const int64_t m = m0 + row;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + row * 32 + (lane & 7) * 4);
      if (m < c_rows && n < c_cols) *reinterpret_cast<f32x4*>(Cz + m * ldc + n) = v;
    }
    wave_lds_sync();  // the stage is read before the next block overwrites it
  }
}

// out[i] = sum_{s < S} part[s * stride + i], in order s = 0, 1, ...; n4 float4 elements.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float4* __restrict__ part, int S, int64_t stride4,
                                                              int64_t n4, float4* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 a = part[i];
    for (int s = 1; s < S; ++s) {
      const float4 b = part[s * stride4 + i];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    out[i] = a;
  }
}

template <int K>
hipError_t launch_grad_logits_k(const BackwardArgs& a, const BackwardPlan& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.T_pad / kRowsB));
  const float zc2 = a.T > 0 ? 2.0f * a.zloss_coef / (float)a.T : 0.0f;
  if (a.n_experts == kRowsA)
    return launch(grad_logits_kernel<K, true>, grid, dim3(kThreads), 0, s, (const uint16_t*)a.x, (const uint16_t*)a.w,
                  a.T, a.d, a.n_experts, a.normalize, a.idx, a.dgates, zc2, p.dzt, p.T_pad);
  return launch(grad_logits_kernel<K, false>, grid, dim3(kThreads), 0, s, (const uint16_t*)a.x, (const uint16_t*)a.w,
                a.T, a.d, a.n_experts, a.normalize, a.idx, a.dgates, zc2, p.dzt, p.T_pad);
}

hipError_t launch_transpose(const uint16_t* in, int64_t R, int64_t R_pad, int64_t C, int64_t ldi, uint16_t* out,
                            int64_t ldo, hipStream_t s) {
  return launch(transpose_bf16_kernel, dim3((unsigned)(R_pad / 64), (unsigned)(C / 64)), dim3(256), 0, s, in, R, C, ldi,
                out, ldo);
}

}  // namespace

BackwardPlan backward_plan(int64_t T, int d, void* workspace) {
  BackwardPlan p{};
  p.T_pad = (T + kRowsB - 1) / kRowsB * kRowsB;
  if (p.T_pad == 0) p.T_pad = kRowsB;
  // Token chunks of dW: 256 c tokens with c <= 8 the largest divisor of T_pad / 256, so the
  // chunks tile the padded rows exactly (a chunk must never run into the next row).
  const int64_t q = p.T_pad / kRowsB;
  int64_t c = 8;
  while (q % c != 0) --c;
  p.k_chunk = kRowsB * c;
  p.splits = (int)(q / c);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t off = 0;
  const size_t dzt_b = al((size_t)kRowsA * p.T_pad * 2), dz_b = dzt_b, wt_b = al((size_t)d * kRowsA * 2);
  const size_t xt_b = al((size_t)d * p.T_pad * 2), part_b = al((size_t)p.splits * kRowsA * d * 4);
  unsigned char* base = static_cast<unsigned char*>(workspace);
  p.dzt = reinterpret_cast<uint16_t*>(base + off);
  off += dzt_b;
  p.dz = reinterpret_cast<uint16_t*>(base + off);
  off += dz_b;
  p.wt = reinterpret_cast<uint16_t*>(base + off);
  off += wt_b;
  p.xt = reinterpret_cast<uint16_t*>(base + off);
  off += xt_b;
  p.part = reinterpret_cast<float*>(base + off);
  off += part_b;
  p.bytes = off;
  return p;
}

hipError_t launch_router_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t s) {
  hipError_t err;
  switch (a.k) {
    case 1: err = launch_grad_logits_k<1>(a, p, s); break;
    case 2: err = launch_grad_logits_k<2>(a, p, s); break;
    case 3: err = launch_grad_logits_k<3>(a, p, s); break;
    case 4: err = launch_grad_logits_k<4>(a, p, s); break;
    case 5: err = launch_grad_logits_k<5>(a, p, s); break;
    case 6: err = launch_grad_logits_k<6>(a, p, s); break;
    case 7: err = launch_grad_logits_k<7>(a, p, s); break;
    default: err = launch_grad_logits_k<8>(a, p, s); break;
  }
  if (err != hipSuccess) return err;
  const int64_t d = a.d;
  // dZ [T_pad][256] from dZ^T; W^T [d][256] (experts past n_experts zero); X^T [d][T_pad].
  if ((err = launch_transpose(p.dzt, kRowsA, kRowsA, p.T_pad, p.T_pad, p.dz, kRowsA, s)) != hipSuccess) return err;
  if ((err = launch_transpose((const uint16_t*)a.w, a.n_experts, kRowsA, d, d, p.wt, kRowsA, s)) != hipSuccess)
    return err;
  if (a.dw != nullptr &&
      (err = launch_transpose((const uint16_t*)a.x, a.T, p.T_pad, d, d, p.xt, p.T_pad, s)) != hipSuccess)
    return err;
  if (a.dx != nullptr && a.T > 0) {
    // dX [T][d] = dZ W: A = dZ rows (tokens), B = W^T rows (columns of d), K = 256 experts.
    err = launch(gemm_nt_kernel, dim3((unsigned)(p.T_pad / kRowsA), (unsigned)((d + kRowsB - 1) / kRowsB), 1),
                 dim3(kThreads), 0, s,
                 (const uint16_t*)p.dz, p.T_pad, (const uint16_t*)p.wt, d, (int64_t)kRowsA, kRowsA / kBK, a.dx, a.T, d,
                 d, (int64_t)0);
    if (err != hipSuccess) return err;
  }
  if (a.dw != nullptr) {
    // dW [n_experts][d] = dZ^T X: A = dZ^T rows (experts), B = X^T rows (columns of d), K = tokens,
    // split into chunks of k_chunk tokens; the partials are then summed in chunk order.
    err = launch(gemm_nt_kernel, dim3(1, (unsigned)((d + kRowsB - 1) / kRowsB), (unsigned)p.splits), dim3(kThreads), 0,
                 s,
                 (const uint16_t*)p.dzt, (int64_t)kRowsA, (const uint16_t*)p.xt, d, p.T_pad, (int)(p.k_chunk / kBK),
                 p.part, (int64_t)kRowsA, d, d, (int64_t)kRowsA * d);
    if (err != hipSuccess) return err;
    const int64_t n4 = (int64_t)a.n_experts * d / 4;
    const int64_t blocks = (n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048;
    err = launch(reduce_partials_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const float4*)p.part, p.splits,
                 (int64_t)kRowsA * d / 4, n4, (float4*)a.dw);
  }
  return err;
}

}  // namespace elb

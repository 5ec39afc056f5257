// One workgroup's 256 x 256 fp32 product tile on CDNA4 matrix cores (gfx950):
//   acc[m][n] = sum_k A[m][k] * B[n][k]        m, n < 256; A, B bf16
// held in registers, with both operands streamed from memory into LDS by buffer-to-LDS DMA.
// Each operand comes in one of two layouts (the policies RowsK and KRows below): rows
// contiguous in k (row-major A[m][k]), or k-major (row-major A^T[k][m], read back transposed
// by gfx950's transposing LDS read).  The router forward uses it with A = the router weights
// and B = a tile of tokens, both rows contiguous in k (the logits, transposed: Z^T = W X^T);
// the router backward's dW = dZ^T X contracts over tokens with both operands k-major.
//
// Work decomposition: 4 waves, one per SIMD; wave w owns B rows 32 NB w .. + 32 NB - 1 against
// all 256 A rows, i.e. 8 x NB accumulators of 32 x 32 (NB = 2: a 256 x 256 tile in 256 AGPRs;
// NB = 1: a 256 x 128 tile, for batches too small to give every CU a 256-row B tile).  With
// ES = 2 the workgroup has 8 waves, two per SIMD, and the waves 2 p and 2 p + 1 split those B
// rows' A rows between them (128 each); with PR as well, only waves 4-7 (one per SIMD) issue
// the DMAs, and waves 0-3 only read LDS and multiply.  A 32 x 32 MFMA output puts one
// B row per lane column: lane l holds column l % 32 of its block, and accumulator r holds A row
// 8 (r / 4) + 4 (l / 32) + (r % 4).
//
// Memory pipeline: k is consumed in stages of 64 elements (128 bytes of every row: a full HBM
//   line per row per visit; 64-byte visits stream markedly slower because all workgroups touch
//   their rows 2*K bytes apart at once).  By default the B stream runs 2 stages ahead in a ring
//   of 3 LDS slots, the A stream 1 stage ahead in a ring of 2 (A is meant to be the operand that
//   stays in L2, well within one stage): the five 32 KiB slots fill the 160 KiB LDS.  Tiles with
//   fewer B rows have shorter stages and smaller B slots, and take deeper rings (NXR, NWR), so
//   that the prefetch still spans the memory latency.  Rows past the end
//   of an operand fall outside its buffer range and arrive as zeros.  Every wave waits for its
//   own DMAs with an explicit vmcnt budget, then one barrier per stage publishes the slot to all
//   waves and frees the slot the next DMA overwrites.  Barriers carry no memory fence: a fence
//   on LDS would wait for every DMA in flight and drain the prefetch.  Near the end, dummy DMAs
//   through an empty-range descriptor keep the vmcnt budget uniform; they move no bytes.  Within
//   a slot, 16-byte chunks are XOR-swizzled per row (see the layouts), which keeps the MFMA
//   operand reads free of LDS bank conflicts.
#pragma once

#include "device_common.hpp"

namespace elb {
namespace tile {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsA = 256;               // A rows per tile
constexpr int kMB = kRowsA / 32;          // 32-row MFMA blocks of A
constexpr int kRowsWave = 64;             // B rows per wave
constexpr int kNB = kRowsWave / 32;       // 32-column MFMA blocks of B
constexpr int kRowsB = kWaves * kRowsWave;  // B rows per tile
constexpr int kBK = 64;                   // k elements per stage
constexpr int kRowB = kBK * 2;            // bytes of one row per stage
constexpr int kSlot = 256 * kRowB;        // one stage of 256 rows: 32 KiB
constexpr int kNX = 3, kPX = 2;           // B ring: slots, stages in flight
constexpr int kNW = 2, kPW = 1;           // A ring
constexpr int kUnroll = 6;                // lcm(kNX, kNW): slots are compile-time constants
constexpr int kKSteps = kBK / 16;         // MFMA k-steps per stage
// The compiler tracks at most 8 distinct LDS DMA targets when it decides which DMAs an LDS
// read must wait for; with more slots it would fall back to waiting for all of them.
static_assert(kNX + kNW <= 8, "at most 8 DMA target slots");
static_assert((kNX + kNW) * kSlot <= 160 * 1024, "LDS");
constexpr int kDma = kSlot / (kWaves * 1024);  // DMA instructions per wave per slot (1 KiB each)

static_assert(kNX == kPX + 1 && kNW == kPW + 1 && kUnroll % kNX == 0 && kUnroll % kNW == 0, "ring shape");
static_assert(kPX >= kPW, "the vmcnt budget of Stream assumes the B stream runs further ahead");

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 63 & 15 | (3 << 14) | (7 << 4);  // lgkmcnt(0) only

// Cache policies of the DMAs.  A stream read exactly once goes non-temporal (nt): streaming it
// through the caches with normal allocation costs an L2-resident operand its place (for the
// router forward, the whole memory pipeline ~20% of its rate).
constexpr int kAuxStream = 2;  // nt
constexpr int kAuxCached = 0;  // default allocation

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

// One wave's share of one slot: kDma 1-KiB DMA instructions (8 rows each).  A dummy DMA (past
// the last stage) keeps the vmcnt budget uniform: it goes through `none`, a descriptor with an
// empty range, so it reads zeros and moves no bytes.  The choice is a scalar select of the
// descriptor; the row offsets stay in their own registers.  (Selecting the offset per DMA
// instead put a VALU write to one shared register before every DMA, which stalls behind the
// previous DMA's operand read whenever the vector memory queue is full, and with it every
// MFMA queued behind.)
template <int AUX, int N>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, __amdgpu_buffer_rsrc_t none,
                                         unsigned char* wave_base, const uint32_t* vo, uint32_t soff,
                                         bool real) {
  const __amdgpu_buffer_rsrc_t use = real ? r : none;
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(use, ELB_AS3(wave_base + i * 1024), 16, vo[i], (int)soff, 0, AUX);
}

// LDS position of 16-byte chunk c of a 128-byte row segment r.  The LDS serves 16 lanes x 16
// bytes per cycle from 64 banks; an MFMA operand read has 16 consecutive rows read the same
// chunk, and XOR-ing the chunk with bits 1..3 of the row spreads those 16 reads over the
// whole 256-byte bank window (rows r and r + 1 already sit in different 128-byte halves).
__device__ __forceinline__ constexpr int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// The LDS ring slots (declared __shared__ by the kernel, 1 KiB aligned): up to four for the B
// stream (x) and four for the A stream (w); x3, w2, w3 only with deeper rings.
struct Slots {
  unsigned char *x0, *x1, *x2, *w0, *w1, *x3 = nullptr, *w2 = nullptr, *w3 = nullptr;
  __device__ __forceinline__ unsigned char* x(int i) const { return i == 0 ? x0 : i == 1 ? x1 : i == 2 ? x2 : x3; }
  __device__ __forceinline__ unsigned char* w(int i) const { return i == 0 ? w0 : i == 1 ? w1 : i == 2 ? w2 : w3; }
};

constexpr int ring_lcm(int a, int b) {
  int l = a;
  while (l % b != 0) l += a;
  return l;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Operand layout: rows contiguous in k.  A slot holds 256 operand rows x 64 k (128 bytes); the
// eight 16-byte chunks of row r sit at chunk ^ ((r >> 1) & 7).  A fragment (32 rows x 16 k) is
// one 16-byte read per lane: row l % 32, k 8 (l / 32) .. + 7.
struct RowsK {
  static constexpr int kReads = 1;  // LDS reads per fragment
  // DMA: a wave fills `rows_wave` consecutive rows; its instruction i fills rows
  // rows_wave * wave + 8 i + lane / 8; lane position p = lane & 7 in the row receives the global
  // chunk stored there, swz(row, p) (the swizzle is its own inverse).  One stage advances 128
  // bytes along every row.
  __device__ static __forceinline__ uint32_t dma_off(int wave, int lane, int i, uint32_t row_bytes, int rows_wave) {
    const int r = wave * rows_wave + 8 * i + (lane >> 3);
    return (uint32_t)r * row_bytes + (uint32_t)(swz(r, lane & 7) << 4);
  }
  __device__ static __forceinline__ uint32_t stage_bytes(uint32_t) { return kRowB; }
  struct Lane {
    uint32_t fo[kKSteps];
    __device__ __forceinline__ void init(int lane) {
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        fo[s] = (uint32_t)(lane & 31) * kRowB + (uint32_t)(swz(lane & 31, 2 * s + (lane >> 5)) << 4);
    }
    // Block `blk` (rows 32 blk .. + 31) at k-step s.
    __device__ __forceinline__ bf16x8 frag(const unsigned char* slot, int blk, int s) const {
      return *reinterpret_cast<const bf16x8*>(slot + fo[s] + blk * (32 * kRowB));
    }
  };
};

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane 4 p + q
// receives element q of the 8-byte pieces addressed by lanes p, p + 4, p + 8, p + 12 (in that
// order).  So if lane 16 b + 4 j + p addresses k row (R + j) at columns C + 4 p .. + 3, lane
// 16 b + 4 p + q receives column C + 4 p + q at k rows R .. R + 3.
__device__ __forceinline__ i16x4 ds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<unsigned char*>(p)));
}

__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  const __attribute__((ext_vector_type(8))) short v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Per-lane constants of a transposed fragment read.  A fragment's lane l (half hh = l / 32)
// holds column l % 32 of its block and, as element i, k row 8 (i / 4) + 4 hh + (i & 3) of the
// 16-row k-step (any fixed assignment of k is valid as long as both operands of a product use
// it).  Reading it takes two transposed reads, elements 0..3 then 4..7: lane 16 b + 4 j + p
// addresses k row 4 (b / 2) + j (+ 8 for the second read), columns 16 (b & 1) + 4 p .. + 3.
struct TrLane {
  uint32_t row;  // 4 (b / 2) + j
  uint32_t col;  // byte offset of the lane's 8-byte piece inside its 64-byte block segment
  uint32_t j;
  __device__ __forceinline__ void init(int lane) {
    const int b = lane >> 4, j_ = (lane >> 2) & 3, p = lane & 3;
    row = (uint32_t)(4 * (b >> 1) + j_);
    col = (uint32_t)(32 * (b & 1) + 8 * p);
    j = (uint32_t)j_;
  }
};

// Operand layout: k-major.  A slot holds 64 k rows x 256 operand columns (512 bytes); the 32
// chunks of k row r sit at chunk ^ ((r & 3) << 2).  A transposed read then has each group of
// 32 lanes read 4 consecutive k rows x 64 bytes, which the swizzle spreads over all 64 banks.
struct KRows {
  static constexpr int kReads = 2;
  // DMA: instruction i of wave `wave` fills k rows 16 wave + 2 i + lane / 32, lane position
  // p = lane & 31 receiving global chunk p ^ ((r & 3) << 2).  One stage advances 64 k rows.
  __device__ static __forceinline__ uint32_t dma_off(int wave, int lane, int i, uint32_t row_bytes, int) {
    const int r = wave * 16 + 2 * i + (lane >> 5);
    return (uint32_t)r * row_bytes + (uint32_t)(((lane & 31) ^ ((r & 3) << 2)) << 4);
  }
  __device__ static __forceinline__ uint32_t stage_bytes(uint32_t row_bytes) { return 64u * row_bytes; }
  struct Lane {
    uint32_t base;  // k row offset + in-segment byte offset
    uint32_t j;
    __device__ __forceinline__ void init(int lane) {
      TrLane t;
      t.init(lane);
      base = t.row * 512u + t.col;
      j = t.j;  // = k row & 3: the swizzle moves block segment blk to blk ^ j
    }
    __device__ __forceinline__ bf16x8 frag(const unsigned char* slot, int blk, int s) const {
      const unsigned char* p = slot + s * (16 * 512) + base + ((((uint32_t)blk) ^ j) << 6);
      return join_tr(ds_read_tr16(p), ds_read_tr16(p + 8 * 512));
    }
  };
};

// The streaming product.  AUX_A / AUX_B: cache policies of the two streams; LA / LB: their
// layouts; NB: 32-row blocks of B per wave; ES: waves sharing one B row range, each with
// 256 / ES of the A rows (ES = 2: 8 waves, two per SIMD, so that one wave's stalled DMA or LDS
// read leaves the other issuing MFMAs).  Wave w owns A blocks (w % ES) * kMB / ES .. and B blocks
// (w / ES) * NB ...  A's rows are `a_row_bytes` apart, B's `b_row_bytes`; `nkb` stages of kBK
// elements are contracted (nkb >= 1).  PR (with ES = 2): only waves kWaves .. 2 kWaves - 1 (one
// per SIMD) issue the DMAs, twice their share each; the other wave of each SIMD only reads LDS
// and issues MFMAs, so no DMA that waits for room in the vector memory pipeline ever holds up
// its MFMAs (a wave issues in order).  TG: token groups (waves / ES); TG = 2 (with ES = 2, NB = 1)
// makes a 4-wave tile of 64 B rows, for batches too small to give every CU even 128 B rows; with
// PR it has 4 more waves (kWaves .. 2 kWaves - 1) that only issue the DMAs and hold no product,
// so that each SIMD again pairs a multiplying wave with a DMA-issuing one.
// NXR / NWR: slots of the B and A rings (each stream runs one stage fewer ahead); a B slot holds
// the tile's 32 TG NB rows (rows-contiguous layout), an A slot 256 rows.
template <int AUX_A, int AUX_B, class LA = RowsK, class LB = RowsK, int NB = kNB, int ES = 1, bool PR = false,
          int TG = kWaves, int NXR = kNX, int NWR = kNW>
struct Stream {
  static constexpr int kNXr = NXR, kPXr = NXR - 1, kNWr = NWR, kPWr = NWR - 1;
  static constexpr int kUnr = ring_lcm(NXR, NWR);  // slots are compile-time constants in the loop
  static constexpr int kSlotB = LB::kReads == 1 ? 32 * TG * NB * kRowB : kSlot;  // bytes of a B slot
  static_assert(NXR + NWR <= 8 && NXR <= 4 && NWR <= 4 && NXR >= 2 && NWR >= 2, "ring shape");
  static_assert(NXR * kSlotB + NWR * kSlot <= 160 * 1024, "LDS");
  static_assert(kPXr >= kPWr, "the vmcnt budget assumes the B stream runs at least as far ahead");
  static_assert(NB == kNB || (NB == 1 && LB::kReads == 1), "a 128-row B tile is laid out rows-contiguous-in-k");
  // Eight waves sharing the DMAs split a slot over 8: only rows-contiguous layouts lay out that way
  // (with PR four waves issue them, as in the 4-wave tile).
  static_assert(ES == 1 || (ES == 2 && (PR || (LA::kReads == 1 && LB::kReads == 1))), "the 8-wave DMA split");
  static_assert(!PR || (ES == 2 && (TG == kWaves || TG == 2)), "DMA-issuing waves need a second wave per SIMD");
  static_assert(TG == kWaves || (TG == 2 && ES == 2 && NB == 1 && LA::kReads == 1 && LB::kReads == 1),
                "the 64-row B tile: 4 multiplying waves, rows-contiguous-in-k");
  static constexpr int kWavesS = TG * ES;
  static constexpr int kMBw = kMB / ES;  // A blocks per wave
  // Waves that issue the DMAs, and DMA instructions per issuing wave per stage (1 KiB each): A's
  // 256 rows, B's 32 TG NB rows (128-byte row segments), over the waves that issue them.
  static constexpr int kSharers = PR ? kWaves : kWavesS;
  static constexpr int kDmaA = kDma * kWaves / kSharers;
  static constexpr int kDmaB = TG * NB * 4 / kSharers;
  // VMEM instructions a wave issues after the later of stage j's DMAs, when it must have stage j.
  // Stage j's A rows go out kPWr iterations ahead, followed in the same iteration by the B rows of
  // stage j + kPXr - kPWr: when the B ring runs further ahead, those are later stages' rows (stage
  // j's B rows went out earlier) and may still be in flight; with equal depths they are stage j's
  // own B rows, and only the (kPWr - 1) later iterations may be.
  static constexpr int kBudget = (kPXr > kPWr ? kDmaB : 0) + (kDmaA + kDmaB) * (kPWr - 1);
  // The same count by walking the issue order (prologue and loop alike: iteration v issues A rows
  // of stage v + kPWr, when >= 0, then B rows of stage v + kPXr): the instructions issued after
  // the last DMA of stage j, up to the wait at the top of iteration j.  In-order completion makes
  // "vmcnt <= kBudget" imply stage j has landed exactly when kBudget is at most this count.
  static constexpr int issued_after(int j) {
    int seq = 0, last = -1;
    for (int v = -kPXr; v < j; ++v) {
      if (v + kPWr >= 0) {
        seq += kDmaA;
        if (v + kPWr == j) last = seq;
      }
      seq += kDmaB;
      if (v + kPXr == j) last = seq;
    }
    return seq - last;
  }
  static constexpr bool budget_holds() {
    for (int j = 0; j < 2 * kUnr; ++j)
      if (kBudget > issued_after(j)) return false;
    return kBudget == issued_after(2 * kUnr);  // and no tighter than it need be in steady state
  }
  static_assert(budget_holds(), "the vmcnt budget must cover both DMA groups of the stage waited for");
  __amdgpu_buffer_rsrc_t ar, br, none;
  uint32_t voa[kDmaA], vob[kDmaB];
  uint32_t wave_off_a, wave_off_b, a_stage, b_stage;
  int nkb;
  // Rotation of the k loop: stage j reads the operands' stage (j + rot) mod nkb (0 <= rot < nkb).
  // Both operands rotate together, so the product is the same sum taken from another starting
  // stage.  Workgroups with different rotations read different columns at the same moment.
  int rot = 0;
  bool issues;  // this wave issues DMAs
  Slots sl;

  // a_bytes / b_bytes: the readable bytes of each operand from its base (rows past them read 0).
  __device__ __forceinline__ void init(const void* a, uint32_t a_bytes, uint32_t a_row_bytes, const void* b,
                                       uint32_t b_bytes, uint32_t b_row_bytes, int n_stages, int wave, int lane,
                                       Slots slots) {
    ar = make_rsrc(a, a_bytes);
    br = make_rsrc(b, b_bytes);
    none = make_rsrc(a, 0u);
    nkb = n_stages;
    sl = slots;
    issues = !PR || wave >= kWaves;
    const int dw = PR ? (wave >= kWaves ? wave - kWaves : 0) : wave;  // the wave's share of the DMAs
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) voa[i] = LA::dma_off(dw, lane, i, a_row_bytes, 256 / kSharers);
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) vob[i] = LB::dma_off(dw, lane, i, b_row_bytes, 32 * TG * NB / kSharers);
    wave_off_a = (uint32_t)dw * (kDmaA * 1024);  // A: 64 rows x 128 B or 16 rows x 512 B
    wave_off_b = (uint32_t)dw * (kDmaB * 1024);
    a_stage = LA::stage_bytes(a_row_bytes);
    b_stage = LB::stage_bytes(b_row_bytes);
  }

  // Byte offset of logical stage v (< nkb) in the operand's k direction, after the rotation.
  // Stages v >= nkb are the trailing dummies: their offset is never read.
  __device__ __forceinline__ uint32_t phys(int v) const {
    const int p = v + rot;
    return (uint32_t)(p >= nkb ? p - nkb : p);
  }

  // Stages 0..kPXr-1 of B and 0..kPWr-1 of A, issued in the same order the steady state uses
  // (A first, then B, per virtual iteration).
  __device__ __forceinline__ void prologue() {
    if (!issues) return;
#pragma unroll
    for (int vi = -kPXr; vi < 0; ++vi) {
      if (vi + kPWr >= 0)
        dma_rows<AUX_A, kDmaA>(ar, none, sl.w((vi + kPWr) % kNWr) + wave_off_a, voa, phys(vi + kPWr) * a_stage,
                               vi + kPWr < nkb);
      dma_rows<AUX_B, kDmaB>(br, none, sl.x((vi + kPXr) % kNXr) + wave_off_b, vob, phys(vi + kPXr) * b_stage,
                             vi + kPXr < nkb);
    }
  }

  // acc <- the product over all nkb stages (after prologue()).  On return every DMA has landed
  // and every wave is past its last operand read (the slots may be reused).  The DMA-only waves
  // of the 64-row PR tile leave acc untouched.
  __device__ __forceinline__ void run(f32x16 (&acc)[kMBw][NB], int wave, int lane) {
    if constexpr (PR) {
      if (!issues)
        run_as<false>(acc, wave, lane);
      else if constexpr (TG == kWaves)
        run_as<true>(acc, wave, lane);
      else
        run_dma_only();
    } else {
      run_as<true>(acc, wave, lane);
    }
  }

  // A wave that only feeds the rings: the same waits, barriers and DMAs per stage as run_as<true>,
  // no LDS reads and no MFMAs.
  __device__ __forceinline__ void run_dma_only() {
    int j0 = 0;
    do {
#pragma unroll
      for (int u = 0; u < kUnr; ++u) {
        const int j = j0 + u;
        if (j >= nkb) break;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kBudget) & ~(15 << 8));
        bare_barrier();
        dma_rows<AUX_A, kDmaA>(ar, none, sl.w((u + kPWr) % kNWr) + wave_off_a, voa, phys(j + kPWr) * a_stage,
                               j + kPWr < nkb);
        dma_rows<AUX_B, kDmaB>(br, none, sl.x((u + kPXr) % kNXr) + wave_off_b, vob, phys(j + kPXr) * b_stage,
                               j + kPXr < nkb);
      }
      j0 += kUnr;
    } while (j0 < nkb);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & ~(15 << 8));
    bare_barrier();
  }

  template <bool DMA>
  __device__ __forceinline__ void run_as(f32x16 (&acc)[kMBw][NB], int wave, int lane) {
    typename LA::Lane la;
    typename LB::Lane lb;
    la.init(lane);
    lb.init(lane);

#pragma unroll
    for (int mb = 0; mb < kMBw; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;
    const int ea = (wave % ES) * kMBw;  // first A block of the wave
    const int tb = (wave / ES) * NB;    // first B block of the wave

    // nkb >= 1 always: a do-while tells the compiler so, and spares it a second, never-run copy
    // of the 256 zero accumulators held across the loop.
    int j0 = 0;
    do {
#pragma unroll
      for (int u = 0; u < kUnr; ++u) {
        const int j = j0 + u;
        if (j >= nkb) break;
        // Own DMAs of stage j are done; after the barrier everyone's are, and every wave has
        // finished reading stage j - 1, whose slots the DMAs below overwrite.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA ? kBudget : 63) & ~(15 << 8));  // and lgkmcnt(0)
        bare_barrier();
        // A DMAs at the head of the stage (they must precede this stage's B DMAs for the vmcnt
        // budget); the B DMAs are spread over the MFMA stream below, so that a DMA waiting for
        // room in the vector memory pipeline only delays MFMAs already queued.
        if constexpr (DMA) {
          dma_rows<AUX_A, kDmaA>(ar, none, sl.w((u + kPWr) % kNWr) + wave_off_a, voa, phys(j + kPWr) * a_stage,
                                 j + kPWr < nkb);
          __builtin_amdgcn_sched_barrier(0);
          dma_rows<AUX_B, kDmaB>(br, none, sl.x((u + kPXr) % kNXr) + wave_off_b, vob, phys(j + kPXr) * b_stage,
                                 j + kPXr < nkb);
        }
        const unsigned char* ws = sl.w(u % kNWr);
        const unsigned char* xs = sl.x(u % kNXr);
        // Operand fragments are double-buffered: the LDS reads of k-step s + 1 go out before
        // the 16 MFMAs of k-step s, so their latency hides behind 512 MFMA cycles (one wave per
        // SIMD has no other wave to hide it).
        bf16x8 a[2][kMBw], b[2][NB];
        auto fetch = [&](int buf, int s) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) b[buf][nb] = lb.frag(xs, tb + nb, s);
#pragma unroll
          for (int mb = 0; mb < kMBw; ++mb) a[buf][mb] = la.frag(ws, ea + mb, s);
        };
        fetch(0, 0);
        fetch(1, 1);
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          if (s >= 1 && s + 1 < kKSteps) fetch((s + 1) & 1, s + 1);
#pragma unroll
          for (int mb = 0; mb < kMBw; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][mb], b[s & 1][nb], acc[mb][nb], 0, 0, 0);
        }
        // Issue order for the scheduler: reads of steps 0 and 1; then per step its MFMAs with
        // kDma / kKSteps B DMAs slotted between them, and the reads of step s + 2.
        // One B DMA after every kMfmaPerDma MFMAs: several per k-step, or one every few k-steps.
        constexpr int kMfmaStage = kKSteps * kMBw * NB;
        static_assert(kMfmaStage % kDmaB == 0 && ((kMfmaStage / kDmaB) % (kMBw * NB) == 0 ||
                                                  (kMBw * NB) % (kMfmaStage / kDmaB) == 0), "DMA interleave");
        constexpr int kMfmaPerDma = kMfmaStage / kDmaB;
        constexpr int kReadsStep = kMBw * LA::kReads + NB * LB::kReads;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kReadsStep, 0);  // DS reads, steps 0 and 1
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          if constexpr (!DMA) {
            __builtin_amdgcn_sched_group_barrier(0x008, kMBw * NB, 0);  // MFMAs, step s
          } else if constexpr (kMfmaPerDma <= kMBw * NB) {
#pragma unroll
            for (int q = 0; q < kMBw * NB / kMfmaPerDma; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerDma, 0);  // MFMAs, step s
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);            // one B DMA
            }
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, kMBw * NB, 0);  // MFMAs, step s
            if ((s + 1) % (kMfmaPerDma / (kMBw * NB)) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          if (s + 2 < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, kReadsStep, 0);  // DS reads, step s + 2
        }
      }
      j0 += kUnr;
    } while (j0 < nkb);

    // Drain the trailing dummy DMAs (they write slots the caller may reuse) and let every wave
    // finish its last operand reads.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0) & ~(15 << 8));
    bare_barrier();
  }
};

}  // namespace tile
}  // namespace elb

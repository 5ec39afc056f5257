/*
 * elb.h - sigmoid Top-K MoE router and expert-bias load balancing on one MI355X (gfx950).
 *
 * C ABI.  Every array argument is a DEVICE pointer owned by the caller; the library never
 * allocates, frees or keeps memory or state between calls.  Every call is asynchronous on
 * `stream` (a hipStream_t; NULL means the default stream) and returns as soon as its
 * kernels are queued.  Arguments are checked synchronously, before any launch: a bad
 * argument returns an error code and queues nothing.  Faults inside a kernel surface at
 * the caller's next synchronisation, as usual in HIP.  No C++ exception crosses the ABI.
 * All functions are thread-safe and re-entrant (no global mutable state).
 *
 * What is computed, per token t and routed expert i (N_r = n_experts):
 *   z_{t,i} = u_t . e_i                      router logit (no bias term)
 *   s_{t,i} = 1 / (1 + exp(-z_{t,i}))        sigmoid score, per expert, not normalised
 *   the K experts with the largest s_{t,i} + b_i are chosen; the bias is used only for
 *   this choice, and the gates come from s alone.
 *   [SMEBU Load Balancing (AI Engineer Exhaustive study note), "How it works", eq. (17);
 *    Arcee Trinity Large Technical Report (paperlayer.ai summary), section 2.3;
 *    hotdry blog post on Trinity Large MoE routing, section on sigmoid routing and Top-K]
 * and once per optimizer step the bias b is moved towards balanced expert loads n_i by
 * SMEBU (eq. (23)-(28) of the study note), or by the Nano/Mini sign step (eq. (20)-(22)),
 * or by the unclamped linear step the note contrasts them with.
 */
#ifndef ELB_H
#define ELB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ELB_VERSION 10800 /* major * 10000 + minor * 100 + patch */

typedef struct ihipStream_t* elb_stream_t; /* hipStream_t; NULL = default stream */

typedef enum {
  ELB_OK = 0,
  ELB_ERR_NULL = 1,        /* a required pointer is NULL                         */
  ELB_ERR_SHAPE = 2,       /* a size is outside the supported range              */
  ELB_ERR_UNSUPPORTED = 3, /* unknown dtype, mode or flag bit                    */
  ELB_ERR_ALIGN = 4,       /* a pointer or row is not 16-byte aligned            */
  ELB_ERR_WORKSPACE = 5,   /* workspace smaller than elb_dispatch_workspace_bytes */
  ELB_ERR_LAUNCH = 6       /* the HIP runtime refused a launch (e.g. wrong GPU)  */
} elb_status;

typedef enum { ELB_F32 = 0, ELB_BF16 = 1 } elb_dtype;

typedef enum {
  ELB_MODE_SMEBU = 0,  /* eq. (23)-(28): tanh-clamped, re-centred, with momentum       */
  ELB_MODE_SIGN = 1,   /* eq. (20)-(22): gamma * sign(nbar - n_i), then re-centre b     */
  ELB_MODE_LINEAR = 2  /* SMEBU with the clamp removed: db_i = lambda * v_i            */
} elb_mode;

/* Flags of elb_router_forward. */
enum {
  ELB_GATES_RAW = 1u << 0,         /* gates = s of the chosen experts, instead of s divided
                                      by its sum over the K chosen (the default)              */
  ELB_ACCUMULATE_COUNTS = 1u << 1, /* add this batch's loads into `counts` (several
                                      micro-batches per optimizer step) instead of
                                      overwriting them                                      */
  ELB_FORCE_GENERIC = 1u << 2      /* use the shape-generic kernel even where the MFMA
                                      kernel applies (tests compare the two)                 */
};

/* Flags of elb_router_backward (beside ELB_GATES_RAW). */
enum {
  ELB_DX_BF16 = 1u << 3 /* dx is written in bf16 (round to nearest even) instead of fp32 */
};

/* Flags of elb_balance_params. */
enum {
  ELB_CLEAR_COUNTS = 1u << 0 /* after the update, set `counts` to zero, so the next step's
                                elb_router_forward can add into it (ELB_ACCUMULATE_COUNTS)
                                without a separate reset                                   */
};

typedef struct {
  int32_t mode;   /* elb_mode                                                     */
  float lambda;   /* SMEBU / linear step size (Trinity Large: 5e-4)                 */
  float beta;     /* momentum factor (Trinity Large: 0.5)                           */
  float kappa;    /* tanh slope (Trinity Large: 2)                                  */
  float gamma;    /* sign-step size                                                 */
  uint32_t flags; /* ELB_CLEAR_COUNTS or 0                                          */
} elb_balance_params;

/*
 * Router forward for one batch of tokens.
 *   x        [T, d] hidden states u_t, row-major, elements of `dtype` (fp32 or bf16).
 *   w        [n_experts, d] router weight rows e_i (expert centroids), row-major, `dtype`.
 *   bias     [n_experts] fp32 expert bias b_i.
 *   topk_idx [T, k] int32 out: chosen experts, in descending s + b; equal values go to the
 *            lower expert index.
 *   gates    [T, k] fp32 out: s of the chosen experts divided by their sum over the k
 *            chosen ("normalized scores", report section 2.3), or s itself with
 *            ELB_GATES_RAW.  Never depends on b.
 *   counts   [n_experts] int32 in/out: n_i, the number of (token, slot) pairs routed to
 *            expert i.  Overwritten unless ELB_ACCUMULATE_COUNTS is set.
 *   logits   [T, n_experts] fp32 out, or NULL: z_{t,i} (a parity aid; costs bandwidth).
 *   lse      [T] fp32 out, or NULL: log sum_i exp(z_{t,i}), the per-token term of the
 *            router z-loss (talk summary "Arcee Halts 400B Blackwell Model Collapse...",
 *            section "Precision Fallbacks, Loss Stabilization, and MaxVio ...").
 * Supported: 0 <= T, T * k < 2^31; 1 <= k <= min(8, n_experts); n_experts <= 256;
 * d >= 1 with every row 16-byte aligned (d % 8 == 0 for bf16, d % 4 == 0 for fp32);
 * x and w 16-byte aligned.  bf16 inputs with d % 64 == 0 run on the MFMA kernel, which ranks
 * s + b by 23-bit fixed-point codes of s + b - min b: differences resolve down to 2^(E-22),
 * where 2^E <= 1 + max b - min b < 2^(E+1) (2.4e-7 for any bias spread below 1, finer than
 * 1e-3 for any spread below 8191; closer candidates go to the lower expert index); the
 * generic kernel (ELB_FORCE_GENERIC) compares s + b exactly in fp32.  Inputs must be finite.
 * Errors: ELB_ERR_NULL, ELB_ERR_SHAPE, ELB_ERR_ALIGN, ELB_ERR_UNSUPPORTED (dtype or flag),
 * ELB_ERR_LAUNCH.
 */
elb_status elb_router_forward(const void* x, int32_t dtype, int64_t T, int32_t d, const void* w,
                              const float* bias, int32_t n_experts, int32_t k, uint32_t flags,
                              int32_t* topk_idx, float* gates, int32_t* counts, float* logits,
                              float* lse, elb_stream_t stream);

/*
 * Bytes of device workspace elb_router_dispatch needs for these sizes (0 when T == 0).
 * Errors are reported as 0 only when the sizes are themselves invalid.
 */
size_t elb_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t n_experts);

/*
 * Counting-sort dispatch of the flat assignments j = t * k + slot by expert (the pages
 * define none; this is the plain stable counting sort):
 *   offsets  [n_experts + 1] int32 out: bucket e is perm[offsets[e] .. offsets[e+1]).
 *   perm     [T * k] int32 out: flat positions j, grouped by expert, ascending within each
 *            expert.
 *   inv_perm [T * k] int32 out, or NULL: perm[inv_perm[j]] == j.
 *   workspace: device memory of at least elb_dispatch_workspace_bytes(T, k, n_experts)
 *            bytes, 16-byte aligned; its contents on entry do not matter.
 * topk_idx entries must lie in [0, n_experts).  Errors: ELB_ERR_NULL, ELB_ERR_SHAPE,
 * ELB_ERR_WORKSPACE, ELB_ERR_ALIGN, ELB_ERR_LAUNCH.
 */
elb_status elb_router_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t n_experts,
                               void* workspace, size_t workspace_bytes, int32_t* offsets,
                               int32_t* perm, int32_t* inv_perm, elb_stream_t stream);

/*
 * elb_router_dispatch for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same sort, the same
 * outputs bit for bit, with no workspace argument.  Its workspace is a static device array of
 * 8 MiB inside the library, one copy per GPU, held until the process ends; the call allocates
 * nothing and frees nothing.  Sizes whose elb_dispatch_workspace_bytes exceeds 8 MiB (at
 * n_experts = 256: more than 2,096,128 tokens) are refused with ELB_ERR_WORKSPACE.  The first
 * call on a GPU looks up that GPU's copy (hipGetSymbolAddress, with the device of `stream`
 * made current for the lookup).  Every call on one GPU shares its copy: calls that overlap on
 * one GPU (on different streams, or from several threads without ordering) race and give
 * wrong results.  Errors: ELB_ERR_NULL, ELB_ERR_SHAPE, ELB_ERR_WORKSPACE, ELB_ERR_ALIGN,
 * ELB_ERR_LAUNCH (also when the lookup fails).
 */
elb_status elb_router_dispatch_noalloc(const int32_t* topk_idx, int64_t T, int32_t k,
                                       int32_t n_experts, int32_t* offsets, int32_t* perm,
                                       int32_t* inv_perm, elb_stream_t stream);

/*
 * One expert-bias update from one optimizer step's loads (study note eq. (20)-(28)).
 *   counts   [n_experts] int32: n_i for the step.
 *   bias     [n_experts] fp32 in/out: b.
 *   momentum [n_experts] fp32 in/out: m (SMEBU and linear modes; untouched by SIGN).
 *   delta_b  [n_experts] fp32 out, or NULL: the applied step (re-centred db for SMEBU and
 *            LINEAR, gamma * sign(nbar - n_i) for SIGN).
 *   maxvio   [2] fp32 out, or NULL: {max n / min n, (max n - nbar) / nbar} of `counts`.
 * SMEBU:  v = (nbar - n) / nbar; db = lambda * tanh(kappa * v); db -= mean(db);
 *         m = beta * m + (1 - beta) * db; b += m.
 * SIGN:   b += gamma * sign(nbar - n); b -= mean(b).
 * LINEAR: as SMEBU with tanh(kappa * v) replaced by v.
 * When every count is 0 the step is skipped (b, m unchanged, delta_b = 0, maxvio NaN).
 * With ELB_CLEAR_COUNTS in params.flags, `counts` is zeroed once it has been read.
 * Supported: 1 <= n_experts <= 1024.  Errors: ELB_ERR_NULL, ELB_ERR_SHAPE,
 * ELB_ERR_UNSUPPORTED (mode or flag), ELB_ERR_LAUNCH.
 */
elb_status elb_smebu_update(int32_t* counts, int32_t n_experts, elb_balance_params params,
                            float* bias, float* momentum, float* delta_b, float* maxvio,
                            elb_stream_t stream);

/*
 * One routed step: elb_router_forward, then elb_router_dispatch of its topk_idx, then (when
 * `update` is non-zero) elb_smebu_update from `counts`.  Each field means what the argument of
 * the same name means in those calls, and the same checks apply.  Compared with the three
 * calls in a row, the router kernel stores each 256-token tile's loads in the dispatch
 * workspace (the dispatch does not count them again; bf16 inputs with d % 64 == 0 only, else
 * a counting pass runs), the dispatch's scan over those tile loads writes (with
 * ELB_ACCUMULATE_COUNTS: adds) `counts` in place of the router kernel's per-tile atomics, and
 * the bias update runs inside the dispatch's launch: two kernels in all (router, dispatch).
 * The counts are the same integers either way.  The update sees `counts` after this batch's loads were added, and changes
 * `bias` only after the router kernel has read it, so the next step routes with the new bias.
 * A training loop with one batch per optimizer step sets ELB_ACCUMULATE_COUNTS and
 * ELB_CLEAR_COUNTS and never resets `counts` itself (they must start at zero).
 * offsets, perm and inv_perm all NULL: no dispatch (workspace is then not used); the update,
 * if any, runs as its own launch after the router kernel.
 * The MFMA router takes 128-token tiles for batches of at most 128 x 256 tokens and 64-token
 * tiles for at most 64 x 256 (so that every compute unit gets a tile); the dispatch then counts
 * the loads itself.
 * timing: NULL, or an array of three hipEvent_t (any may be NULL): [0] takes the end time
 * stamp of an empty one-wave kernel launched right before the router kernel, [1] the router
 * kernel's own end, [2] the end of the step's last kernel (all through hipExtLaunchKernel; with
 * T == 0 an empty kernel stands in for the router kernel, and when the router kernel is the
 * step's only kernel [2] goes to an empty kernel after it).  Events created with
 * hipEventDisableSystemFence are bound to the kernels' time stamps; with other events the
 * runtime records markers after the kernels, which adds their cost to the interval.  Either way the next kernel starts a few
 * microseconds later than it would without the event.  A measuring aid.
 */
typedef struct {
  /* elb_router_forward */
  const void* x;
  int32_t dtype;
  int64_t T;
  int32_t d;
  const void* w;
  float* bias;
  int32_t n_experts;
  int32_t k;
  uint32_t flags;
  int32_t* topk_idx;
  float* gates;
  int32_t* counts;
  float* logits;
  float* lse;
  float* zloss; /* [1] out, or NULL: elb_zloss of this batch's lse (lse must then be given) */
  /* elb_router_dispatch */
  void* workspace;
  size_t workspace_bytes;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  /* elb_smebu_update, run when update != 0 */
  int32_t update;
  elb_balance_params params;
  float* momentum;
  float* delta_b;
  float* maxvio;
  /* measuring aid */
  void* const* timing;
} elb_step_args;

elb_status elb_route_step(const elb_step_args* args, elb_stream_t stream);

/*
 * Bias updates of n_layers MoE layers in one launch, each from its own loads: the arguments of
 * elb_smebu_update stacked layer-major.  counts, bias, momentum, delta_b are [n_layers][n_experts]
 * and maxvio is [n_layers][2] (per-layer MaxVio telemetry).  Layer l's result is exactly what
 * elb_smebu_update gives on layer l's rows; layers do not interact (the update is stated per
 * router: "SMEBU Load Balancing", "How it works").  Supported: n_layers >= 1,
 * 1 <= n_experts <= 1024, n_layers * n_experts < 2^31.  Errors as elb_smebu_update.
 */
elb_status elb_smebu_update_layers(int32_t* counts, int32_t n_layers, int32_t n_experts, elb_balance_params params,
                                   float* bias, float* momentum, float* delta_b, float* maxvio,
                                   elb_stream_t stream);

/*
 * Router z-loss of one batch from the per-token log-sum-exps of elb_router_forward:
 *   out[0] = mean_t lse[t]^2   (0 when T == 0)
 * (talk summary "Arcee Halts 400B Blackwell Model Collapse...", section "Precision Fallbacks,
 * Loss Stabilization, and MaxVio ..."; the weight is applied by the caller).  Summed in
 * float64 in a fixed order: deterministic.  Errors: ELB_ERR_NULL, ELB_ERR_SHAPE (T < 0),
 * ELB_ERR_ALIGN, ELB_ERR_LAUNCH.
 */
elb_status elb_zloss(const float* lse, int64_t T, float* out, elb_stream_t stream);

/*
 * Expert-contiguous copy of the token rows (the gather before the routed experts):
 *   x_perm[inv_perm[t * k + j]] = x[t]   for every token t and slot j,
 * so rows offsets[e] .. offsets[e+1] of x_perm are expert e's tokens, in the order of
 * elb_router_dispatch's perm.  Rows are copied bit for bit.
 *   x       [T, d] of `dtype` (fp32 or bf16), row-major; every row 16-byte aligned.
 *   inv_perm[T * k] int32: a permutation of 0 .. T*k-1 (elb_router_dispatch's inv_perm).
 *   x_perm  [T * k, d] of `dtype` out.
 * Each token row is read once.  Errors: ELB_ERR_NULL, ELB_ERR_SHAPE, ELB_ERR_UNSUPPORTED
 * (dtype), ELB_ERR_ALIGN, ELB_ERR_LAUNCH.
 */
elb_status elb_permute_rows(const void* x, int32_t dtype, int64_t T, int32_t d, int32_t k, const int32_t* inv_perm,
                            void* x_perm, elb_stream_t stream);

/*
 * Gated combine of the routed experts' outputs back to token order (Arcee Trinity Large
 * Technical Report, section 2.3: the gating scores weight the routed experts' outputs):
 *   y[t] = sum_{j=0}^{k-1} gates[t, j] * expert_out[inv_perm[t * k + j]]
 * accumulated in fp32 in slot order with fused multiply-adds.
 *   expert_out [T * k, d] of `dtype` (fp32 or bf16), rows in expert-contiguous order.
 *   gates      [T, k] fp32 (elb_router_forward's gates).
 *   y          [T, d] out, fp32 or bf16 (y_dtype; bf16 rounds to nearest even).
 * d % 8 == 0 for bf16 expert_out, d % 4 == 0 for fp32; pointers 16-byte aligned.  Errors:
 * ELB_ERR_NULL, ELB_ERR_SHAPE, ELB_ERR_UNSUPPORTED, ELB_ERR_ALIGN, ELB_ERR_LAUNCH.
 */
elb_status elb_unpermute_combine(const void* expert_out, int32_t dtype, int64_t T, int32_t d, int32_t k,
                                 const int32_t* inv_perm, const float* gates, void* y, int32_t y_dtype,
                                 elb_stream_t stream);

/*
 * Router backward: gradients of
 *   L = sum_{t,j} dgates[t,j] * gates[t,j] + zloss_coef * mean_t lse_t^2
 * with respect to the tokens and the router weights, at the forward's selection topk_idx (the
 * bias gets no gradient: it only acts inside Top-K).  The pages give no backward; this is the
 * chain rule through the forward above (gates normalised over the K chosen unless
 * ELB_GATES_RAW; the z-loss of the talk summary "Arcee Halts 400B Blackwell Model Collapse...",
 * section "Precision Fallbacks, Loss Stabilization, and MaxVio ..."):
 *   dL/dz_{t,i_j} = dL/ds_j s_j (1 - s_j),  dL/ds_j = (G_j - sum_m G_m g_m) / S (raw: G_j),
 *   dL/dz_{t,i}  += (2 zloss_coef / T) lse_t softmax(z_t)_i,
 *   dx = dL/dZ W [T, d] fp32 (bf16 with ELB_DX_BF16, rounded to nearest even),
 *   dw = dL/dZ^T X [n_experts, d] fp32 (either may be NULL).
 * The logits are recomputed from x and w on the matrix cores; dL/dz is rounded to bf16 before
 * the two products, which accumulate in fp32.
 *   x, w, topk_idx as in elb_router_forward (bf16 only, d % 64 == 0); dgates [T, k] fp32;
 *   dx and dw 16-byte aligned.
 *   workspace: at least elb_backward_workspace_bytes(T, d, n_experts) bytes, 256-byte aligned;
 *   contents on entry do not matter.  topk_idx entries must lie in [0, n_experts).
 * Supported: 0 <= T <= 2^22, T * k < 2^31, 1 <= k <= min(8, n_experts), n_experts <= 256.
 * Errors: ELB_ERR_NULL, ELB_ERR_SHAPE, ELB_ERR_UNSUPPORTED (dtype, d % 64, flag other than
 * ELB_GATES_RAW and ELB_DX_BF16), ELB_ERR_ALIGN, ELB_ERR_WORKSPACE, ELB_ERR_LAUNCH.
 */
size_t elb_backward_workspace_bytes(int64_t T, int32_t d, int32_t n_experts);
elb_status elb_router_backward(const void* x, int32_t dtype, int64_t T, int32_t d, const void* w, int32_t n_experts,
                               int32_t k, uint32_t flags, const int32_t* topk_idx, const float* dgates,
                               float zloss_coef, void* dx, float* dw, void* workspace, size_t workspace_bytes,
                               elb_stream_t stream);

/*
 * MaxVio of one step's loads: out[0] = max n / min n (the talk's definition, section
 * "The MaxVio Metric and the Day-4 Crisis"; +inf when an expert got nothing), out[1] =
 * (max n - nbar) / nbar.  Both NaN when every count is 0.  Supported: 1 <= n_experts <= 1024.
 */
elb_status elb_maxvio(const int32_t* counts, int32_t n_experts, float* out, elb_stream_t stream);

/*
 * A plain streaming read of `bytes` bytes at src: out[0] ^= the XOR of all its 32-bit words
 * (the caller sets out[0] first).  Not part of the routed step: it is the measured reference
 * for the router's HBM roofline (the bandwidth one read-only pass over HBM reaches on this
 * GPU, reported beside the published peak), and the XOR lets a test check every byte was read.
 * src 16-byte aligned, bytes % 16 == 0 (0 is a no-op), out 4-byte aligned.  Errors: ELB_ERR_NULL,
 * ELB_ERR_SHAPE (bytes not a multiple of 16), ELB_ERR_ALIGN, ELB_ERR_LAUNCH.
 */
elb_status elb_stream_xor(const void* src, size_t bytes, uint32_t* out, elb_stream_t stream);

/* Static description of a status code (never NULL). */
const char* elb_status_str(elb_status status);

/* ELB_VERSION of the built library. */
int elb_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ELB_H */

// C-ABI entry points of libelb: argument checks, then kernel selection and launch.
// Every check happens before anything is queued; include/elb.h states the contract.
#include "../../include/elb.h"

#include "elb_kernels.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

elb_status from_hip(hipError_t e) { return e == hipSuccess ? ELB_OK : ELB_ERR_LAUNCH; }

constexpr uint32_t kKnownFlags = ELB_GATES_RAW | ELB_ACCUMULATE_COUNTS | ELB_FORCE_GENERIC;
constexpr uint32_t kKnownBalanceFlags = ELB_CLEAR_COUNTS;

elb_status check_forward(const void* x, int32_t dtype, int64_t T, int32_t d, const void* w, const float* bias,
                         int32_t n_experts, int32_t k, uint32_t flags, const int32_t* topk_idx, const float* gates,
                         const int32_t* counts, const float* logits, const float* lse) {
  if (w == nullptr || bias == nullptr || counts == nullptr) return ELB_ERR_NULL;
  if (T > 0 && (x == nullptr || topk_idx == nullptr || gates == nullptr)) return ELB_ERR_NULL;
  if (dtype != ELB_F32 && dtype != ELB_BF16) return ELB_ERR_UNSUPPORTED;
  if (flags & ~kKnownFlags) return ELB_ERR_UNSUPPORTED;
  if (T < 0 || d < 1 || n_experts < 1 || n_experts > 256 || k < 1 || k > 8 || k > n_experts) return ELB_ERR_SHAPE;
  if (T * (int64_t)k >= (int64_t(1) << 31) || T * (int64_t)n_experts >= (int64_t(1) << 62)) return ELB_ERR_SHAPE;
  const int64_t elem = dtype == ELB_F32 ? 4 : 2;
  if ((d * elem) % 16 != 0 || !aligned(w, 16)) return ELB_ERR_ALIGN;
  if (T > 0 && (!aligned(x, 16) || !aligned(topk_idx, 16) || !aligned(gates, 16))) return ELB_ERR_ALIGN;
  if (!aligned(bias, 4) || !aligned(counts, 4) || !aligned(logits, 4) || !aligned(lse, 4)) return ELB_ERR_ALIGN;
  return ELB_OK;
}

elb_status check_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t n_experts, const void* workspace,
                          size_t workspace_bytes, const int32_t* offsets, const int32_t* perm,
                          const int32_t* inv_perm) {
  if (offsets == nullptr) return ELB_ERR_NULL;
  if (T > 0 && (topk_idx == nullptr || perm == nullptr || workspace == nullptr)) return ELB_ERR_NULL;
  if (T < 0 || k < 1 || k > 8 || n_experts < 1 || n_experts > 256) return ELB_ERR_SHAPE;
  if (T * (int64_t)k >= (int64_t(1) << 31)) return ELB_ERR_SHAPE;
  if (workspace_bytes < elb::dispatch_workspace_bytes(T, n_experts)) return ELB_ERR_WORKSPACE;
  if (!aligned(topk_idx, 4) || !aligned(offsets, 4) || !aligned(perm, 4) || !aligned(inv_perm, 4) ||
      !aligned(workspace, 16))
    return ELB_ERR_ALIGN;
  return ELB_OK;
}

elb_status check_update(const int32_t* counts, int32_t n_experts, const elb_balance_params& params, const float* bias,
                        const float* momentum, const float* delta_b, const float* maxvio) {
  if (params.mode != ELB_MODE_SMEBU && params.mode != ELB_MODE_SIGN && params.mode != ELB_MODE_LINEAR)
    return ELB_ERR_UNSUPPORTED;
  if (params.flags & ~kKnownBalanceFlags) return ELB_ERR_UNSUPPORTED;
  if (counts == nullptr || bias == nullptr) return ELB_ERR_NULL;
  if (params.mode != ELB_MODE_SIGN && momentum == nullptr) return ELB_ERR_NULL;
  if (n_experts < 1 || n_experts > 1024) return ELB_ERR_SHAPE;
  if (!aligned(counts, 4) || !aligned(bias, 4) || !aligned(momentum, 4) || !aligned(delta_b, 4) || !aligned(maxvio, 4))
    return ELB_ERR_ALIGN;
  return ELB_OK;
}

elb::BalanceArgs balance_args(int32_t* counts, int32_t n_experts, const elb_balance_params& p, float* bias,
                              float* momentum, float* delta_b, float* maxvio) {
  return elb::BalanceArgs{counts, n_experts, p.mode, p.lambda, p.beta, p.kappa, p.gamma,
                          (p.flags & ELB_CLEAR_COUNTS) ? 1 : 0, bias, momentum, delta_b, maxvio};
}

}  // namespace

extern "C" {

elb_status elb_router_forward(const void* x, int32_t dtype, int64_t T, int32_t d, const void* w, const float* bias,
                              int32_t n_experts, int32_t k, uint32_t flags, int32_t* topk_idx, float* gates,
                              int32_t* counts, float* logits, float* lse, elb_stream_t stream) {
  const elb_status st =
      check_forward(x, dtype, T, d, w, bias, n_experts, k, flags, topk_idx, gates, counts, logits, lse);
  if (st != ELB_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!(flags & ELB_ACCUMULATE_COUNTS)) {
    const hipError_t err = elb::launch_fill_i32(counts, n_experts, 0, s);
    if (err != hipSuccess) return ELB_ERR_LAUNCH;
  }
  if (T == 0) return ELB_OK;
  const elb::RouterArgs a{x,      dtype, T,      d,   w,   bias,    n_experts, k,
                          flags,  topk_idx, gates, counts, logits, lse, nullptr, 0};
  if (!(flags & ELB_FORCE_GENERIC) && elb::router_mfma_applies(a)) return from_hip(elb::launch_router_mfma(a, s));
  return from_hip(elb::launch_router_generic(a, s));
}

size_t elb_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t n_experts) {
  if (T < 0 || k < 1 || k > 8 || n_experts < 1 || n_experts > 256) return 0;
  if (T * (int64_t)k >= (int64_t(1) << 31)) return 0;
  return elb::dispatch_workspace_bytes(T, n_experts);
}

elb_status elb_router_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t n_experts, void* workspace,
                               size_t workspace_bytes, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                               elb_stream_t stream) {
  const elb_status st =
      check_dispatch(topk_idx, T, k, n_experts, workspace, workspace_bytes, offsets, perm, inv_perm);
  if (st != ELB_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(elb::launch_dispatch(topk_idx, T, k, n_experts, workspace, false, nullptr, false, nullptr, offsets, perm,
                                       inv_perm, s));
}

elb_status elb_router_dispatch_noalloc(const int32_t* topk_idx, int64_t T, int32_t k, int32_t n_experts,
                                       int32_t* offsets, int32_t* perm, int32_t* inv_perm, elb_stream_t stream) {
  // The checks of elb_router_dispatch, with the static scratch standing in for the workspace.
  if (offsets == nullptr) return ELB_ERR_NULL;
  if (T > 0 && (topk_idx == nullptr || perm == nullptr)) return ELB_ERR_NULL;
  if (T < 0 || k < 1 || k > 8 || n_experts < 1 || n_experts > 256) return ELB_ERR_SHAPE;
  if (T * (int64_t)k >= (int64_t(1) << 31)) return ELB_ERR_SHAPE;
  if (elb::dispatch_workspace_bytes(T, n_experts) > elb::kDispatchScratchBytes) return ELB_ERR_WORKSPACE;
  if (!aligned(topk_idx, 4) || !aligned(offsets, 4) || !aligned(perm, 4) || !aligned(inv_perm, 4))
    return ELB_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (elb::dispatch_scratch(s, &ws) != hipSuccess) return ELB_ERR_LAUNCH;
  return from_hip(elb::launch_dispatch(topk_idx, T, k, n_experts, ws, false, nullptr, false, nullptr, offsets, perm, inv_perm, s));
}

elb_status elb_smebu_update(int32_t* counts, int32_t n_experts, elb_balance_params params, float* bias,
                            float* momentum, float* delta_b, float* maxvio, elb_stream_t stream) {
  const elb_status st = check_update(counts, n_experts, params, bias, momentum, delta_b, maxvio);
  if (st != ELB_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(elb::launch_balance(balance_args(counts, n_experts, params, bias, momentum, delta_b, maxvio), s));
}

elb_status elb_route_step(const elb_step_args* args, elb_stream_t stream) {
  if (args == nullptr) return ELB_ERR_NULL;
  const elb_step_args& a = *args;
  elb_status st = check_forward(a.x, a.dtype, a.T, a.d, a.w, a.bias, a.n_experts, a.k, a.flags, a.topk_idx, a.gates,
                                a.counts, a.logits, a.lse);
  if (st != ELB_OK) return st;
  // No dispatch outputs at all: route (and update) only.
  const bool dispatch = a.offsets != nullptr || a.perm != nullptr || a.inv_perm != nullptr;
  if (dispatch) {
    st = check_dispatch(a.topk_idx, a.T, a.k, a.n_experts, a.workspace, a.workspace_bytes, a.offsets, a.perm,
                        a.inv_perm);
    if (st != ELB_OK) return st;
  }
  if (a.update != 0) {
    st = check_update(a.counts, a.n_experts, a.params, a.bias, a.momentum, a.delta_b, a.maxvio);
    if (st != ELB_OK) return st;
  }
  if (a.zloss != nullptr && a.lse == nullptr) return ELB_ERR_NULL;
  if (!aligned(a.zloss, 4)) return ELB_ERR_ALIGN;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool accumulate = (a.flags & ELB_ACCUMULATE_COUNTS) != 0;
  // With a dispatch, the expert loads come from its scan over the per-tile loads (which it needs
  // anyway), not from the router's global atomics; it also clears them for an empty batch.
  if (!accumulate && !dispatch) {
    if (elb::launch_fill_i32(a.counts, a.n_experts, 0, s) != hipSuccess) return ELB_ERR_LAUNCH;
  }
  const elb::DispatchGeom g = elb::dispatch_geometry(a.T);
  elb::RouterArgs ra{a.x,     a.dtype,    a.T,      a.d,      a.w,     a.bias, a.n_experts,
                     a.k,     a.flags,    a.topk_idx, a.gates, dispatch ? nullptr : a.counts, a.logits, a.lse,
                     static_cast<int32_t*>(a.workspace), g.stride};
  const bool mfma = !(a.flags & ELB_FORCE_GENERIC) && elb::router_mfma_applies(ra);
  const bool loads_ready = dispatch && mfma && elb::router_mfma_full_tile(a.T);  // the router fills the table
  if (!loads_ready) ra.tile_loads = nullptr;
  hipEvent_t ev_end = nullptr;  // the end of the step's last kernel
  if (a.timing != nullptr) {
    // From the end of an empty kernel launched just before the router kernel to its end.
    if (a.timing[0] != nullptr && elb::launch_mark(static_cast<hipEvent_t>(a.timing[0]), s) != hipSuccess)
      return ELB_ERR_LAUNCH;
    ra.ev_stop = static_cast<hipEvent_t>(a.timing[1]);
    ev_end = static_cast<hipEvent_t>(a.timing[2]);
  }
  const bool router_last = a.zloss == nullptr && !dispatch && a.update == 0;
  if (a.T > 0) {
    const hipError_t err = mfma ? elb::launch_router_mfma(ra, s) : elb::launch_router_generic(ra, s);
    if (err != hipSuccess) return ELB_ERR_LAUNCH;
  } else if (ra.ev_stop != nullptr && elb::launch_mark(ra.ev_stop, s) != hipSuccess) {  // no router kernel
    return ELB_ERR_LAUNCH;
  }
  // A step of the router kernel alone: the end event follows it on an empty kernel.
  if (router_last) return ev_end != nullptr ? from_hip(elb::launch_mark(ev_end, s)) : ELB_OK;
  if (a.zloss != nullptr &&
      elb::launch_zloss(a.lse, a.T, a.zloss, s, (!dispatch && a.update == 0) ? ev_end : nullptr) != hipSuccess)
    return ELB_ERR_LAUNCH;
  const elb::BalanceArgs upd =
      balance_args(a.counts, a.n_experts, a.params, a.bias, a.momentum, a.delta_b, a.maxvio);
  if (!dispatch) return a.update != 0 ? from_hip(elb::launch_balance(upd, s, ev_end)) : ELB_OK;
  return from_hip(elb::launch_dispatch(a.topk_idx, a.T, a.k, a.n_experts, a.workspace, loads_ready, a.counts, accumulate,
                                       a.update != 0 ? &upd : nullptr, a.offsets, a.perm, a.inv_perm, s, ev_end));
}

elb_status elb_smebu_update_layers(int32_t* counts, int32_t n_layers, int32_t n_experts, elb_balance_params params,
                                   float* bias, float* momentum, float* delta_b, float* maxvio, elb_stream_t stream) {
  const elb_status st = check_update(counts, n_experts, params, bias, momentum, delta_b, maxvio);
  if (st != ELB_OK) return st;
  if (n_layers < 1 || (int64_t)n_layers * n_experts >= (int64_t(1) << 31)) return ELB_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(
      elb::launch_balance_layers(balance_args(counts, n_experts, params, bias, momentum, delta_b, maxvio), n_layers, s));
}

elb_status elb_zloss(const float* lse, int64_t T, float* out, elb_stream_t stream) {
  if (out == nullptr || (T > 0 && lse == nullptr)) return ELB_ERR_NULL;
  if (T < 0) return ELB_ERR_SHAPE;
  if (!aligned(lse, 4) || !aligned(out, 4)) return ELB_ERR_ALIGN;
  return from_hip(elb::launch_zloss(lse, T, out, reinterpret_cast<hipStream_t>(stream)));
}

elb_status elb_permute_rows(const void* x, int32_t dtype, int64_t T, int32_t d, int32_t k, const int32_t* inv_perm,
                            void* x_perm, elb_stream_t stream) {
  if (T > 0 && (x == nullptr || inv_perm == nullptr || x_perm == nullptr)) return ELB_ERR_NULL;
  if (dtype != ELB_F32 && dtype != ELB_BF16) return ELB_ERR_UNSUPPORTED;
  if (T < 0 || d < 1 || k < 1 || k > 8 || T * (int64_t)k >= (int64_t(1) << 31)) return ELB_ERR_SHAPE;
  const int64_t row_bytes = (int64_t)d * (dtype == ELB_F32 ? 4 : 2);
  if (row_bytes % 16 != 0 || !aligned(x, 16) || !aligned(x_perm, 16) || !aligned(inv_perm, 4)) return ELB_ERR_ALIGN;
  return from_hip(elb::launch_permute_rows(x, T, row_bytes, k, inv_perm, x_perm, reinterpret_cast<hipStream_t>(stream)));
}

elb_status elb_unpermute_combine(const void* expert_out, int32_t dtype, int64_t T, int32_t d, int32_t k,
                                 const int32_t* inv_perm, const float* gates, void* y, int32_t y_dtype,
                                 elb_stream_t stream) {
  if (T > 0 && (expert_out == nullptr || inv_perm == nullptr || gates == nullptr || y == nullptr)) return ELB_ERR_NULL;
  if ((dtype != ELB_F32 && dtype != ELB_BF16) || (y_dtype != ELB_F32 && y_dtype != ELB_BF16))
    return ELB_ERR_UNSUPPORTED;
  if (T < 0 || d < 1 || k < 1 || k > 8 || T * (int64_t)k >= (int64_t(1) << 31)) return ELB_ERR_SHAPE;
  if (d % (dtype == ELB_BF16 ? 8 : 4) != 0) return ELB_ERR_ALIGN;
  if (!aligned(expert_out, 16) || !aligned(y, 16) || !aligned(inv_perm, 4) || !aligned(gates, 4)) return ELB_ERR_ALIGN;
  return from_hip(elb::launch_combine(expert_out, dtype, T, d, k, inv_perm, gates, y, y_dtype,
                                      reinterpret_cast<hipStream_t>(stream)));
}

size_t elb_backward_workspace_bytes(int64_t T, int32_t d, int32_t n_experts) {
  if (T < 0 || T > (int64_t(1) << 22) || d < 64 || d % 64 != 0 || n_experts < 1 || n_experts > 256) return 0;
  return elb::backward_plan(T, d, nullptr).bytes;
}

elb_status elb_router_backward(const void* x, int32_t dtype, int64_t T, int32_t d, const void* w, int32_t n_experts,
                               int32_t k, uint32_t flags, const int32_t* topk_idx, const float* dgates,
                               float zloss_coef, void* dx, float* dw, void* workspace, size_t workspace_bytes,
                               elb_stream_t stream) {
  if (w == nullptr || workspace == nullptr) return ELB_ERR_NULL;
  if (T > 0 && (x == nullptr || topk_idx == nullptr || dgates == nullptr)) return ELB_ERR_NULL;
  if (dtype != ELB_BF16 || (flags & ~(uint32_t)(ELB_GATES_RAW | ELB_DX_BF16))) return ELB_ERR_UNSUPPORTED;
  if (T < 0 || T > (int64_t(1) << 22) || n_experts < 1 || n_experts > 256 || k < 1 || k > 8 || k > n_experts)
    return ELB_ERR_SHAPE;
  if (T * (int64_t)k >= (int64_t(1) << 31) || d < 1 || (int64_t)d * 2 * 256 >= (int64_t(1) << 30)) return ELB_ERR_SHAPE;
  if (d % 64 != 0) return ELB_ERR_UNSUPPORTED;
  if (!(zloss_coef == zloss_coef) || zloss_coef - zloss_coef != 0.0f) return ELB_ERR_SHAPE;  // NaN or infinite
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(topk_idx, 4) || !aligned(dgates, 4) || !aligned(dx, 16) ||
      !aligned(dw, 16) || !aligned(workspace, 256))
    return ELB_ERR_ALIGN;
  const elb::BackwardPlan plan = elb::backward_plan(T, d, workspace);
  if (workspace_bytes < plan.bytes) return ELB_ERR_WORKSPACE;
  if (dx == nullptr && dw == nullptr) return ELB_OK;
  const elb::BackwardArgs a{x,      T,          d,  w, n_experts, k, (flags & ELB_GATES_RAW) ? 0 : 1, topk_idx,
                            dgates, zloss_coef, dx, (flags & ELB_DX_BF16) != 0, dw};
  return from_hip(elb::launch_router_backward(a, plan, reinterpret_cast<hipStream_t>(stream)));
}

elb_status elb_maxvio(const int32_t* counts, int32_t n_experts, float* out, elb_stream_t stream) {
  if (counts == nullptr || out == nullptr) return ELB_ERR_NULL;
  if (n_experts < 1 || n_experts > 1024) return ELB_ERR_SHAPE;
  if (!aligned(counts, 4) || !aligned(out, 4)) return ELB_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const elb::BalanceArgs a{const_cast<int32_t*>(counts), n_experts, -1, 0.f, 0.f, 0.f, 0.f, 0,
                           nullptr, nullptr, nullptr, out};
  return from_hip(elb::launch_balance(a, s));
}

elb_status elb_stream_xor(const void* src, size_t bytes, uint32_t* out, elb_stream_t stream) {
  if (out == nullptr || (bytes > 0 && src == nullptr)) return ELB_ERR_NULL;
  if (bytes % 16 != 0) return ELB_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(out, 4)) return ELB_ERR_ALIGN;
  return from_hip(elb::launch_stream_xor(src, (int64_t)(bytes / 16), out, reinterpret_cast<hipStream_t>(stream)));
}

const char* elb_status_str(elb_status status) {
  switch (status) {
    case ELB_OK: return "ok";
    case ELB_ERR_NULL: return "a required pointer is NULL";
    case ELB_ERR_SHAPE: return "a size is outside the supported range";
    case ELB_ERR_UNSUPPORTED: return "unknown dtype, mode or flag";
    case ELB_ERR_ALIGN: return "a pointer or row is not aligned as required";
    case ELB_ERR_WORKSPACE: return "workspace smaller than elb_dispatch_workspace_bytes";
    case ELB_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
  }
  return "unknown status";
}

int elb_version(void) { return ELB_VERSION; }

}  // extern "C"

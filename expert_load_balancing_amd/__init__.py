"""Sigmoid Top-K MoE router with SMEBU expert-bias load balancing on AMD MI355X (gfx950).

Thin PyTorch binding over libelb.so (C ABI in include/elb.h).  These functions only check
and marshal arguments: tensors must already live on the GPU, outputs are allocated with
torch (plain device memory), and every step of the computation runs in the library's HIP
kernels on the current torch stream.  Nothing here computes the method itself.

    idx, gates, counts = router_forward(x, w, bias, k=4)
    offsets, perm, inv = router_dispatch(idx, n_experts=256)
    delta_b, maxvio = smebu_update(counts, bias, momentum)      # updates bias, momentum in place
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import (  # noqa: F401
    ELB_ACCUMULATE_COUNTS,
    ELB_BF16,
    ELB_F32,
    ELB_FORCE_GENERIC,
    ELB_GATES_RAW,
    ELB_MODE_LINEAR,
    ELB_MODE_SIGN,
    ELB_MODE_SMEBU,
    BalanceParams,
    ElbError,
    check,
    lib,
)

__all__ = ["router_forward", "router_dispatch", "dispatch_workspace_bytes", "smebu_update", "maxvio",
           "version", "ElbError", "MODES"]

MODES = {"smebu": ELB_MODE_SMEBU, "sign": ELB_MODE_SIGN, "linear": ELB_MODE_LINEAR}
_DTYPES = {torch.float32: ELB_F32, torch.bfloat16: ELB_BF16}


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype | None = None, device: torch.device | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def version() -> int:
    return int(lib().elb_version())


def router_forward(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor, k: int, *, gates_raw: bool = False,
                   counts: torch.Tensor | None = None, accumulate: bool = False, want_logits: bool = False,
                   want_lse: bool = False, force_generic: bool = False, out: tuple | None = None):
    """Route the tokens x [T, d] over the experts w [N_r, d] with expert bias b [N_r].

    Returns (topk_idx [T, k] int32, gates [T, k] fp32, counts [N_r] int32) and, when asked,
    logits [T, N_r] fp32 and the per-token log-sum-exp [T] fp32.  ``counts`` may be passed
    in to be overwritten (or added to, with ``accumulate=True``); ``out`` may hold
    preallocated (topk_idx, gates) tensors.
    """
    _need(x, "x")
    dev = x.device
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    _need(w, "w", x.dtype, dev)
    _need(bias, "bias", torch.float32, dev)
    if x.dim() != 2 or w.dim() != 2 or bias.dim() != 1 or w.shape[1] != x.shape[1] or bias.shape[0] != w.shape[0]:
        raise ValueError(f"shapes do not match: x {tuple(x.shape)}, w {tuple(w.shape)}, bias {tuple(bias.shape)}")
    T, d = x.shape
    n_e = w.shape[0]
    if out is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    else:
        idx, gates = out
        _need(idx, "topk_idx", torch.int32, dev)
        _need(gates, "gates", torch.float32, dev)
    if counts is None:
        if accumulate:
            raise ValueError("accumulate=True needs a counts tensor")
        counts = torch.empty(n_e, dtype=torch.int32, device=dev)
    else:
        _need(counts, "counts", torch.int32, dev)
    logits = torch.empty((T, n_e), dtype=torch.float32, device=dev) if want_logits else None
    lse = torch.empty(T, dtype=torch.float32, device=dev) if want_lse else None
    flags = (ELB_GATES_RAW if gates_raw else 0) | (ELB_ACCUMULATE_COUNTS if accumulate else 0) | (
        ELB_FORCE_GENERIC if force_generic else 0)
    st = lib().elb_router_forward(_ptr(x), _DTYPES[x.dtype], T, d, _ptr(w), _ptr(bias), n_e, k, flags, _ptr(idx),
                                  _ptr(gates), _ptr(counts), _ptr(logits), _ptr(lse), _stream(dev))
    check("elb_router_forward", st)
    res = (idx, gates, counts)
    if want_logits:
        res += (logits,)
    if want_lse:
        res += (lse,)
    return res


def dispatch_workspace_bytes(T: int, k: int, n_experts: int) -> int:
    return int(lib().elb_dispatch_workspace_bytes(T, k, n_experts))


def router_dispatch(topk_idx: torch.Tensor, n_experts: int, *, workspace: torch.Tensor | None = None,
                    want_inv: bool = True):
    """Stable counting sort of topk_idx [T, k] by expert: (offsets [N_r+1], perm [T*k], inv [T*k] or None)."""
    _need(topk_idx, "topk_idx", torch.int32)
    dev = topk_idx.device
    T, k = topk_idx.shape
    need = dispatch_workspace_bytes(T, k, n_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", device=dev)
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev) if want_inv else None
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().elb_router_dispatch(_ptr(topk_idx), T, k, n_experts, _ptr(workspace), nbytes, _ptr(offsets),
                                   _ptr(perm), _ptr(inv), _stream(dev))
    check("elb_router_dispatch", st)
    return offsets, perm, inv


def smebu_update(counts: torch.Tensor, bias: torch.Tensor, momentum: torch.Tensor | None, *, mode: str = "smebu",
                 lam: float = 5e-4, beta: float = 0.5, kappa: float = 2.0, gamma: float = 1e-3,
                 want_delta: bool = False, want_maxvio: bool = True):
    """Update bias (and momentum) in place from one step's counts.  Returns (delta_b or None, maxvio[2] or None)."""
    _need(counts, "counts", torch.int32)
    dev = counts.device
    _need(bias, "bias", torch.float32, dev)
    if momentum is not None:
        _need(momentum, "momentum", torch.float32, dev)
    n_e = counts.numel()
    if bias.numel() != n_e or (momentum is not None and momentum.numel() != n_e):
        raise ValueError("counts, bias and momentum must have the same length")
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}")
    delta = torch.empty(n_e, dtype=torch.float32, device=dev) if want_delta else None
    mv = torch.empty(2, dtype=torch.float32, device=dev) if want_maxvio else None
    params = BalanceParams(MODES[mode], lam, beta, kappa, gamma)
    st = lib().elb_smebu_update(_ptr(counts), n_e, params, _ptr(bias), _ptr(momentum), _ptr(delta), _ptr(mv),
                                _stream(dev))
    check("elb_smebu_update", st)
    return delta, mv


def maxvio(counts: torch.Tensor) -> torch.Tensor:
    """[max n / min n, (max n - nbar) / nbar] of one step's loads, as a device tensor."""
    _need(counts, "counts", torch.int32)
    out = torch.empty(2, dtype=torch.float32, device=counts.device)
    check("elb_maxvio", lib().elb_maxvio(_ptr(counts), counts.numel(), _ptr(out), _stream(counts.device)))
    return out

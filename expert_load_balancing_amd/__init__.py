"""Sigmoid Top-K MoE router with SMEBU expert-bias load balancing on AMD MI355X (gfx950).

Thin PyTorch binding over libelb.so (C ABI in include/elb.h).  These functions only check
and marshal arguments: tensors must already live on the GPU, outputs are allocated with
torch (plain device memory), and every step of the computation runs in the library's HIP
kernels on the current torch stream.  Nothing here computes the method itself.

    idx, gates, counts = router_forward(x, w, bias, k=4)
    offsets, perm, inv = router_dispatch(idx, n_experts=256)
    delta_b, maxvio = smebu_update(counts, bias, momentum)      # updates bias, momentum in place

or, for a training loop with one batch per optimizer step, all three in three kernels with
buffers allocated once:

    step = RouterStep(w, bias, momentum, k=4, max_tokens=T)
    out = step(x)            # out.topk_idx, out.gates, out.offsets, out.perm, out.maxvio, ...
"""

from __future__ import annotations

import ctypes
from typing import NamedTuple

import torch

from ._lib import (  # noqa: F401
    ELB_ACCUMULATE_COUNTS,
    ELB_BF16,
    ELB_CLEAR_COUNTS,
    ELB_DX_BF16,
    ELB_F32,
    ELB_FORCE_GENERIC,
    ELB_GATES_RAW,
    ELB_MODE_LINEAR,
    ELB_MODE_SIGN,
    ELB_MODE_SMEBU,
    BalanceParams,
    ElbError,
    StepArgs,
    check,
    lib,
)

__all__ = ["router_forward", "router_dispatch", "router_dispatch_noalloc", "dispatch_workspace_bytes", "smebu_update", "smebu_update_layers",
           "maxvio", "zloss", "permute_rows", "unpermute_combine", "router_backward", "backward_workspace_bytes", "RouterStep", "StepOutputs", "version", "ElbError",
           "MODES"]

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
    # Sizes first (a buffer too small would be written past its end on the device), then
    # dtype, device and layout.
    for t, name in ((x, "x"), (w, "w"), (bias, "bias")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
    if x.dim() != 2 or w.dim() != 2 or bias.dim() != 1 or w.shape[1] != x.shape[1] or bias.shape[0] != w.shape[0]:
        raise ValueError(f"shapes do not match: x {tuple(x.shape)}, w {tuple(w.shape)}, bias {tuple(bias.shape)}")
    T, d = x.shape
    n_e = w.shape[0]
    if out is not None:
        if len(out) != 2 or any(not isinstance(t, torch.Tensor) for t in out):
            raise TypeError("out must be a (topk_idx, gates) pair of tensors")
        if out[0].numel() != T * k or out[1].numel() != T * k:
            raise ValueError(f"out: topk_idx and gates must hold T*k = {T * k} entries, got "
                             f"{out[0].numel()} and {out[1].numel()}")
    if counts is not None and (not isinstance(counts, torch.Tensor) or counts.numel() != n_e):
        raise ValueError(f"counts must be a tensor of N_r = {n_e} entries")
    _need(x, "x")
    dev = x.device
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    _need(w, "w", x.dtype, dev)
    _need(bias, "bias", torch.float32, dev)
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
                    want_inv: bool = True, out: tuple | None = None):
    """Stable counting sort of topk_idx [T, k] by expert: (offsets [N_r+1], perm [T*k], inv [T*k] or None).

    ``out``: (offsets, perm, inv or None) int32 tensors to write instead of new ones.
    """
    if not isinstance(topk_idx, torch.Tensor) or topk_idx.dim() != 2:
        raise ValueError("topk_idx must be a [T, k] tensor")
    _need(topk_idx, "topk_idx", torch.int32)
    dev = topk_idx.device
    T, k = topk_idx.shape
    need = dispatch_workspace_bytes(T, k, n_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", device=dev)
    if out is not None:
        offsets, perm, inv = out
        _need(offsets, "offsets", torch.int32, dev)
        _need(perm, "perm", torch.int32, dev)
        if inv is not None:
            _need(inv, "inv", torch.int32, dev)
        if offsets.numel() != n_experts + 1 or perm.numel() != T * k or (inv is not None and inv.numel() != T * k):
            raise ValueError("router_dispatch: out tensors have the wrong sizes")
    else:
        offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(T * k, dtype=torch.int32, device=dev)
        inv = torch.empty(T * k, dtype=torch.int32, device=dev) if want_inv else None
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().elb_router_dispatch(_ptr(topk_idx), T, k, n_experts, _ptr(workspace), nbytes, _ptr(offsets),
                                   _ptr(perm), _ptr(inv), _stream(dev))
    check("elb_router_dispatch", st)
    return offsets, perm, inv


def router_dispatch_noalloc(topk_idx: torch.Tensor, n_experts: int, out: tuple):
    """router_dispatch through the library's allocation-free entry point, into caller buffers
    ``out`` = (offsets [N_r+1], perm [T*k], inv [T*k] or None), int32 on topk_idx's device.  The
    library uses a static per-GPU workspace (8 MiB); calls overlapping on one GPU race."""
    if not isinstance(topk_idx, torch.Tensor) or topk_idx.dim() != 2:
        raise ValueError("topk_idx must be a [T, k] tensor")
    T, k = topk_idx.shape
    offsets, perm, inv = out
    if offsets.numel() != n_experts + 1 or perm.numel() != T * k or (inv is not None and inv.numel() != T * k):
        raise ValueError("router_dispatch_noalloc: out tensors have the wrong sizes")
    _need(topk_idx, "topk_idx", torch.int32)
    dev = topk_idx.device
    _need(offsets, "offsets", torch.int32, dev)
    _need(perm, "perm", torch.int32, dev)
    if inv is not None:
        _need(inv, "inv", torch.int32, dev)
    st = lib().elb_router_dispatch_noalloc(_ptr(topk_idx), T, k, n_experts, _ptr(offsets), _ptr(perm), _ptr(inv),
                                           _stream(dev))
    check("elb_router_dispatch_noalloc", st)
    return offsets, perm, inv


def smebu_update(counts: torch.Tensor, bias: torch.Tensor, momentum: torch.Tensor | None, *, mode: str = "smebu",
                 lam: float = 5e-4, beta: float = 0.5, kappa: float = 2.0, gamma: float = 1e-3,
                 want_delta: bool = False, want_maxvio: bool = True, clear_counts: bool = False):
    """Update bias (and momentum) in place from one step's counts.  Returns (delta_b or None, maxvio[2] or None).

    With ``clear_counts`` the counts are zeroed once read, ready for the next step's accumulation.
    """
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
    params = BalanceParams(MODES[mode], lam, beta, kappa, gamma, ELB_CLEAR_COUNTS if clear_counts else 0)
    st = lib().elb_smebu_update(_ptr(counts), n_e, params, _ptr(bias), _ptr(momentum), _ptr(delta), _ptr(mv),
                                _stream(dev))
    check("elb_smebu_update", st)
    return delta, mv


def smebu_update_layers(counts: torch.Tensor, bias: torch.Tensor, momentum: torch.Tensor | None, *,
                        mode: str = "smebu", lam: float = 5e-4, beta: float = 0.5, kappa: float = 2.0,
                        gamma: float = 1e-3, want_delta: bool = False, want_maxvio: bool = True,
                        clear_counts: bool = False):
    """One update per MoE layer in one launch: counts, bias, momentum are [L, N_r] (each layer's
    own loads, b and m).  Returns (delta_b [L, N_r] or None, maxvio [L, 2] or None)."""
    _need(counts, "counts", torch.int32)
    dev = counts.device
    _need(bias, "bias", torch.float32, dev)
    if momentum is not None:
        _need(momentum, "momentum", torch.float32, dev)
    if counts.dim() != 2 or bias.shape != counts.shape or (momentum is not None and momentum.shape != counts.shape):
        raise ValueError("counts, bias and momentum must all be [L, N_r]")
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}")
    L, n_e = counts.shape
    delta = torch.empty((L, n_e), dtype=torch.float32, device=dev) if want_delta else None
    mv = torch.empty((L, 2), dtype=torch.float32, device=dev) if want_maxvio else None
    params = BalanceParams(MODES[mode], lam, beta, kappa, gamma, ELB_CLEAR_COUNTS if clear_counts else 0)
    st = lib().elb_smebu_update_layers(_ptr(counts), L, n_e, params, _ptr(bias), _ptr(momentum), _ptr(delta),
                                       _ptr(mv), _stream(dev))
    check("elb_smebu_update_layers", st)
    return delta, mv


def zloss(lse: torch.Tensor) -> torch.Tensor:
    """mean_t lse_t^2 of per-token log-sum-exps [T], as a device scalar tensor [1]."""
    _need(lse, "lse", torch.float32)
    out = torch.empty(1, dtype=torch.float32, device=lse.device)
    check("elb_zloss", lib().elb_zloss(_ptr(lse), lse.numel(), _ptr(out), _stream(lse.device)))
    return out


def permute_rows(x: torch.Tensor, inv_perm: torch.Tensor, k: int, *, out: torch.Tensor | None = None) -> torch.Tensor:
    """Expert-contiguous copy of the token rows: out[inv_perm[t*k + j]] = x[t]; out is [T*k, d]."""
    _need(x, "x")
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    dev = x.device
    _need(inv_perm, "inv_perm", torch.int32, dev)
    T, d = x.shape
    if inv_perm.numel() != T * k:
        raise ValueError(f"inv_perm must hold T*k = {T * k} entries")
    if out is None:
        out = torch.empty((T * k, d), dtype=x.dtype, device=dev)
    else:
        _need(out, "out", x.dtype, dev)
    st = lib().elb_permute_rows(_ptr(x), _DTYPES[x.dtype], T, d, k, _ptr(inv_perm), _ptr(out), _stream(dev))
    check("elb_permute_rows", st)
    return out


def unpermute_combine(expert_out: torch.Tensor, gates: torch.Tensor, inv_perm: torch.Tensor, *,
                      out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """y[t] = sum_j gates[t, j] * expert_out[inv_perm[t*k + j]] (fp32 accumulation); y is [T, d]."""
    _need(expert_out, "expert_out")
    if expert_out.dtype not in _DTYPES or out_dtype not in _DTYPES:
        raise TypeError("expert_out and the output must be float32 or bfloat16")
    dev = expert_out.device
    _need(gates, "gates", torch.float32, dev)
    _need(inv_perm, "inv_perm", torch.int32, dev)
    T, k = gates.shape
    d = expert_out.shape[1]
    if expert_out.shape[0] != T * k or inv_perm.numel() != T * k:
        raise ValueError("expert_out and inv_perm must hold T*k rows")
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", out_dtype, dev)
    st = lib().elb_unpermute_combine(_ptr(expert_out), _DTYPES[expert_out.dtype], T, d, k, _ptr(inv_perm),
                                     _ptr(gates), _ptr(out), _DTYPES[out_dtype], _stream(dev))
    check("elb_unpermute_combine", st)
    return out


def backward_workspace_bytes(T: int, d: int, n_experts: int) -> int:
    return int(lib().elb_backward_workspace_bytes(T, d, n_experts))


def router_backward(x: torch.Tensor, w: torch.Tensor, topk_idx: torch.Tensor, dgates: torch.Tensor, *,
                    gates_raw: bool = False, zloss_coef: float = 0.0, want_dx: bool = True, want_dw: bool = True,
                    dx_dtype: torch.dtype = torch.float32, workspace: torch.Tensor | None = None):
    """Gradients of sum(dgates * gates) + zloss_coef * mean(lse^2) at the selection topk_idx:
    returns (dx [T, d] of dx_dtype (float32, or bfloat16 rounded to nearest even) or None,
    dw [N_r, d] fp32 or None).  bf16 x and w, d % 64 == 0."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(w, "w", torch.bfloat16, dev)
    _need(topk_idx, "topk_idx", torch.int32, dev)
    _need(dgates, "dgates", torch.float32, dev)
    T, d = x.shape
    n_e = w.shape[0]
    k = topk_idx.shape[1]
    if w.shape[1] != d or topk_idx.shape[0] != T or dgates.shape != topk_idx.shape:
        raise ValueError("shapes do not match")
    need = backward_workspace_bytes(T, d, n_e)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", device=dev)
    if dx_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"dx_dtype must be float32 or bfloat16, got {dx_dtype}")
    dx = torch.empty((T, d), dtype=dx_dtype, device=dev) if want_dx else None
    dw = torch.empty((n_e, d), dtype=torch.float32, device=dev) if want_dw else None
    flags = (ELB_GATES_RAW if gates_raw else 0) | (ELB_DX_BF16 if dx_dtype == torch.bfloat16 else 0)
    st = lib().elb_router_backward(_ptr(x), ELB_BF16, T, d, _ptr(w), n_e, k, flags,
                                   _ptr(topk_idx), _ptr(dgates), float(zloss_coef), _ptr(dx), _ptr(dw),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    check("elb_router_backward", st)
    return dx, dw


def maxvio(counts: torch.Tensor) -> torch.Tensor:
    """[max n / min n, (max n - nbar) / nbar] of one step's loads, as a device tensor."""
    _need(counts, "counts", torch.int32)
    out = torch.empty(2, dtype=torch.float32, device=counts.device)
    check("elb_maxvio", lib().elb_maxvio(_ptr(counts), counts.numel(), _ptr(out), _stream(counts.device)))
    return out


def stream_xor(t: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """One streaming read of t's bytes (16-byte multiple): out[0] ^= the XOR of its 32-bit words
    (out: one int32 on t's device, zeroed here when not given).  The bench's measured HBM read
    reference."""
    _need(t, "t")
    if out is None:
        out = torch.zeros(1, dtype=torch.int32, device=t.device)
    else:
        _need(out, "out", torch.int32, t.device)
    check("elb_stream_xor", lib().elb_stream_xor(_ptr(t), t.numel() * t.element_size(), _ptr(out), _stream(t.device)))
    return out


class StepOutputs(NamedTuple):
    """Views of one RouterStep call's outputs (valid until the next call)."""

    topk_idx: torch.Tensor   # [T, k] int32
    gates: torch.Tensor      # [T, k] fp32
    counts: torch.Tensor     # [N_r] int32 (zero after a step that cleared them)
    offsets: torch.Tensor | None  # [N_r + 1] int32 (None without dispatch)
    perm: torch.Tensor | None     # [T * k] int32 (None without dispatch)
    inv_perm: torch.Tensor | None
    lse: torch.Tensor | None
    zloss: torch.Tensor | None
    delta_b: torch.Tensor | None
    maxvio: torch.Tensor | None


class RouterStep:
    """Route, dispatch (optional) and update (optional) the expert bias in one library call
    (elb_route_step).

    Holds the router weight w [N_r, d], the bias b [N_r] and momentum m [N_r] (updated in place
    when ``update``), and output buffers sized for up to ``max_tokens`` tokens, allocated once.
    ``counts`` start at zero; with ``update`` and ``clear_counts`` each call routes with the
    current bias, then applies one bias update from this batch's loads and leaves the counts
    zeroed for the next call.  Without ``update`` the loads accumulate across calls (several
    micro-batches per optimizer step) until an update with ``clear_counts`` consumes them.
    ``dispatch=False`` skips the counting-sort dispatch (offsets, perm, inv_perm are then None).
    """

    def __init__(self, w: torch.Tensor, bias: torch.Tensor, momentum: torch.Tensor | None, k: int, max_tokens: int,
                 *, update: bool = True, mode: str = "smebu", lam: float = 5e-4, beta: float = 0.5,
                 kappa: float = 2.0, gamma: float = 1e-3, clear_counts: bool = True, gates_raw: bool = False,
                 want_inv: bool = True, want_lse: bool = False, want_zloss: bool = False, want_delta: bool = False,
                 want_maxvio: bool = True, force_generic: bool = False, dispatch: bool = True):
        _need(w, "w")
        dev = w.device
        if w.dtype not in _DTYPES:
            raise TypeError(f"w must be float32 or bfloat16, got {w.dtype}")
        _need(bias, "bias", torch.float32, dev)
        if momentum is not None:
            _need(momentum, "momentum", torch.float32, dev)
        n_e, d = w.shape
        if bias.shape != (n_e,) or (momentum is not None and momentum.shape != (n_e,)):
            raise ValueError("bias and momentum must have one entry per row of w")
        if mode not in MODES:
            raise ValueError(f"mode must be one of {sorted(MODES)}")
        self.w, self.bias, self.momentum, self.k, self.max_tokens = w, bias, momentum, k, max_tokens
        self.device = dev
        T, i32, f32 = max_tokens, torch.int32, torch.float32
        self.topk_idx = torch.empty((T, k), dtype=i32, device=dev)
        self.gates = torch.empty((T, k), dtype=f32, device=dev)
        self.counts = torch.zeros(n_e, dtype=i32, device=dev)
        self.offsets = torch.empty(n_e + 1, dtype=i32, device=dev) if dispatch else None
        self.perm = torch.empty(T * k, dtype=i32, device=dev) if dispatch else None
        self.inv_perm = torch.empty(T * k, dtype=i32, device=dev) if (dispatch and want_inv) else None
        self.lse = torch.empty(T, dtype=f32, device=dev) if (want_lse or want_zloss) else None
        self.zloss = torch.empty(1, dtype=f32, device=dev) if want_zloss else None
        self.delta_b = torch.empty(n_e, dtype=f32, device=dev) if (update and want_delta) else None
        self.maxvio = torch.empty(2, dtype=f32, device=dev) if (update and want_maxvio) else None
        ws_bytes = dispatch_workspace_bytes(T, k, n_e) if dispatch else 0
        self.workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if dispatch else None
        flags = ELB_ACCUMULATE_COUNTS | (ELB_GATES_RAW if gates_raw else 0) | (ELB_FORCE_GENERIC if force_generic else 0)
        a = StepArgs()
        a.dtype, a.d, a.w, a.bias = _DTYPES[w.dtype], d, w.data_ptr(), bias.data_ptr()
        a.n_experts, a.k, a.flags = n_e, k, flags
        a.topk_idx, a.gates, a.counts = self.topk_idx.data_ptr(), self.gates.data_ptr(), self.counts.data_ptr()
        a.logits, a.lse, a.zloss = None, _ptr(self.lse).value, _ptr(self.zloss).value
        a.workspace, a.workspace_bytes = _ptr(self.workspace).value, 0 if self.workspace is None else self.workspace.numel()
        a.offsets, a.perm, a.inv_perm = _ptr(self.offsets).value, _ptr(self.perm).value, _ptr(self.inv_perm).value
        a.update = 1 if update else 0
        a.params = BalanceParams(MODES[mode], lam, beta, kappa, gamma, ELB_CLEAR_COUNTS if clear_counts else 0)
        a.momentum, a.delta_b, a.maxvio = _ptr(momentum).value, _ptr(self.delta_b).value, _ptr(self.maxvio).value
        a.timing = None
        self._args = a
        self._timing = None

    def set_timing(self, start=None, stop=None, end=None) -> None:
        """Bracket the kernels of later calls with timing events (torch.cuda.Event or any object
        with a ``cuda_event`` handle): ``start`` takes the end of an empty kernel launched just
        before the router kernel, ``stop`` the router kernel's own end, ``end`` the end of the
        step's last kernel; any may be None, and ``set_timing()`` stops it."""
        if start is None and stop is None and end is None:
            self._timing, self._args.timing = None, None
            return
        handles = []
        for ev in (start, stop, end):
            if ev is not None and ev.cuda_event == 0:  # torch creates the HIP event on first record
                ev.record(torch.cuda.current_stream(self.device))
            handles.append(None if ev is None else ev.cuda_event)
        self._timing = (ctypes.c_void_p * 3)(*handles)
        self._args.timing = ctypes.cast(self._timing, ctypes.c_void_p).value

    def __call__(self, x: torch.Tensor) -> StepOutputs:
        _need(x, "x", self.w.dtype, self.device)
        T = x.shape[0]
        if x.dim() != 2 or x.shape[1] != self.w.shape[1] or T > self.max_tokens:
            raise ValueError(f"x must be [T <= {self.max_tokens}, {self.w.shape[1]}], got {tuple(x.shape)}")
        a = self._args
        a.x, a.T = x.data_ptr(), T
        check("elb_route_step", lib().elb_route_step(ctypes.byref(a), _stream(self.device)))
        k = self.k
        return StepOutputs(self.topk_idx[:T], self.gates[:T], self.counts, self.offsets,
                           None if self.perm is None else self.perm[:T * k],
                           None if self.inv_perm is None else self.inv_perm[:T * k],
                           None if self.lse is None else self.lse[:T], self.zloss, self.delta_b, self.maxvio)

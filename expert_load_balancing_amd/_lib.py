"""ctypes view of libelb.so: the C ABI declared in include/elb.h, nothing more.

The library is loaded from this package directory only.  If it is missing or cannot be
loaded, every entry point raises: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libelb.so")

ELB_F32, ELB_BF16 = 0, 1
ELB_MODE_SMEBU, ELB_MODE_SIGN, ELB_MODE_LINEAR = 0, 1, 2
ELB_GATES_RAW, ELB_ACCUMULATE_COUNTS, ELB_FORCE_GENERIC = 1, 2, 4
ELB_CLEAR_COUNTS = 1
ELB_DX_BF16 = 8

STATUS_NAMES = {0: "ELB_OK", 1: "ELB_ERR_NULL", 2: "ELB_ERR_SHAPE", 3: "ELB_ERR_UNSUPPORTED",
                4: "ELB_ERR_ALIGN", 5: "ELB_ERR_WORKSPACE", 6: "ELB_ERR_LAUNCH"}

# Every function the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I32, _I64, _U32, _SZ, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_float


class BalanceParams(ctypes.Structure):
    _fields_ = [("mode", _I32), ("lambda_", _F), ("beta", _F), ("kappa", _F), ("gamma", _F), ("flags", _U32)]


class StepArgs(ctypes.Structure):
    """elb_step_args, field for field."""

    _fields_ = [
        ("x", _P), ("dtype", _I32), ("T", _I64), ("d", _I32), ("w", _P), ("bias", _P), ("n_experts", _I32),
        ("k", _I32), ("flags", _U32), ("topk_idx", _P), ("gates", _P), ("counts", _P), ("logits", _P), ("lse", _P),
        ("zloss", _P), ("workspace", _P), ("workspace_bytes", _SZ), ("offsets", _P), ("perm", _P), ("inv_perm", _P),
        ("update", _I32), ("params", BalanceParams), ("momentum", _P), ("delta_b", _P), ("maxvio", _P),
        ("timing", _P),
    ]


SIGNATURES = {
    "elb_router_forward": (_I32, [_P, _I32, _I64, _I32, _P, _P, _I32, _I32, _U32, _P, _P, _P, _P, _P, _P]),
    "elb_dispatch_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "elb_router_dispatch": (_I32, [_P, _I64, _I32, _I32, _P, _SZ, _P, _P, _P, _P]),
    "elb_router_dispatch_noalloc": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _P]),
    "elb_smebu_update": (_I32, [_P, _I32, BalanceParams, _P, _P, _P, _P, _P]),
    "elb_route_step": (_I32, [ctypes.POINTER(StepArgs), _P]),
    "elb_smebu_update_layers": (_I32, [_P, _I32, _I32, BalanceParams, _P, _P, _P, _P, _P]),
    "elb_zloss": (_I32, [_P, _I64, _P, _P]),
    "elb_permute_rows": (_I32, [_P, _I32, _I64, _I32, _I32, _P, _P, _P]),
    "elb_unpermute_combine": (_I32, [_P, _I32, _I64, _I32, _I32, _P, _P, _P, _I32, _P]),
    "elb_backward_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "elb_router_backward": (_I32, [_P, _I32, _I64, _I32, _P, _I32, _I32, _U32, _P, _P, _F, _P, _P, _P, _SZ, _P]),
    "elb_maxvio": (_I32, [_P, _I32, _P, _P]),
    "elb_stream_xor": (_I32, [_P, _SZ, _P, _P]),
    "elb_status_str": (ctypes.c_char_p, [_I32]),
    "elb_version": (ctypes.c_int, []),
}

_lib = None


class ElbError(RuntimeError):
    """A libelb entry point returned a non-zero elb_status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libelb.so was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m expert_load_balancing_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise ElbError(fn, status, lib().elb_status_str(status).decode())

"""The allocation-free dispatch entry point (elb_router_dispatch_noalloc) against
elb_router_dispatch, through the C ABI: bit-identical offsets, perm and inv on two calls in a
row, the second with a smaller batch (the static workspace keeps the first call's contents,
which must not matter), then without inv, with an empty batch, and on the stress workload's
whole batch of routed indices (262,144 tokens)."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import check_dispatch, log

pytestmark = pytest.mark.gpu


def buffers(T, k, n_e, inv=True):
    i32 = torch.int32
    return (torch.full((n_e + 1,), -7, dtype=i32, device="cuda"), torch.full((T * k,), -7, dtype=i32, device="cuda"),
            torch.full((T * k,), -7, dtype=i32, device="cuda") if inv else None)


def both(idx, n_e, inv=True):
    T, k = idx.shape
    want = elb.router_dispatch(idx, n_e, want_inv=inv)
    got = elb.router_dispatch_noalloc(idx, n_e, buffers(T, k, n_e, inv))
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        if w is None:
            assert g is None
        else:
            assert torch.equal(g, w)
    return [None if t is None else t.cpu().numpy() for t in got]


def test_noalloc_dispatch_matches_the_workspace_entry_point():
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for T, k, n_e in ((300_000, 4, 256), (1000, 4, 256), (777, 8, 64), (5, 1, 3)):
        log(f"noalloc dispatch T={T} k={k} N_r={n_e}")
        idx = torch.randint(0, n_e, (T, k), generator=gen, device="cuda", dtype=torch.int32)
        offs, perm, inv = both(idx, n_e)
        check_dispatch(offs, perm, inv, idx.cpu().numpy(), n_e)
    both(idx, n_e, inv=False)
    empty = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    offs, perm, _ = elb.router_dispatch_noalloc(empty, 256, buffers(0, 4, 256))
    torch.cuda.synchronize()
    assert (offs.cpu().numpy() == 0).all()


def test_noalloc_dispatch_on_the_stress_batch():
    """The stress workload's own routing (skewed loads, duplicate rows), then a smaller batch."""
    wl = datagen.WORKLOADS["stress"]
    x = torch.from_numpy(datagen.tokens(wl).view(np.int16)).cuda().view(torch.bfloat16)
    w = torch.from_numpy(datagen.router_weight(wl).view(np.int16)).cuda().view(torch.bfloat16)
    b = torch.from_numpy(datagen.initial_bias(wl)).cuda()
    idx, _, _ = elb.router_forward(x, w, b, wl.k)
    offs, perm, inv = both(idx, wl.n_experts)
    check_dispatch(offs, perm, inv, idx.cpu().numpy(), wl.n_experts)
    both(idx[:4099].contiguous(), wl.n_experts)

"""A seeded random sweep of router and step shapes against the oracle: combinations the listed
cases leave out (odd expert counts, every K, d from one to many 64-element stages, ragged T on
every tile size, both input dtypes and both kernels, raw and normalised gates), 48 draws, each
small enough for the oracle.  The draws come from a fixed seed, so a failure names a case that
reruns the same way."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import check_counts, check_dispatch, compare_logits, compare_route, log, to_dev

pytestmark = pytest.mark.gpu


def draws(n=48, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        n_e = int(rng.choice([3, 16, 37, 64, 100, 129, 200, 255, 256]))
        k = int(rng.integers(1, min(8, n_e) + 1))
        d = 64 * int(rng.integers(1, 25))
        T = int(rng.integers(1, 3000))
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        kind = "clusters" if rng.random() < 0.5 else "iid"
        raw = bool(rng.random() < 0.25)
        out.append((i, T, d, n_e, k, dtype, kind, raw))
    return out


@pytest.mark.parametrize("i,T,d,n_e,k,dtype,kind,raw", draws())
def test_router_and_step_sweep(i, T, d, n_e, k, dtype, kind, raw):
    log(f"sweep {i}: T={T} d={d} N_r={n_e} K={k} {dtype} {kind} raw_gates={raw}")
    wl = datagen.WORKLOADS["large"].replace(T=T, d=d, n_experts=n_e, k=k, dtype=dtype, seed=1000 + i,
                                            token_kind=kind, n_clusters=8 if kind == "clusters" else 0)
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    for generic in (False, True):
        idx, gates, counts, logits = elb.router_forward(xd, wd, bd, k, want_logits=True, gates_raw=raw,
                                                        force_generic=generic)
        torch.cuda.synchronize()
        idx_h, gates_h = idx.cpu().numpy(), gates.cpu().numpy()
        compare_route(idx_h, gates_h, x, w, b, k, normalize=not raw)
        check_counts(counts.cpu().numpy(), idx_h, n_e)
        compare_logits(logits.cpu().numpy(), x, w)
    # The fused step (default kernel choice) routes and dispatches the same batch identically.
    step = elb.RouterStep(wd, to_dev(b), None, k, T, update=False, gates_raw=raw)
    out = step(xd)
    torch.cuda.synchronize()
    assert np.array_equal(out.topk_idx.cpu().numpy(), elb.router_forward(xd, wd, bd, k, gates_raw=raw)[0].cpu().numpy())
    check_dispatch(out.offsets.cpu().numpy(), out.perm.cpu().numpy(), out.inv_perm.cpu().numpy(),
                   out.topk_idx.cpu().numpy(), n_e)

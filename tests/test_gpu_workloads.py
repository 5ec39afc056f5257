"""The full-size workloads, in the launch configuration the benchmark times: routing checked
against the oracle on a seeded sample of tokens (plus first, last, ragged-tail and duplicate
rows), and everything that holds at any size checked on the whole batch: K distinct experts
per token, normalised gates summing to one, counts from the GPU's own indices, dispatch
bit-exact, and the bias update against the oracle fed the GPU's counts."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import (check_balance, check_counts, check_dispatch, check_maxvio, compare_route, log, sample_rows,
                      to_dev)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key", ["tiny", "sign", "large", "stress"])
def test_full_size_workload(key):
    wl = datagen.WORKLOADS[key]
    log(f"workload {wl.label}: generating inputs")
    x, w = datagen.tokens(wl), datagen.router_weight(wl)
    b0, m0 = datagen.initial_bias(wl), datagen.initial_momentum(wl)
    xd, wd, bd, md = to_dev(x), to_dev(w), to_dev(b0), to_dev(m0)
    log(f"workload {wl.label}: running on the GPU")
    idx, gates, counts = elb.router_forward(xd, wd, bd, wl.k)
    offs = perm = inv = None
    if wl.dispatch:
        offs, perm, inv = elb.router_dispatch(idx, wl.n_experts)
    delta, mv = elb.smebu_update(counts, bd, md, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa,
                                 gamma=wl.gamma, want_delta=True)
    torch.cuda.synchronize()
    idx_h, gates_h, counts_h = idx.cpu().numpy(), gates.cpu().numpy(), counts.cpu().numpy()

    # Whole batch: K distinct experts in range, gates sum to one, counts exact.
    assert idx_h.min() >= 0 and idx_h.max() < wl.n_experts
    assert (np.diff(np.sort(idx_h, axis=1), axis=1) > 0).all(), "a token chose an expert twice"
    assert np.allclose(gates_h.sum(1), 1.0, atol=2e-6) and (gates_h > 0).all()
    counts64 = check_counts(counts_h, idx_h, wl.n_experts)
    assert counts64.sum() == wl.T * wl.k

    # Oracle on a sample (all of it for the tiny workload).
    dst, src = datagen.duplicate_rows(wl)
    rows = np.arange(wl.T) if wl.T <= 4096 else sample_rows(wl.T, 3000, wl.seed, extra=np.r_[dst[:200], src[:200]])
    rep = compare_route(idx_h, gates_h, x, w, b0, wl.k, rows)
    log(f"  sampled {rep.n_tokens} tokens: ties={rep.ties} (mismatched {rep.tie_mismatch}), "
        f"order-ties={rep.order_ties}, gate rel err {rep.max_gate_rel:.2e}")
    if len(dst):
        assert (idx_h[dst] == idx_h[src]).all()
        assert (gates_h[dst].view(np.uint32) == gates_h[src].view(np.uint32)).all()

    if wl.dispatch:
        check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx_h, wl.n_experts)
    err = check_balance(wl.mode, counts64, b0, m0, bd.cpu().numpy(), md.cpu().numpy(), wl, delta.cpu().numpy())
    check_maxvio(mv.cpu().numpy(), counts64)
    log(f"  MaxVio {mv.cpu().numpy()[0]:.3f}, b/m error {err:.2e}")


@pytest.mark.parametrize("key", ["tiny", "sign", "large", "stress"])
def test_full_size_workload_fused_step(key):
    """The same workloads through elb_route_step (one call, three or four kernels): outputs equal
    the separate calls' bit for bit -- the generic kernel plus a counting pass for the fp32
    workload, the dispatch scan over 1024 tiles for the stress workload."""
    wl = datagen.WORKLOADS[key]
    log(f"fused step on {wl.label}")
    x, w = datagen.tokens(wl), datagen.router_weight(wl)
    b0, m0 = datagen.initial_bias(wl), datagen.initial_momentum(wl)
    xd, wd = to_dev(x), to_dev(w)
    kw = dict(mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa, gamma=wl.gamma)
    bs, ms = to_dev(b0), to_dev(m0)
    cs = torch.zeros(wl.n_experts, dtype=torch.int32, device="cuda")
    idx, gates, _ = elb.router_forward(xd, wd, bs, wl.k, counts=cs, accumulate=True)
    offs, perm, inv = elb.router_dispatch(idx, wl.n_experts)
    counts_sep = cs.clone()
    delta, mv = elb.smebu_update(cs, bs, ms, want_delta=True, clear_counts=True, **kw)
    bf, mf = to_dev(b0), to_dev(m0)
    out = elb.RouterStep(wd, bf, mf, wl.k, wl.T, want_delta=True, **kw)(xd)
    torch.cuda.synchronize()
    pairs = [(out.topk_idx, idx), (out.gates, gates), (out.offsets, offs), (out.perm, perm), (out.inv_perm, inv),
             (bf, bs), (mf, ms), (out.delta_b, delta), (out.maxvio, mv)]
    for got, want in pairs:
        assert np.array_equal(got.cpu().numpy(), want.cpu().numpy(), equal_nan=True)
    assert (out.counts.cpu().numpy() == 0).all()
    check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx.cpu().numpy(), wl.n_experts)
    check_balance(wl.mode, counts_sep.cpu().numpy().astype(np.int64), b0, m0, bf.cpu().numpy(), mf.cpu().numpy(), wl,
                  out.delta_b.cpu().numpy())

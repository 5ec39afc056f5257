"""The full-size workloads, in the launch configuration the benchmark times: routing of every
token checked against the oracle (in row chunks), with near-ties counted and reported, and
everything else on the whole batch: K distinct experts per token, normalised gates summing to
one, counts from the GPU's own indices, dispatch bit-exact, duplicate rows bit-identical, and
the bias update against the oracle fed the GPU's counts."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
import oracle
from gpu_util import check_balance, check_counts, check_dispatch, check_maxvio, compare_route, log, order_tol, to_dev

pytestmark = pytest.mark.gpu


def k_rotation(rows: np.ndarray, T: int, d: int) -> np.ndarray:
    """The stage at which the MFMA router starts the k loop for these token rows: its workgroup's
    tile index modulo the number of 64-element stages when rows are a multiple of 4 KiB apart,
    else 0 (tiles of 256 tokens above 128 x 256 tokens, 128 above 64 x 256, else 64)."""
    if (2 * d) % 4096:
        return np.zeros(len(rows), dtype=np.int64)
    tile = 256 if T > 128 * 256 else 128 if T > 64 * 256 else 64
    return (rows // tile) % (d // 64)


def check_duplicates(idx_h, gates_h, x, w, b0, wl, dst, src):
    """Exact copies of rows.  Copies whose workgroups run the k loop from the same stage take the
    same fp32 accumulation order and must match bit for bit.  Copies that start at different
    stages sum the same products in another order: they must choose the same experts in the same
    order wherever the oracle separates the candidates by more than the comparison's resolution,
    and carry gates within a few fp32 ulps."""
    same = k_rotation(dst, wl.T, wl.d) == k_rotation(src, wl.T, wl.d)
    assert (idx_h[dst[same]] == idx_h[src[same]]).all()
    assert (gates_h[dst[same]].view(np.uint32) == gates_h[src[same]].view(np.uint32)).all()
    other_d, other_s = dst[~same], src[~same]
    if len(other_d):
        r = oracle.route(x[other_d], w, b0, wl.k, keep=True)
        tol = order_tol(b0)
        q = np.sort(r.scores + np.asarray(b0, np.float64)[None, :], axis=1)[:, ::-1][:, :wl.k + 1]
        separated = (np.diff(-q, axis=1) >= tol).all(axis=1)  # every adjacent gap among the top K+1
        assert (idx_h[other_d[separated]] == idx_h[other_s[separated]]).all()
        same_sel = (idx_h[other_d] == idx_h[other_s]).all(axis=1)
        gd, gs = gates_h[other_d[same_sel]].astype(np.float64), gates_h[other_s[same_sel]].astype(np.float64)
        assert np.allclose(gd, gs, rtol=1e-5, atol=1e-9), np.abs(gd - gs).max()
        log(f"  duplicates: {int(same.sum())} bit-identical (same k start), {len(other_d)} from another k start: "
            f"{int(separated.sum())} separated and identical, {int((~same_sel).sum())} reordered within resolution")
    else:
        log(f"  duplicates: {int(same.sum())} bit-identical")


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

    # Every token against the oracle.
    dst, src = datagen.duplicate_rows(wl)
    rep = compare_route(idx_h, gates_h, x, w, b0, wl.k)
    assert rep.n_tokens == wl.T
    log(f"  {wl.label}: {rep}")
    if len(dst):
        check_duplicates(idx_h, gates_h, x, w, b0, wl, dst, src)

    if wl.dispatch:
        check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx_h, wl.n_experts)
    err = check_balance(wl.mode, counts64, b0, m0, bd.cpu().numpy(), md.cpu().numpy(), wl, delta.cpu().numpy())
    check_maxvio(mv.cpu().numpy(), counts64)
    log(f"  MaxVio {mv.cpu().numpy()[0]:.3f}, b/m error {err:.2e}")


@pytest.mark.parametrize("key", ["tiny", "sign", "large", "stress"])
def test_full_size_workload_fused_step(key):
    """The same workloads through elb_route_step (one call: the router kernel, then the dispatch
    launch, with a counting pass between them where the router's tiles are not the dispatch's):
    outputs equal the separate calls' bit for bit -- the generic kernel plus a counting pass for
    the fp32 workload, the dispatch's scan blocks over 1024 tiles for the stress workload."""
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

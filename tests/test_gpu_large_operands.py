"""Operands past 4 GiB: a 720,901 x 3072 bf16 token batch (4.43 GB), so that byte offsets into
the tokens, the permuted rows (17.7 GB), the combined output and dX (8.9 GB each) overflow 32
bits.  Routing is checked against the oracle on sampled rows, including the rows around the
4 GiB mark and the ragged tail; everything that holds at any size is checked on the whole
batch.  dW, a sum over every token, is checked against two half batches (the per-token chain
rule does not depend on the batch without the z-loss)."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
import oracle
from gpu_util import check_balance, check_counts, check_dispatch, check_maxvio, compare_route, log, sample_rows, to_dev

pytestmark = pytest.mark.gpu

T, D, N_E, K = 720_901, 3072, 256, 4


def host_rows(xd: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of the given token rows."""
    sel = xd[torch.from_numpy(rows).to(xd.device)]
    return sel.view(torch.int16).cpu().numpy().view(np.uint16)


def test_router_dispatch_moe_ops_and_backward_past_4gib():
    wl = datagen.WORKLOADS["large"].replace(T=T, seed=41)
    assert T * D * 2 > 2 ** 32
    log(f"large operands: T={T} d={D} ({T * D * 2 / 1e9:.2f} GB of tokens)")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    xd = torch.randn((T, D), generator=gen, device="cuda").to(torch.bfloat16)
    w, b0, m0 = datagen.router_weight(wl), datagen.initial_bias(wl), datagen.initial_momentum(wl)
    wd, bd, md = to_dev(w), to_dev(b0), to_dev(m0)

    # ---- router, dispatch, update (separate calls), then the fused step on the same inputs ----
    idx, gates, counts = elb.router_forward(xd, wd, bd, K)
    offs, perm, inv = elb.router_dispatch(idx, N_E)
    delta, mv = elb.smebu_update(counts, bd, md, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa,
                                 gamma=wl.gamma, want_delta=True)
    bf, mf = to_dev(b0), to_dev(m0)
    out = elb.RouterStep(wd, bf, mf, K, T, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa, gamma=wl.gamma,
                         want_delta=True)(xd)
    torch.cuda.synchronize()
    for a, b in [(out.topk_idx, idx), (out.gates, gates), (out.offsets, offs), (out.perm, perm),
                 (out.inv_perm, inv), (bf, bd), (mf, md)]:
        assert torch.equal(a, b)
    idx_h, gates_h, counts_h = idx.cpu().numpy(), gates.cpu().numpy(), counts.cpu().numpy()
    assert idx_h.min() >= 0 and idx_h.max() < N_E
    assert (np.diff(np.sort(idx_h, axis=1), axis=1) > 0).all()
    assert np.allclose(gates_h.sum(1), 1.0, atol=2e-6)
    counts64 = check_counts(counts_h, idx_h, N_E)
    check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx_h, N_E)
    check_balance(wl.mode, counts64, b0, m0, bd.cpu().numpy(), md.cpu().numpy(), wl, delta.cpu().numpy())
    check_maxvio(mv.cpu().numpy(), counts64)
    mark = 2 ** 32 // (D * 2)  # the first row past 4 GiB of tokens
    rows = sample_rows(T, 1500, seed=7, extra=range(mark - 8, mark + 8))
    xs = host_rows(xd, rows)
    rep = compare_route(idx_h[rows], gates_h[rows], xs, w, b0, K)
    log(f"  routing: {rep.n_tokens} sampled tokens, ties {rep.ties}, gate rel err {rep.max_gate_rel:.2e}")

    # ---- permute and combine: xp is 17.7 GB, y 8.9 GB ----
    xp = elb.permute_rows(xd, inv, K)
    rows_t = torch.from_numpy(rows).to("cuda")
    pos = inv.view(T, K)[rows_t].long()  # [n, K]
    for j in range(K):
        assert torch.equal(xp[pos[:, j]], xd[rows_t]), f"permuted copy {j} differs"
    y = elb.unpermute_combine(xp, gates, inv)
    del xp
    y_h = y[rows_t].cpu().numpy().astype(np.float64)
    del y
    x64 = oracle.widen(xs)
    g64 = gates_h[rows].astype(np.float64)
    want = g64.sum(1, keepdims=True) * x64  # every copy of a token is the token itself
    bound = (K + 1) * 2.0 ** -24 * np.abs(g64).sum(1, keepdims=True) * np.abs(x64)
    assert (np.abs(y_h - want) <= bound + 1e-30).all(), "combine beyond its rounding bound"

    # ---- backward: dX (8.9 GB, fp32) on sampled rows against the oracle ----
    dg = torch.randn((T, K), generator=gen, device="cuda")
    zc = 1e-3
    dx, _ = elb.router_backward(xd, wd, idx, dg, zloss_coef=zc, want_dw=False)
    dx_h = dx[rows_t].cpu().numpy().astype(np.float64)
    del dx
    w64 = oracle.widen(w)
    z = oracle.router_logits(xs, w)
    dz = oracle.logit_grads(z, idx_h[rows], dg.cpu().numpy()[rows], normalize=True, zloss_coef=0.0)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    dz += zc * (2.0 / T) * (zmax + np.log(e.sum(axis=1, keepdims=True))) * e / e.sum(axis=1, keepdims=True)
    bound = (2.0 ** -8 + 2.0 ** -16 + 256 * 2.0 ** -24) * (np.abs(dz) @ np.abs(w64))
    err = np.abs(dx_h - dz @ w64)
    assert (err <= bound + 1e-30).all(), f"dx sampled: worst {err.max():.3g}"

    # ---- dW over the whole batch equals the sum over its two halves (no z-loss) ----
    _, dw = elb.router_backward(xd, wd, idx, dg, want_dx=False)
    h = 360_448  # a multiple of 256: the halves keep the same 256-token tiles
    _, dw1 = elb.router_backward(xd[:h], wd, idx[:h], dg[:h], want_dx=False)
    _, dw2 = elb.router_backward(xd[h:], wd, idx[h:], dg[h:], want_dx=False)
    torch.cuda.synchronize()
    full, parts = dw.double().cpu().numpy(), (dw1.double() + dw2.double()).cpu().numpy()
    scale = np.abs(full).max()
    assert scale > 0 and np.abs(full - parts).max() <= 1e-4 * scale, np.abs(full - parts).max() / scale
    log(f"  dW halves agree to {np.abs(full - parts).max() / scale:.1e} of max |dW|")

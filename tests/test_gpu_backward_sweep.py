"""A seeded random sweep of the router backward against the oracle's chain rule (pinned by
finite differences): N_r from 1 to 256, every K, d of 1-40 stages of 64 (one to several column
tiles), T up to 2500 (from one token range to dozens), raw and normalised gates, with and
without the z-loss, fp32 and bf16 dX; 20 draws from a fixed seed.  Bounds as in
test_gpu_backward.py; the bf16 dX must be the fp32 dX rounded to nearest even, bit for bit."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
import oracle
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def draws(n=20, seed=4096):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        n_e = int(rng.choice([1, 5, 16, 64, 100, 128, 200, 256]))
        k = int(rng.integers(1, min(8, n_e) + 1))
        d = 64 * int(rng.integers(1, 41))
        T = int(rng.integers(1, 2500))
        normalize = bool(rng.random() < 0.7)
        zc = 0.0 if rng.random() < 0.4 else float(10 ** rng.uniform(-4, -0.5))
        bf16_dx = bool(rng.random() < 0.3)
        out.append((i, T, d, n_e, k, normalize, zc, bf16_dx))
    return out


@pytest.mark.parametrize("i,T,d,n_e,k,normalize,zc,bf16_dx", draws())
def test_backward_sweep(i, T, d, n_e, k, normalize, zc, bf16_dx):
    log(f"backward sweep {i}: T={T} d={d} N_r={n_e} K={k} normalize={normalize} zloss={zc:.3g} bf16_dx={bf16_dx}")
    wl = datagen.WORKLOADS["large"].replace(T=T, d=d, n_experts=n_e, k=k, seed=7000 + i, n_clusters=8)
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    xd, wd = to_dev(x), to_dev(w)
    idx, _, _ = elb.router_forward(xd, wd, to_dev(b), k, gates_raw=not normalize)
    G = np.random.default_rng(i).standard_normal((T, k)).astype(np.float32)
    dx, dw = elb.router_backward(xd, wd, idx, to_dev(G), gates_raw=not normalize, zloss_coef=zc)
    torch.cuda.synchronize()
    if bf16_dx:  # the same accumulation, rounded to nearest even at the store
        dxb, _ = elb.router_backward(xd, wd, idx, to_dev(G), gates_raw=not normalize, zloss_coef=zc, want_dw=False,
                                     dx_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(dxb, dx.to(torch.bfloat16)), "bf16 dX is not the fp32 dX rounded to nearest even"
    z = oracle.router_logits(x, w)
    dz = oracle.logit_grads(z, idx.cpu().numpy(), G, normalize=normalize, zloss_coef=zc)
    x64, w64 = oracle.widen(x), oracle.widen(w)
    rel = 2.0 ** -8 + 2.0 ** -16  # dL/dz rounded to bf16 (8 significant bits) after its fp32 evaluation
    mag = np.abs(dz)
    extra = np.zeros_like(mag)  # absolute error of the fp32 dL/dz where it cancels
    if normalize:
        # (G_j - sum_k G_k g_k) / S cancels (exactly, with one expert or equal G): its fp32
        # evaluation errs by a few ulps of the terms, |G_j| + sum_k |G_k| g_k, not of the result.
        s = oracle.sigmoid_scores(z)
        rows = np.arange(T)[:, None]
        ix = idx.cpu().numpy().astype(np.int64)
        sel = s[rows, ix]
        S = sel.sum(axis=1, keepdims=True)
        terms = np.abs(G) + (np.abs(G) * sel / S).sum(axis=1, keepdims=True)
        extra[rows, ix] = 2.0 ** -20 * terms / S * sel * (1.0 - sel)
    bx = (rel + n_e * 2.0 ** -24) * (mag @ np.abs(w64)) + (1.0 + rel) * (extra @ np.abs(w64))
    bw = (rel + T * 2.0 ** -24) * (mag.T @ np.abs(x64)) + (1.0 + rel) * (extra.T @ np.abs(x64))
    for got, ref, bound, what in ((dx.cpu().numpy(), dz @ w64, bx, "dx"), (dw.cpu().numpy(), dz.T @ x64, bw, "dw")):
        err = np.abs(got.astype(np.float64) - ref)
        assert (err <= bound + 1e-30).all(), f"{what}: worst {err.max():.3g}"

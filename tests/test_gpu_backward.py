"""GPU parity of the router backward (elb_router_backward) against the oracle's chain rule.

The oracle (oracle/backward.py, pinned by finite differences) is evaluated at the GPU forward's
own selection.  Tolerance, elementwise, from the arithmetic: the kernel computes dL/dz in fp32
(~1e-5 relative, within 2^-16: fp32 logits, hardware exp2 / rcp / log), rounds it to bf16 (8
significant bits: at most 2^-8 relative), then accumulates the products in fp32 over n terms
(n 2^-24 relative), so
    |dx - dx_ref| <= (2^-8 + 2^-16 + n 2^-24) (|dz_ref| @ |W|)    (n = 256 experts)
    |dw - dw_ref| <= (2^-8 + 2^-16 + n 2^-24) (|dz_ref|^T @ |X|)  (n = T tokens)
"""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
import oracle
from gpu_util import log, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def make(T, d, n_e, k, seed):
    wl = datagen.WORKLOADS["large"].replace(T=T, d=d, n_experts=n_e, k=k, seed=seed, n_clusters=8)
    return datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)


def run(x, w, b, k, normalize, zc, seed):
    xd, wd = to_dev(x), to_dev(w)
    idx, gates, _ = elb.router_forward(xd, wd, to_dev(b), k, gates_raw=not normalize)
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((x.shape[0], k)).astype(np.float32)
    dx, dw = elb.router_backward(xd, wd, idx, to_dev(G), gates_raw=not normalize, zloss_coef=zc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), G, dx.cpu().numpy(), dw.cpu().numpy()


def check(got, ref, bound, what):
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > bound + 1e-30
    assert not bad.any(), f"{what}: {int(bad.sum())} elements over the bound; worst {err.max():.3g} " \
                          f"(bound there {bound.flat[np.argmax(err)]:.3g})"
    return float((err / np.maximum(bound, 1e-30)).max())


@pytest.mark.parametrize("T,d,n_e,k,normalize,zc", [
    (700, 256, 256, 4, True, 0.0),
    (300, 128, 200, 3, False, 0.5),
    (513, 64, 16, 2, True, 1e-2),
    (1024, 512, 256, 8, True, 0.1),
    (1, 64, 8, 1, True, 0.0),
    (2100, 192, 64, 4, False, 0.0),   # d not a multiple of 256: one column tile, 33 token ranges
    (777, 320, 256, 4, True, 0.05),   # two column tiles, the second with 64 live columns
    (4113, 1088, 128, 2, False, 0.0),  # 5 column tiles -> 51 token ranges of 1-2 stages
    (300, 8192, 256, 4, True, 0.02),   # wide rows: 32 column tiles, 128 W stages in the dX phase
    (200, 128, 1, 1, True, 0.3),       # a single expert: the normalised gate is 1, dL/dz only the z-loss
])
def test_backward_matches_oracle(T, d, n_e, k, normalize, zc):
    log(f"backward T={T} d={d} N_r={n_e} K={k} normalize={normalize} zloss={zc}")
    x, w, b = make(T, d, n_e, k, seed=T + d)
    idx, G, dx, dw = run(x, w, b, k, normalize, zc, seed=T)
    z = oracle.router_logits(x, w)
    dz = oracle.logit_grads(z, idx, G, normalize=normalize, zloss_coef=zc)
    x64, w64 = oracle.widen(x), oracle.widen(w)
    rx = check(dx, dz @ w64, (2.0 ** -8 + 2.0 ** -16 + n_e * 2.0 ** -24) * (np.abs(dz) @ np.abs(w64)), "dx")
    rw = check(dw, dz.T @ x64, (2.0 ** -8 + 2.0 ** -16 + T * 2.0 ** -24) * (np.abs(dz).T @ np.abs(x64)), "dw")
    log(f"  worst error / bound: dx {rx:.3f}, dw {rw:.3f}")


def test_backward_uniform_upstream_normalised_is_zero():
    """Normalised gates sum to one, so equal upstream gradients across a token's slots give
    exactly zero gradients (the chosen-expert part cancels in fp32 up to rounding)."""
    x, w, b = make(600, 256, 256, 4, seed=5)
    xd, wd = to_dev(x), to_dev(w)
    idx, gates, _ = elb.router_forward(xd, wd, to_dev(b), 4)
    G = np.repeat(np.random.default_rng(1).standard_normal((600, 1)), 4, axis=1).astype(np.float32)
    dx, dw = elb.router_backward(xd, wd, idx, to_dev(G))
    torch.cuda.synchronize()
    # |dL/dz| <= |G| (rounding of g sum, ~1e-7) s(1-s)/S: tiny against the gradients of test above.
    assert np.abs(dx.cpu().numpy()).max() < 1e-5 and np.abs(dw.cpu().numpy()).max() < 1e-3


def test_backward_empty_and_optional_outputs():
    x, w, b = make(300, 128, 64, 2, seed=9)
    wd = to_dev(w)
    empty_x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    idx0 = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    g0 = torch.zeros((0, 2), dtype=torch.float32, device="cuda")
    dx, dw = elb.router_backward(empty_x, wd, idx0, g0, zloss_coef=0.3)
    torch.cuda.synchronize()
    assert dx.shape == (0, 128) and (dw.cpu().numpy() == 0).all()
    xd = to_dev(x)
    idx, _, _ = elb.router_forward(xd, wd, to_dev(b), 2)
    G = to_dev(np.ones((300, 2), np.float32))
    dx_only, none = elb.router_backward(xd, wd, idx, G, want_dw=False)
    none2, dw_only = elb.router_backward(xd, wd, idx, G, want_dx=False)
    both = elb.router_backward(xd, wd, idx, G)
    torch.cuda.synchronize()
    assert none is None and none2 is None
    assert torch.equal(dx_only, both[0]) and torch.equal(dw_only, both[1])


def test_backward_deterministic():
    x, w, b = make(3000, 512, 256, 4, seed=13)
    a = run(x, w, b, 4, True, 0.2, seed=3)
    c = run(x, w, b, 4, True, 0.2, seed=3)
    assert np.array_equal(a[2], c[2]) and np.array_equal(a[3], c[3])


def test_backward_full_size_sampled():
    """The bench shape (T = 65536, d = 3072, N_r = 256, K = 4) with the z-loss: dx on sampled
    tokens against the oracle; dw against the oracle on all tokens of a 16384-token batch."""
    wl = datagen.WORKLOADS["large"]
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    idx, G, dx, _ = run(x, w, b, wl.k, True, 1e-2, seed=21)
    rows = sample_rows(wl.T, 400, seed=3)
    w64 = oracle.widen(w)
    z = oracle.router_logits(x[rows], w)
    # The z-loss term uses mean over the whole batch: 2 c / T with T = the batch size.
    dz = oracle.logit_grads(z, idx[rows], G[rows], normalize=True, zloss_coef=0.0)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    dz += 1e-2 * (2.0 / wl.T) * (zmax + np.log(e.sum(axis=1, keepdims=True))) * e / e.sum(axis=1, keepdims=True)
    check(dx[rows], dz @ w64, (2.0 ** -8 + 2.0 ** -16 + 256 * 2.0 ** -24) * (np.abs(dz) @ np.abs(w64)), "dx sampled")
    # dw needs every token's dz: a 16384-token batch of the same workload.
    T2 = 16384
    idx2, G2, _, dw = run(x[:T2], w, b, wl.k, True, 1e-2, seed=22)
    dz2 = oracle.logit_grads(oracle.router_logits(x[:T2], w), idx2, G2, normalize=True, zloss_coef=1e-2)
    x64 = oracle.widen(x[:T2])
    check(dw, dz2.T @ x64, (2.0 ** -8 + 2.0 ** -16 + T2 * 2.0 ** -24) * (np.abs(dz2).T @ np.abs(x64)), "dw 16384 tokens")


def test_backward_stress_size():
    """The largest workload (T = 262144, d = 4096: 16 column tiles x 16 token ranges of 16384
    tokens for dW), with the z-loss: dx on sampled tokens, dw against the oracle over the whole
    batch, accumulated in 16384-token chunks (the chain rule is per token, dw a sum over them)."""
    wl = datagen.WORKLOADS["stress"]
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    log(f"backward stress T={wl.T} d={wl.d}")
    zc = 1e-3
    idx, G, dx, dw = run(x, w, b, wl.k, True, zc, seed=31)
    w64 = oracle.widen(w)
    rows = sample_rows(wl.T, 300, seed=5)
    z = oracle.router_logits(x[rows], w)
    dz = oracle.logit_grads(z, idx[rows], G[rows], normalize=True, zloss_coef=0.0)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    dz += zc * (2.0 / wl.T) * (zmax + np.log(e.sum(axis=1, keepdims=True))) * e / e.sum(axis=1, keepdims=True)
    check(dx[rows], dz @ w64, (2.0 ** -8 + 2.0 ** -16 + 256 * 2.0 ** -24) * (np.abs(dz) @ np.abs(w64)), "dx sampled")
    ref = np.zeros((wl.n_experts, wl.d))
    mag = np.zeros((wl.n_experts, wl.d))
    C = 16384
    for c0 in range(0, wl.T, C):
        zc_ = oracle.router_logits(x[c0:c0 + C], w)
        d_ = oracle.logit_grads(zc_, idx[c0:c0 + C], G[c0:c0 + C], normalize=True, zloss_coef=0.0)
        zm = zc_.max(axis=1, keepdims=True)
        ec = np.exp(zc_ - zm)
        d_ += zc * (2.0 / wl.T) * (zm + np.log(ec.sum(axis=1, keepdims=True))) * ec / ec.sum(axis=1, keepdims=True)
        xc = oracle.widen(x[c0:c0 + C])
        ref += d_.T @ xc
        mag += np.abs(d_).T @ np.abs(xc)
    r = check(dw, ref, (2.0 ** -8 + 2.0 ** -16 + wl.T * 2.0 ** -24) * mag, "dw whole batch")
    log(f"  worst dw error / bound {r:.3f}")


@pytest.mark.parametrize("T,d,n_e,k", [(700, 256, 256, 4), (2100, 192, 64, 4), (4113, 1088, 128, 2)])
def test_backward_bf16_dx_is_rounded_fp32(T, d, n_e, k):
    """With ELB_DX_BF16 the kernel runs the same fp32 accumulation and rounds at the store: dx in
    bf16 is exactly the fp32 dx rounded to nearest even, and dw is unchanged."""
    x, w, b = make(T, d, n_e, k, seed=T + 1)
    xd, wd = to_dev(x), to_dev(w)
    idx, _, _ = elb.router_forward(xd, wd, to_dev(b), k)
    G = to_dev(np.random.default_rng(T).standard_normal((T, k)).astype(np.float32))
    dx32, dw32 = elb.router_backward(xd, wd, idx, G, zloss_coef=0.05)
    dx16, dw16 = elb.router_backward(xd, wd, idx, G, zloss_coef=0.05, dx_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert dx16.dtype == torch.bfloat16
    assert torch.equal(dx16, dx32.to(torch.bfloat16))
    assert torch.equal(dw16, dw32)
    log(f"T={T} d={d}: bf16 dx == rne(fp32 dx)")

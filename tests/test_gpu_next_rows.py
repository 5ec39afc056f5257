"""GPU parity of the rows next to the hot path: the router z-loss reduction, the batched
multi-layer bias update with per-layer MaxVio, the expert-contiguous permute and the gated
combine, each against the oracle on the same seeded inputs.

Tolerances (derived here, from the arithmetic each kernel does):
  * z-loss: the kernel sums the given fp32 lse values in float64, so against the oracle fed the
    same lse it agrees to float64 rounding plus one fp32 rounding of the result (rtol 1e-6);
  * permute: a copy, bit-exact;
  * combine: K fused multiply-adds in fp32; each rounds once, so
    |y - y_ref| <= (K + 1) 2^-24 sum_j |g_j e_j|; a bf16 output adds the round-to-nearest-even
    half ulp, at most 2^-8 of the fp32 value (8 significant bits), i.e. 2^-8 (|y_ref| + that
    bound), and must equal the bf16 rounding of the fp32 result bit for bit;
  * batched update: per layer, the single-layer bar (1e-6 against the oracle), and bit-identical
    to one elb_smebu_update call per layer.
"""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
import oracle
from gpu_util import BM_TOL, check_maxvio, log, to_dev

pytestmark = pytest.mark.gpu


def bf16_bits(rng, shape, scale=1.0):
    return datagen.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def random_routing(rng, T, n_e, k):
    idx = np.stack([rng.choice(n_e, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    offs, perm, inv = oracle.dispatch_permutation(idx, n_e)
    return idx, perm.astype(np.int32), inv.astype(np.int32)


def combine_bound(eo64, g, inv, k):
    """(K + 1) 2^-24 sum_j |g_j e_j| per output element."""
    rows = inv.astype(np.int64).reshape(g.shape[0], k)
    s = np.zeros((g.shape[0], eo64.shape[1]))
    for j in range(k):
        s += np.abs(g[:, j:j + 1]) * np.abs(eo64[rows[:, j]])
    return (k + 1) * 2.0 ** -24 * s


# ------------------------------------------------------------------------- z-loss (F1)

@pytest.mark.parametrize("T", [0, 1, 1000, 1025, 8191, 8192, 16385, 70001])
def test_zloss_matches_oracle(T):
    rng = np.random.default_rng(T + 5)
    lse = (rng.standard_normal(T) * 3 + 5).astype(np.float32)
    out = elb.zloss(to_dev(lse))
    torch.cuda.synchronize()
    want = oracle.z_loss_from_lse(lse)
    got = float(out.cpu()[0])
    assert abs(got - want) <= 1e-6 * abs(want) + 1e-30, (got, want)
    again = elb.zloss(to_dev(lse))
    torch.cuda.synchronize()
    assert float(again.cpu()[0]) == got  # deterministic


@pytest.mark.parametrize("shift", [1, 2, 3])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 4099, 70001])
def test_zloss_unaligned_start(T, shift):
    """lse starting 4, 8 or 12 bytes past a 16-byte boundary (the kernel adds the elements before
    the first boundary separately): the same bar against the oracle."""
    rng = np.random.default_rng(T * 7 + shift)
    lse = (rng.standard_normal(T) * 3 + 5).astype(np.float32)
    buf = torch.zeros(T + 8, dtype=torch.float32, device="cuda")
    view = buf[shift:shift + T]
    view.copy_(torch.from_numpy(lse))
    assert view.data_ptr() % 16 == 4 * shift
    out = elb.zloss(view)
    torch.cuda.synchronize()
    want = oracle.z_loss_from_lse(lse)
    got = float(out.cpu()[0])
    assert abs(got - want) <= 1e-6 * abs(want) + 1e-30, (got, want)


def test_zloss_fused_in_step():
    """RouterStep's z-loss equals elb_zloss of its own lse, and its lse matches the oracle's."""
    wl = datagen.WORKLOADS["large"].replace(T=1500, d=512, seed=77, n_clusters=8)
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    step = elb.RouterStep(to_dev(w), to_dev(b), torch.zeros(256, device="cuda"), 4, wl.T, want_zloss=True)
    out = step(to_dev(x))
    torch.cuda.synchronize()
    lse = out.lse.cpu().numpy()
    direct = elb.zloss(out.lse)
    torch.cuda.synchronize()
    assert float(direct.cpu()[0]) == float(out.zloss.cpu()[0])
    want_loss, want_lse = oracle.router_z_loss(oracle.router_logits(x, w))
    assert np.abs(lse - want_lse).max() <= 2e-2 * np.abs(want_lse).max()
    assert abs(float(out.zloss.cpu()[0]) - want_loss) <= 2e-2 * want_loss
    log(f"z-loss gpu {float(out.zloss.cpu()[0]):.6f} oracle {want_loss:.6f}")


# ------------------------------------------------------------------------- layers (F2)

@pytest.mark.parametrize("mode", ["smebu", "sign", "linear"])
def test_update_layers_matches_oracle(mode):
    L, n_e = 61, 256
    rng = np.random.default_rng(100 + len(mode))
    counts = np.stack([rng.multinomial(4 * 8192, rng.dirichlet(np.full(n_e, 0.5 + l % 5))) for l in range(L)])
    counts = counts.astype(np.int32)
    counts[3] = 128        # uniform layer
    counts[7, :40] = 0     # dead experts
    counts[11] = 0         # a layer with no tokens: skipped
    b0 = (rng.standard_normal((L, n_e)) * 0.01).astype(np.float32)
    m0 = (rng.standard_normal((L, n_e)) * 1e-4).astype(np.float32) if mode != "sign" else np.zeros((L, n_e), np.float32)
    wl = datagen.WORKLOADS["large"]
    kw = dict(mode=mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa, gamma=1e-3)
    cd, bd, md = to_dev(counts), to_dev(b0), to_dev(m0)
    delta, mv = elb.smebu_update_layers(cd, bd, md, want_delta=True, clear_counts=True, **kw)
    torch.cuda.synchronize()
    assert (cd.cpu().numpy() == 0).all(), "clear_counts zeroes every layer's loads"
    b_gpu, m_gpu, d_gpu, mv_gpu = (t.cpu().numpy() for t in (bd, md, delta, mv))
    steps = oracle.balance_layers(counts, b0, m0, **kw)
    for l, st in enumerate(steps):
        assert np.abs(b_gpu[l] - st.bias).max() <= BM_TOL, l
        assert np.abs(m_gpu[l] - st.momentum).max() <= BM_TOL, l
        assert np.abs(d_gpu[l] - st.delta_b).max() <= BM_TOL, l
        check_maxvio(mv_gpu[l], counts[l])
    # Bit-identical to one single-layer call per layer.
    for l in (0, 3, 7, 11, L - 1):
        b1, m1 = to_dev(b0[l]), to_dev(m0[l])
        d1, mv1 = elb.smebu_update(to_dev(counts[l]), b1, m1, want_delta=True, **kw)
        torch.cuda.synchronize()
        for got, want in ((b1, b_gpu[l]), (m1, m_gpu[l]), (d1, d_gpu[l]), (mv1, mv_gpu[l])):
            assert np.array_equal(got.cpu().numpy(), want, equal_nan=True), l


def test_update_layers_single_layer_and_many_experts():
    rng = np.random.default_rng(8)
    for L, n_e in ((1, 4), (2, 1024), (300, 16)):
        counts = rng.integers(0, 50, size=(L, n_e)).astype(np.int32)
        b0 = (rng.standard_normal((L, n_e)) * 0.01).astype(np.float32)
        m0 = np.zeros((L, n_e), np.float32)
        bd, md = to_dev(b0), to_dev(m0)
        _, mv = elb.smebu_update_layers(to_dev(counts), bd, md)
        torch.cuda.synchronize()
        for l, st in enumerate(oracle.balance_layers(counts, b0, m0)):
            assert np.abs(bd.cpu().numpy()[l] - st.bias).max() <= BM_TOL
            check_maxvio(mv.cpu().numpy()[l], counts[l])


# ------------------------------------------------------------------------- permute / combine (F3)

@pytest.mark.parametrize("T,d,n_e,k,dtype", [
    (1, 8, 4, 1, "bf16"), (1001, 256, 256, 4, "bf16"), (777, 3072, 256, 4, "bf16"), (300, 100, 16, 2, "f32"),
    (513, 64, 64, 8, "bf16"), (200, 4104, 32, 3, "bf16"), (0, 256, 256, 4, "bf16"),
])
def test_permute_rows_bit_exact(T, d, n_e, k, dtype):
    log(f"permute T={T} d={d} K={k} {dtype}")
    rng = np.random.default_rng(T + d)
    x = bf16_bits(rng, (T, d)) if dtype == "bf16" else rng.standard_normal((T, d)).astype(np.float32)
    idx, perm, inv = random_routing(rng, T, n_e, k) if T else (None, np.zeros(0, np.int32), np.zeros(0, np.int32))
    xp = elb.permute_rows(to_dev(x), to_dev(inv), k)
    torch.cuda.synchronize()
    got = xp.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else xp.cpu().numpy()
    want = oracle.permute_rows(x, perm, k)
    assert got.shape == want.shape and (got == want).all()


@pytest.mark.parametrize("T,d,n_e,k,in_dt", [
    (1001, 256, 256, 4, "bf16"), (777, 3072, 256, 4, "bf16"), (300, 100, 16, 2, "f32"), (513, 64, 64, 8, "bf16"),
    (129, 8, 8, 1, "bf16"), (65, 4, 5, 3, "f32"),
])
def test_combine_matches_oracle(T, d, n_e, k, in_dt):
    log(f"combine T={T} d={d} K={k} in={in_dt}")
    rng = np.random.default_rng(3 * T + d)
    _, perm, inv = random_routing(rng, T, n_e, k)
    eo = bf16_bits(rng, (T * k, d), 2.0) if in_dt == "bf16" else (rng.standard_normal((T * k, d)) * 2).astype(np.float32)
    g = rng.random((T, k)).astype(np.float32)
    g /= g.sum(axis=1, keepdims=True)
    eod, gd, invd = to_dev(eo), to_dev(g), to_dev(inv)
    y32 = elb.unpermute_combine(eod, gd, invd, out_dtype=torch.float32)
    y16 = elb.unpermute_combine(eod, gd, invd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.combine(eo, g, inv, k)
    bound = combine_bound(oracle.widen(eo), g, inv, k)
    err = np.abs(y32.cpu().numpy().astype(np.float64) - ref)
    assert (err <= bound + 1e-30).all(), f"fp32 combine error {err.max()} (bound {bound.max()})"
    # bf16 output: the round-to-nearest-even of the fp32 result, bit for bit, and within the bound.
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    y16f = y16.float().cpu().numpy().astype(np.float64)
    assert (np.abs(y16f - ref) <= bound + 2.0 ** -8 * (np.abs(ref) + bound) + 1e-30).all()


def test_identity_experts_round_trip():
    """Route a batch, permute its tokens, apply identity experts and combine with the normalised
    gates: the tokens come back (sum_j g = 1), to fp32 combine accuracy."""
    wl = datagen.WORKLOADS["large"].replace(T=3000, d=512, seed=91, n_clusters=8)
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    xd = to_dev(x)
    step = elb.RouterStep(to_dev(w), to_dev(b), None, 4, wl.T, update=False)
    out = step(xd)
    xp = elb.permute_rows(xd, out.inv_perm, 4)
    y = elb.unpermute_combine(xp, out.gates, out.inv_perm)
    torch.cuda.synchronize()
    x64 = oracle.widen(x)
    g = out.gates.cpu().numpy().astype(np.float64)
    gsum = g.sum(axis=1, keepdims=True)  # 1 up to the gates' own fp32 rounding
    bound = 5 * 2.0 ** -24 * np.abs(x64) * 1.0 + np.abs(gsum - 1) * np.abs(x64)
    assert (np.abs(y.cpu().numpy() - x64 * gsum) <= bound + 1e-30).all()
    assert np.abs(y.cpu().numpy() - x64).max() <= 1e-5 * np.abs(x64).max()


def test_permute_combine_full_size_sampled():
    """The bench shape (T = 65536, d = 3072, K = 4) in the launch configuration the bench times:
    sampled rows against the oracle, and properties that hold at any size."""
    wl = datagen.WORKLOADS["large"]
    T, d, k, n_e = wl.T, wl.d, wl.k, wl.n_experts
    rng = np.random.default_rng(4242)
    x = bf16_bits(rng, (T, d))
    idx, perm, inv = random_routing(rng, T, n_e, k)
    xd, invd = to_dev(x), to_dev(inv)
    xp = elb.permute_rows(xd, invd, k)
    g = rng.random((T, k)).astype(np.float32)
    gd = to_dev(g)
    y = elb.unpermute_combine(xp, gd, invd)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[rng.choice(T * k, 2000, replace=False), [0, T * k - 1]])
    xp_s = xp[torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    assert (xp_s == x[perm[rows] // k]).all()
    toks = np.unique(np.r_[rng.choice(T, 500, replace=False), [0, T - 1]])
    ys = y[torch.from_numpy(toks).cuda()].cpu().numpy().astype(np.float64)
    x64 = oracle.widen(x[toks])
    gs = g[toks].astype(np.float64)
    ref = x64 * gs.sum(axis=1, keepdims=True)  # the experts are identities here
    bound = (k + 1) * 2.0 ** -24 * np.abs(x64) * np.abs(gs).sum(axis=1, keepdims=True)
    assert (np.abs(ys - ref) <= bound + 1e-30).all()

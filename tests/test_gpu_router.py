"""GPU parity of the router forward against the oracle, element by element, on shapes the
oracle finishes in seconds: several 256-token tiles, ragged tails, every K, padded expert
counts, exact ties, duplicate tokens, empty batches and count accumulation."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
import oracle
from gpu_util import compare_logits, compare_route, check_counts, log, to_dev

pytestmark = pytest.mark.gpu


def make(T, d, n_e, k, dtype="bf16", seed=7, kind="clusters"):
    wl = datagen.WORKLOADS["large"].replace(T=T, d=d, n_experts=n_e, k=k, dtype=dtype, seed=seed, token_kind=kind,
                                            n_clusters=8 if kind == "clusters" else 0)
    return wl, datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)


def run(x, w, b, k, **kw):
    res = elb.router_forward(to_dev(x), to_dev(w), to_dev(b), k, want_logits=True, **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in res]


@pytest.mark.parametrize("T,d,n_e,k,kind", [
    (1000, 256, 256, 4, "clusters"),   # 4 tiles, ragged tail of 232
    (256, 512, 256, 4, "iid"),         # exactly one tile
    (777, 320, 256, 1, "iid"),
    (513, 192, 256, 2, "clusters"),
    (300, 128, 256, 3, "iid"),
    (640, 256, 256, 8, "clusters"),
    (450, 256, 200, 4, "iid"),         # padded experts (200 of 256)
    (129, 64, 16, 2, "iid"),           # tiny expert count, d = one stage
    (2048, 1024, 256, 4, "clusters"),
    (300, 8192, 256, 4, "clusters"),   # wide rows: 16 KiB per token
    (200, 128, 1, 1, "iid"),           # a single expert
    (1000, 128, 8, 8, "clusters"),     # K = N_r: every expert chosen, ordered by s + b
    (333, 64, 255, 7, "iid"),          # one padded expert slot, odd K
])
@pytest.mark.parametrize("kernel", ["mfma", "generic"])
def test_router_matches_oracle(T, d, n_e, k, kind, kernel):
    log(f"router parity kernel={kernel} T={T} d={d} N_r={n_e} K={k} tokens={kind}")
    wl, x, w, b = make(T, d, n_e, k, kind=kind)
    idx, gates, counts, logits = run(x, w, b, k, force_generic=(kernel == "generic"))
    rep = compare_route(idx, gates, x, w, b, k)
    check_counts(counts, idx, n_e)
    err = compare_logits(logits, x, w)
    log(f"  ties={rep.ties} (mismatched {rep.tie_mismatch}) order-ties={rep.order_ties} "
        f"gate rel err={rep.max_gate_rel:.2e} logit abs err={err:.2e}")


@pytest.mark.parametrize("T", [
    1000,    # 64-token tiles: 16 of them, ragged tail of 40
    16383,   # 64-token tiles: 256 of them, ragged tail of 63
    16384,   # the largest batch on 64-token tiles
    16385,   # the smallest on 128-token tiles: 129 tiles, the last holding one token
    32767,   # 128-token tiles: 256 of them, ragged tail of 127
    32768,   # the largest batch on 128-token tiles
    32769,   # the smallest on 256-token tiles: 129 tiles, the last holding one token
    40000,   # 256-token tiles with a ragged tail of 64
])
def test_router_tile_sizes(T):
    """The three MFMA tile sizes and the switches between them, with ragged tails."""
    log(f"router tile sizes T={T}")
    wl, x, w, b = make(T, 256, 256, 4, kind="clusters")
    idx, gates, counts, logits = run(x, w, b, 4)
    rep = compare_route(idx, gates, x, w, b, 4)
    check_counts(counts, idx, 256)
    compare_logits(logits, x, w)
    log(f"  ties={rep.ties} (mismatched {rep.tie_mismatch}) gate rel err={rep.max_gate_rel:.2e}")


@pytest.mark.parametrize("T,n_e,k", [(33000, 200, 8), (40000, 64, 1), (36000, 256, 3),
                                     (9000, 200, 8), (5000, 64, 1), (16000, 256, 3), (20000, 100, 5)])
def test_router_full_tile_shapes(T, n_e, k):
    """Each tile size (256 tokens on 8 waves; 128 on 8; 64 on 4) with padded experts (some waves
    hold none), several K, and the log-sum-exp combined across the two waves of a token."""
    log(f"router full tile T={T} N_r={n_e} K={k}")
    wl, x, w, b = make(T, 128, n_e, k, kind="clusters")
    res = elb.router_forward(to_dev(x), to_dev(w), to_dev(b), k, want_logits=True, want_lse=True)
    torch.cuda.synchronize()
    idx, gates, counts, logits, lse = [t.cpu().numpy() for t in res]
    compare_route(idx, gates, x, w, b, k)
    check_counts(counts, idx, n_e)
    compare_logits(logits, x, w)
    _, want = oracle.router_z_loss(oracle.router_logits(x, w))
    assert np.allclose(lse.astype(np.float64), want, rtol=1e-5, atol=1e-5), np.abs(lse - want).max()


def test_fp32_tiny_workload():
    wl = datagen.WORKLOADS["tiny"]
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    log(f"fp32 workload {wl.label}")
    idx, gates, counts, logits = run(x, w, b, wl.k)
    rep = compare_route(idx, gates, x, w, b, wl.k)
    check_counts(counts, idx, wl.n_experts)
    err = compare_logits(logits, x, w)
    assert err < 1e-5, err  # fp32 inputs keep fp32-exact logits
    log(f"  ties={rep.ties} gate rel err={rep.max_gate_rel:.2e} logit err={err:.2e}")


@pytest.mark.parametrize("kernel", ["mfma", "generic"])
def test_raw_gates(kernel):
    wl, x, w, b = make(600, 256, 256, 4)
    idx, gates, counts, _ = run(x, w, b, 4, gates_raw=True, force_generic=(kernel == "generic"))
    compare_route(idx, gates, x, w, b, 4, normalize=False)


@pytest.mark.parametrize("kernel", ["mfma", "generic"])
def test_exact_ties_go_to_the_lower_index(kernel):
    """Two pairs of experts get identical weight rows and bias, hence identical s + b in every
    token.  Pair (37, 200) is made so attractive that both are always chosen: 37 must be listed
    first.  Pair (5, 129) sits near the selection boundary: wherever only one of them fits, it
    must be 5, and wherever both are chosen, 5 comes first."""
    wl, x, w, b = make(2048, 256, 256, 4, kind="iid")
    w, b = w.copy(), b.copy()
    for lo, hi in ((37, 200), (5, 129)):
        w[hi] = w[lo]
    top = b.max()
    b[37] = b[200] = np.float32(top + 0.6)
    b[5] = b[129] = np.float32(top + 0.02)
    idx, gates, counts, _ = run(x, w, b, 4, force_generic=(kernel == "generic"))
    for lo, hi, min_both, min_one in ((37, 200, 2000, 0), (5, 129, 30, 30)):
        has_lo, has_hi = (idx == lo).any(1), (idx == hi).any(1)
        assert not (has_hi & ~has_lo).any(), f"expert {hi} chosen without its lower-index twin {lo}"
        both = has_lo & has_hi
        assert both.sum() >= min_both and (has_lo & ~has_hi).sum() >= min_one, (both.sum(), (has_lo & ~has_hi).sum())
        assert (np.argmax(idx == lo, axis=1)[both] < np.argmax(idx == hi, axis=1)[both]).all()
    compare_route(idx, gates, x, w, b, 4)


@pytest.mark.parametrize("kernel", ["mfma", "generic"])
def test_duplicate_tokens_route_identically(kernel):
    wl, x, w, b = make(1024, 256, 256, 4)
    x = x.copy()
    src = np.array([3, 3, 500, 900])
    dst = np.array([700, 1023, 255, 256])  # across tiles, waves and lane halves
    x[dst] = x[src]
    idx, gates, _, logits = run(x, w, b, 4, force_generic=(kernel == "generic"))
    assert (idx[dst] == idx[src]).all()
    assert (gates[dst].view(np.uint32) == gates[src].view(np.uint32)).all()
    assert (logits[dst].view(np.uint32) == logits[src].view(np.uint32)).all()


def test_mfma_and_generic_agree():
    """Both kernels pass the oracle protocol on the same inputs, choose the same expert sets
    wherever the choice is decided, and produce logits within fp32 accumulation noise."""
    wl, x, w, b = make(1500, 512, 256, 4)
    i1, g1, c1, z1 = run(x, w, b, 4)
    i2, g2, c2, z2 = run(x, w, b, 4, force_generic=True)
    compare_route(i1, g1, x, w, b, 4)
    compare_route(i2, g2, x, w, b, 4)
    r = oracle.route(x, w, b, 4)
    decided = r.gap >= 1e-3
    assert (np.sort(i1, 1)[decided] == np.sort(i2, 1)[decided]).all()
    assert np.allclose(z1, z2, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("kernel", ["mfma", "generic"])
def test_empty_batch_and_accumulation(kernel):
    dev = "cuda"
    wl, x, w, b = make(300, 256, 256, 4)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    counts = torch.full((256,), 123, dtype=torch.int32, device=dev)
    elb.router_forward(xd[:0], wd, bd, 4, counts=counts, force_generic=(kernel == "generic"))
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0, "empty batch must leave zero counts"
    idx1, _, _ = elb.router_forward(xd[:100], wd, bd, 4, counts=counts, force_generic=(kernel == "generic"))
    idx2, _, _ = elb.router_forward(xd[100:], wd, bd, 4, counts=counts, accumulate=True,
                                    force_generic=(kernel == "generic"))
    torch.cuda.synchronize()
    both = np.concatenate([idx1.cpu().numpy(), idx2.cpu().numpy()])
    check_counts(counts.cpu().numpy(), both, 256)
    assert int(counts.sum()) == 300 * 4


@pytest.mark.parametrize("kernel", ["mfma", "generic"])
def test_lse_for_router_z_loss(kernel):
    wl, x, w, b = make(700, 256, 256, 4)
    res = elb.router_forward(to_dev(x), to_dev(w), to_dev(b), 4, want_lse=True, force_generic=(kernel == "generic"))
    torch.cuda.synchronize()
    lse = res[3].cpu().numpy().astype(np.float64)
    _, want = oracle.router_z_loss(oracle.router_logits(x, w))
    assert np.allclose(lse, want, rtol=1e-5, atol=1e-5), np.abs(lse - want).max()


def test_bias_shift_leaves_routing_unchanged():
    """Adding one constant to every b_i changes no choice and no gate (gates never see b)."""
    wl, x, w, b = make(800, 256, 256, 4)
    i1, g1, c1, _ = run(x, w, b, 4)
    i2, g2, c2, _ = run(x, w, (b + np.float32(0.25)).astype(np.float32), 4)
    r = oracle.route(x, w, b, 4)
    decided = r.gap >= 1e-3
    assert (i1[decided] == i2[decided]).all()
    same = (i1 == i2).all(1)
    assert np.allclose(g1[same], g2[same], rtol=1e-6, atol=0)


def test_determinism():
    wl, x, w, b = make(3000, 512, 256, 4)
    a = run(x, w, b, 4)
    c = run(x, w, b, 4)
    for u, v in zip(a, c):
        assert (u.view(np.uint32) == v.view(np.uint32)).all()


@pytest.mark.parametrize("spread", [40.0, 1000.0])
@pytest.mark.parametrize("kernel", ["mfma", "generic"])
def test_wide_bias_spread(spread, kernel):
    """A bias range far wider than SMEBU ever produces: the selection must still be exact to
    the tie band.  48 experts sit near +spread/2 (jittered by 0.05), 48 near 0 and the rest near
    -spread/2, so every token picks among the top group and the scores decide; a second bias
    draws every b_i uniformly over the whole range."""
    wl, x, w, _ = make(3000, 512, 256, 4, kind="clusters")
    rng = np.random.default_rng(int(spread))
    groups = np.repeat([0.5, 0.0, -0.5], [48, 48, 160])[rng.permutation(256)]
    b1 = (groups * spread + rng.normal(0.0, 0.05, 256)).astype(np.float32)
    b2 = rng.uniform(-spread / 2, spread / 2, 256).astype(np.float32)
    for b in (b1, b2):
        log(f"bias spread {float(b.max() - b.min()):.1f} kernel={kernel}")
        idx, gates, counts, _ = run(x, w, b, 4, force_generic=(kernel == "generic"))
        rep = compare_route(idx, gates, x, w, b, 4)
        check_counts(counts, idx, 256)
        log(f"  {rep}")


@pytest.mark.parametrize("T,d", [(3000, 2048), (20000, 4096), (40000, 4096), (40000, 2048)])
def test_rotated_k_loop(T, d):
    """Rows a multiple of 4 KiB apart: every workgroup starts its k loop at another stage (all
    three tile sizes); routing and logits still match the oracle, and duplicated rows placed in
    tiles with different starting stages still choose the same experts wherever the choice is
    separated by more than the comparison's resolution."""
    log(f"rotated k loop T={T} d={d}")
    wl, x, w, b = make(T, d, 256, 4, kind="clusters")
    x = x.copy()
    src = np.array([0, 1, 2, 3, 5, 7])
    dst = np.array([300, 700, 1201, 2500, T - 1, T // 2])  # other tiles: other starting stages
    assert len(set(dst.tolist()) | set(src.tolist())) == 12
    x[dst] = x[src]
    idx, gates, counts, logits = run(x, w, b, 4)
    rep = compare_route(idx, gates, x, w, b, 4)
    check_counts(counts, idx, 256)
    compare_logits(logits, x, w)
    r = oracle.route(x[src], w, b, 4, keep=True)
    q = np.sort(r.scores + b.astype(np.float64)[None, :], axis=1)[:, ::-1][:, :5]
    sep = (np.diff(-q, axis=1) >= 1e-5).all(axis=1)
    assert (idx[dst][sep] == idx[src][sep]).all()
    assert np.allclose(logits[dst], logits[src], rtol=1e-5, atol=1e-5)
    log(f"  {rep}")

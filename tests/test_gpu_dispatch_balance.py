"""GPU parity of the dispatch permutation and of the bias updates against the oracle."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import check_balance, check_dispatch, check_maxvio, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,k,n_e,skew", [
    (1, 1, 16, 0.0), (1, 4, 256, 0.0), (257, 4, 256, 0.0), (1000, 2, 16, 1.5), (4096, 4, 256, 1.2),
    (65536, 4, 256, 1.1), (65535, 4, 256, 0.0), (65280, 2, 256, 1.0), (65537, 4, 256, 0.5), (70001, 3, 200, 0.8), (262144, 4, 256, 1.1), (5, 8, 8, 0.0),
    (1300, 8, 64, 1.0), (513, 5, 256, 0.0), (777, 6, 100, 2.0), (2049, 7, 9, 0.0), (300, 1, 1, 0.0),
])
def test_dispatch_matches_oracle(T, k, n_e, skew):
    log(f"dispatch T={T} K={k} N_r={n_e} skew={skew}")
    rng = np.random.default_rng(T + k)
    if skew:
        p = np.arange(1, n_e + 1, dtype=np.float64) ** (-skew)
        p /= p.sum()
    else:
        p = None
    idx = np.stack([rng.choice(n_e, size=k, replace=False, p=p) for _ in range(min(T, 2000))])
    idx = np.resize(idx, (T, k)).astype(np.int32)  # repeated rows beyond 2000: heavy duplication
    offs, perm, inv = elb.router_dispatch(to_dev(idx), n_e)
    torch.cuda.synchronize()
    check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx, n_e)


def test_dispatch_single_expert_and_empty():
    idx = np.zeros((3000, 1), dtype=np.int32)
    offs, perm, inv = elb.router_dispatch(to_dev(idx), 4)
    torch.cuda.synchronize()
    check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx, 4)
    empty = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    offs, perm, inv = elb.router_dispatch(empty, 256)
    torch.cuda.synchronize()
    assert (offs.cpu().numpy() == 0).all() and perm.numel() == 0


def test_dispatch_concentrated_and_repeated_ids():
    # Every token picks the same experts (each 64-lane run holds one expert 64 times), and
    # tokens that name one expert in several slots (the sort is defined for any ids).
    same = np.tile(np.array([[3, 1, 2, 0]], dtype=np.int32), (5000, 1))
    rng = np.random.default_rng(11)
    rep = rng.integers(0, 3, size=(3001, 4)).astype(np.int32)
    for idx, n_e in ((same, 256), (rep, 3), (rep, 256)):
        offs, perm, inv = elb.router_dispatch(to_dev(idx), n_e)
        torch.cuda.synchronize()
        check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx, n_e)


@pytest.mark.parametrize("T", [9000, 8900, 70000])  # 36 tiles; 35 (one padding column); 274
def test_dispatch_without_inverse_and_reused_workspace(T):
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 256, size=(T, 4)).astype(np.int32)
    need = elb.dispatch_workspace_bytes(T, 4, 256)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")  # garbage contents on entry
    for _ in range(2):
        offs, perm, inv = elb.router_dispatch(to_dev(idx), 256, workspace=ws, want_inv=False)
        torch.cuda.synchronize()
        assert inv is None
        check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), None, idx, 256)


def test_dispatch_into_given_outputs():
    """out=: the same permutation written into the caller's tensors (stale contents first);
    outputs of the wrong size are refused before any launch."""
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 200, size=(4500, 3)).astype(np.int32)
    outs = (torch.full((201,), -7, dtype=torch.int32, device="cuda"),
            torch.full((13500,), -7, dtype=torch.int32, device="cuda"),
            torch.full((13500,), -7, dtype=torch.int32, device="cuda"))
    offs, perm, inv = elb.router_dispatch(to_dev(idx), 200, out=outs)
    torch.cuda.synchronize()
    assert offs is outs[0] and perm is outs[1] and inv is outs[2]
    check_dispatch(offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), idx, 200)
    ref = elb.router_dispatch(to_dev(idx), 200)
    torch.cuda.synchronize()
    for a, b in zip((offs, perm, inv), ref):
        assert torch.equal(a, b)
    with pytest.raises(ValueError):
        elb.router_dispatch(to_dev(idx), 200, out=(outs[0], outs[1][:100], None))


WL = datagen.WORKLOADS["large"]


def random_counts(rng, n, total, skew):
    p = rng.dirichlet(np.full(n, 1.0 / max(skew, 1e-3)))
    return rng.multinomial(total, p).astype(np.int32)


@pytest.mark.parametrize("mode", ["smebu", "sign", "linear"])
@pytest.mark.parametrize("n_e", [4, 16, 256, 1000, 1024])
def test_balance_matches_oracle(mode, n_e):
    log(f"balance mode={mode} N_r={n_e}")
    rng = np.random.default_rng(n_e)
    b = (rng.standard_normal(n_e) * 0.01).astype(np.float32)
    m = (rng.standard_normal(n_e) * 1e-4).astype(np.float32) if mode != "sign" else np.zeros(n_e, np.float32)
    bd, md = to_dev(b), to_dev(m)
    for step in range(20):
        c = random_counts(rng, n_e, 4 * 32768, skew=1.0 + step)
        if step == 3:
            c[:] = 512  # exactly uniform loads
        if step == 5:
            c[: n_e // 2] = 0  # dead experts
        b_prev, m_prev = bd.cpu().numpy(), md.cpu().numpy()
        delta, mv = elb.smebu_update(to_dev(c), bd, md, mode=mode, lam=WL.lam, beta=WL.beta, kappa=WL.kappa,
                                     gamma=1e-3, want_delta=True)
        torch.cuda.synchronize()
        check_balance(mode, c, b_prev, m_prev, bd.cpu().numpy(), md.cpu().numpy(), WL.replace(gamma=1e-3),
                      delta.cpu().numpy())
        check_maxvio(mv.cpu().numpy(), c)


def test_worked_example_on_gpu():
    """n = [8, 4, 2, 2], b0 = [.01, -.02, .005, .005]: the two SMEBU steps worked by hand."""
    import pins

    t1, t2 = pins._tanh(1.0), pins._tanh(2.0)
    lam, beta = 5e-4, 0.5
    db = lam * np.array([-t2, 0.0, t1, t1]) - lam * (2 * t1 - t2) / 4
    b0 = np.array([0.01, -0.02, 0.005, 0.005])
    m1 = (1 - beta) * db
    b1 = b0 + m1
    m2 = beta * m1 + (1 - beta) * db
    b2 = b1 + m2
    bd, md = to_dev(b0.astype(np.float32)), torch.zeros(4, dtype=torch.float32, device="cuda")
    c = to_dev(np.array([8, 4, 2, 2], dtype=np.int32))
    elb.smebu_update(c, bd, md)
    torch.cuda.synchronize()
    assert np.abs(bd.cpu().numpy() - b1).max() < 1e-6 and np.abs(md.cpu().numpy() - m1).max() < 1e-7
    _, mv = elb.smebu_update(c, bd, md)
    torch.cuda.synchronize()
    assert np.abs(bd.cpu().numpy() - b2).max() < 1e-6 and np.abs(md.cpu().numpy() - m2).max() < 1e-7
    assert mv.cpu().numpy().tolist() == [4.0, 1.0]


def test_no_tokens_skips_update():
    b0 = np.array([0.1, -0.2, 0.3], dtype=np.float32)
    m0 = np.array([0.01, 0.02, 0.03], dtype=np.float32)
    b, m = to_dev(b0), to_dev(m0)
    for mode in ("smebu", "sign", "linear"):
        delta, mv = elb.smebu_update(torch.zeros(3, dtype=torch.int32, device="cuda"), b, m, mode=mode,
                                     want_delta=True)
        torch.cuda.synchronize()
        assert (b.cpu().numpy() == b0).all() and (m.cpu().numpy() == m0).all()
        assert (delta.cpu().numpy() == 0).all() and np.isnan(mv.cpu().numpy()).all()


def test_maxvio_entry_point():
    for c in ([8, 4, 2, 2], [5, 5, 5, 5], [3, 0, 1], [12, 1, 4, 3], [0, 0]):
        arr = np.array(c, dtype=np.int32)
        mv = elb.maxvio(to_dev(arr))
        torch.cuda.synchronize()
        check_maxvio(mv.cpu().numpy(), arr)


@pytest.mark.parametrize("mode", ["smebu", "sign"])
def test_balance_clear_counts(mode):
    """ELB_CLEAR_COUNTS: identical update, and the loads are zero afterwards."""
    rng = np.random.default_rng(5)
    c = random_counts(rng, 256, 4 * 65536, skew=2.0)
    b0 = (rng.standard_normal(256) * 0.01).astype(np.float32)
    m0 = (rng.standard_normal(256) * 1e-4).astype(np.float32)
    outs = []
    for clear in (False, True):
        cd, bd, md = to_dev(c), to_dev(b0), to_dev(m0)
        delta, mv = elb.smebu_update(cd, bd, md, mode=mode, want_delta=True, clear_counts=clear)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (bd, md, delta, mv)])
        assert (cd.cpu().numpy() == (0 if clear else c)).all()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)

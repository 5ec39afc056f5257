"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, not by the oracle.

Every pin takes the oracle package as an argument (``orc``) so the same checks can be run
against deliberately broken copies of it (tests/test_oracle_mutants.py): a pin set is only
worth something if a plausible slip in the oracle makes one of them fail.

Sources of the expected values, pin by pin:
  * closed forms worked by hand from the equations of "SMEBU Load Balancing" ("How it
    works", eq. (20)-(28)), written as exact rationals or via math.exp, not via the
    oracle's numpy expressions;
  * the study note's own numeric fact that a 2x overloaded expert has v_i = -1 whatever the
    batch size (same section, after eq. (24));
  * brute force over every K-subset of experts on tiny inputs;
  * pure-Python loops (matrix product, bucket sort, logsumexp) and scipy's expit;
  * hand-decoded bf16 bit patterns.
"""

from __future__ import annotations

import itertools
import struct
import math
from fractions import Fraction

import numpy as np

LAM, BETA, KAPPA, GAMMA = 5e-4, 0.5, 2.0, 1e-3


def _tanh(x: float) -> float:
    """tanh from its exponential definition (independent of numpy's tanh)."""
    e = math.exp(2.0 * x)
    return (e - 1.0) / (e + 1.0)


def _close(a, b, rtol=1e-12, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.allclose(a, b, rtol=rtol, atol=atol), f"{what}: {a} != {b}"


# ------------------------------------------------------------------ router ---------------

def pin_widen_bf16(orc):
    """bf16 bit patterns decoded by hand: sign * 1.mantissa * 2^(exp-127), denormals too."""
    pats = {0x3F80: 1.0, 0xC000: -2.0, 0x3F81: 1.0 + 2.0 ** -7, 0x0001: 2.0 ** -133,
            0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x8000: -0.0, 0x3E80: 0.25}
    bits = np.array(list(pats), dtype=np.uint16)
    _close(orc.widen(bits), list(pats.values()), rtol=0, what="bf16 decode")


def pin_logits_naive(orc):
    """z[t,i] = sum_k x[t,k] w[i,k] against a pure-Python triple loop (fp32 and bf16 inputs)."""
    rng = np.random.default_rng(7)
    for dt in ("f32", "bf16"):
        x = rng.standard_normal((5, 7)).astype(np.float32)
        w = rng.standard_normal((3, 7)).astype(np.float32)
        if dt == "bf16":
            x = (x.view(np.uint32) >> 16).astype(np.uint16)
            w = (w.view(np.uint32) >> 16).astype(np.uint16)
            dec = lambda v: struct.unpack(">f", struct.pack(">I", int(v) << 16))[0]  # noqa: E731
            xv = [[dec(v) for v in row] for row in x]
            wv = [[dec(v) for v in row] for row in w]
        else:
            xv = [[float(v) for v in row] for row in x]
            wv = [[float(v) for v in row] for row in w]
        ref = [[sum(xv[t][k] * wv[i][k] for k in range(7)) for i in range(3)] for t in range(5)]
        _close(orc.router_logits(x, w), ref, rtol=1e-12, atol=1e-14, what=f"logits {dt}")


def pin_sigmoid(orc):
    """sigma(0) = 1/2, sigma(-z) = 1 - sigma(z), scipy's expit, saturation without NaN."""
    from scipy.special import expit

    z = np.linspace(-30, 30, 601)
    s = orc.sigmoid_scores(z)
    _close(orc.sigmoid_scores(np.array([0.0])), [0.5], rtol=0, what="sigma(0)")
    _close(s + orc.sigmoid_scores(-z), np.ones_like(z), rtol=1e-15, atol=1e-15, what="symmetry")
    _close(s, expit(z), rtol=1e-14, atol=1e-300, what="expit")
    big = orc.sigmoid_scores(np.array([-1000.0, 1000.0]))
    _close(big, [0.0, 1.0], rtol=0, atol=0, what="saturation")


def pin_topk_bruteforce(orc):
    """The chosen set maximises sum q over all K-subsets; listed in descending q; gap exact."""
    rng = np.random.default_rng(11)
    for n, k in ((8, 1), (8, 2), (8, 3), (8, 4), (16, 2), (6, 6)):
        q = rng.standard_normal((20, n))
        idx, gap = orc.select_topk(q, k)
        for t in range(q.shape[0]):
            best = max(itertools.combinations(range(n), k), key=lambda c: sum(q[t, list(c)]))
            assert set(idx[t].tolist()) == set(best), (n, k, t)
            vals = q[t, idx[t]]
            assert all(vals[j] > vals[j + 1] for j in range(k - 1)), "not descending"
            rest = [q[t, i] for i in range(n) if i not in best]
            want = (min(vals) - max(rest)) if rest else math.inf
            assert gap[t] == want, ("gap", gap[t], want)


def pin_topk_ties(orc):
    """Equal q: the lower expert index is chosen first."""
    q = np.array([[0.5, 0.7, 0.7, 0.1], [0.3, 0.3, 0.3, 0.3], [0.1, 0.2, 0.2, 0.2]])
    idx2, gap2 = orc.select_topk(q, 2)
    assert idx2.tolist() == [[1, 2], [0, 1], [1, 2]], idx2.tolist()
    assert gap2.tolist() == [0.7 - 0.5, 0.0, 0.0]
    idx3, _ = orc.select_topk(q, 3)
    assert idx3.tolist() == [[1, 2, 0], [0, 1, 2], [1, 2, 3]], idx3.tolist()


def pin_bias_after_sigmoid(orc):
    """Top-K ranks sigmoid(z) + b (eq. (17)); a bias inside the sigmoid would choose otherwise.

    z = [4, 0], b = [0, 0.5]: sigmoid(4) + 0 = 0.982 < sigmoid(0) + 0.5 = 1.0, so expert 1
    wins, whereas sigmoid(4 + 0) = 0.982 > sigmoid(0 + 0.5) = 0.622 would pick expert 0.
    """
    x = np.array([[1.0]], dtype=np.float32)
    w = np.array([[4.0], [0.0]], dtype=np.float32)
    r = orc.route(x, w, np.array([0.0, 0.5]), 1)
    assert r.idx.tolist() == [[1]], r.idx.tolist()


def pin_gates_hand(orc):
    """Gates from s only: z = [0, ln 3] -> s = [1/2, 3/4]; normalised gates 0.6 / 0.4.

    With b = [0.3, 0] the order flips (q = [0.8, 0.75]) but each expert keeps its gate.
    """
    x = np.array([[1.0]], dtype=np.float32)
    w = np.array([[0.0], [math.log(3.0)]], dtype=np.float32)
    ln3 = float(np.float32(math.log(3.0)))
    s1 = 1.0 / (1.0 + math.exp(-ln3))
    r = orc.route(x, w, np.zeros(2), 2)
    assert r.idx.tolist() == [[1, 0]]
    _close(r.gates, [[s1 / (s1 + 0.5), 0.5 / (s1 + 0.5)]], rtol=1e-15, what="normalised gates")
    r = orc.route(x, w, np.array([0.3, 0.0]), 2)
    assert r.idx.tolist() == [[0, 1]]
    _close(r.gates, [[0.5 / (s1 + 0.5), s1 / (s1 + 0.5)]], rtol=1e-15, what="gates with bias")
    r = orc.route(x, w, np.zeros(2), 2, normalize=False)
    _close(r.gates, [[s1, 0.5]], rtol=1e-15, what="raw gates")
    r = orc.route(x, w, np.zeros(2), 1)
    _close(r.gates, [[1.0]], rtol=0, what="K=1 normalised gate")


def pin_bias_shift_invariance(orc):
    """Adding one constant to every b_i changes neither the choice nor the gates."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    w = (rng.standard_normal((16, 32)) * 0.3).astype(np.float32)
    b = rng.standard_normal(16) * 0.05
    r0 = orc.route(x, w, b, 4)
    r1 = orc.route(x, w, b + 0.125, 4)
    ok = r0.gap > 1e-9
    assert (r0.idx[ok] == r1.idx[ok]).all()
    _close(r0.gates[ok], r1.gates[ok], rtol=1e-13, what="gates under bias shift")


# ------------------------------------------------------------------ loads ----------------

def pin_counts_naive(orc):
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 10, size=(200, 3))
    want = [0] * 10
    for e in idx.ravel().tolist():
        want[e] += 1
    got = orc.expert_loads(idx, 10)
    assert got.tolist() == want and int(got.sum()) == idx.size


def pin_maxvio_hand(orc):
    """MaxVio = max load / min load (the talk's definition); relative excess (max-nbar)/nbar."""
    r, e = orc.max_violation(np.array([8, 4, 2, 2]))
    assert (r, e) == (4.0, 1.0), (r, e)
    r, e = orc.max_violation(np.array([5, 5, 5, 5]))
    assert (r, e) == (1.0, 0.0)
    r, e = orc.max_violation(np.array([3, 0, 1]))
    assert r == math.inf and abs(e - 1.25) < 1e-15, (r, e)
    r, e = orc.max_violation(np.array([12, 1, 4, 3]))  # nbar = 5
    assert (r, e) == (12.0, 1.4), (r, e)
    r, e = orc.max_violation(np.zeros(4, dtype=np.int64))
    assert math.isnan(r) and math.isnan(e)


def pin_dispatch_naive(orc):
    """Counting sort against a pure-Python bucket loop, plus the permutation's invariants."""
    rng = np.random.default_rng(9)
    n_e = 12
    idx = rng.integers(0, n_e, size=(300, 4))
    idx[7] = idx[3]  # repeated rows
    flat = idx.ravel().tolist()
    perm_ref, offs_ref = [], [0]
    for e in range(n_e):
        perm_ref += [j for j, v in enumerate(flat) if v == e]
        offs_ref.append(len(perm_ref))
    offsets, perm, inv = orc.dispatch_permutation(idx, n_e)
    assert perm.tolist() == perm_ref and offsets.tolist() == offs_ref
    assert (perm[inv] == np.arange(len(flat))).all()
    assert offsets[-1] == len(flat)


# ------------------------------------------------------------------ balance --------------

def pin_violation_scale_free(orc):
    """A 2x overloaded expert has v = -1 whether the batch holds 10^3 or 10^7 assignments."""
    for a in (250, 2_500_000):
        counts = np.array([2 * a, a // 2, a // 2, a])  # sum 4a, nbar = a
        v = orc.normalized_violation(counts)
        _close(v, [-1.0, 0.5, 0.5, 0.0], rtol=0, atol=0, what=f"v at nbar={a}")


def pin_uniform_loads(orc):
    """Balanced loads give a zero step; the momentum then only decays: m' = beta m, b' = b + m'."""
    b = np.array([0.01, -0.02, 0.004, 0.006])
    m = np.array([1e-4, -2e-4, 3e-4, -2e-4])
    n = np.array([7, 7, 7, 7])
    for mode in ("smebu", "linear"):
        st = orc.balance_step(n, b, m, mode=mode, lam=LAM, beta=BETA, kappa=KAPPA)
        _close(st.delta_b, np.zeros(4), rtol=0, atol=0, what=f"{mode} zero step")
        _close(st.momentum, BETA * m, rtol=0, atol=0, what=f"{mode} decayed momentum")
        _close(st.bias, b + BETA * m, rtol=0, atol=0, what=f"{mode} bias")
    st = orc.balance_step(n, b, m, mode="sign", gamma=GAMMA)
    _close(st.delta_b, np.zeros(4), rtol=0, atol=0, what="sign zero step")
    _close(st.bias, b - b.mean(), rtol=1e-15, atol=1e-18, what="sign re-centre only")
    _close(st.momentum, m, rtol=0, atol=0, what="sign leaves m")


def pin_recentred_bounds(orc):
    """After (26): sum db = 0; before it |db| < lambda; after it |db| <= 2 lambda (N-1)/N."""
    rng = np.random.default_rng(13)
    for _ in range(20):
        n = rng.integers(0, 50, size=32)
        n[0] = 0
        st = orc.balance_step(n, np.zeros(32), np.zeros(32), mode="smebu", lam=LAM, beta=BETA, kappa=KAPPA)
        assert abs(st.delta_b.sum()) < 1e-17
        assert np.all(np.abs(st.delta_b_raw) < LAM)
        assert np.all(np.abs(st.delta_b) <= 2 * LAM * 31 / 32)
        st = orc.balance_step(n, np.zeros(32), np.zeros(32), mode="linear", lam=LAM, beta=BETA)
        assert abs(st.delta_b_raw.sum()) < 1e-15 and abs(st.delta_b.sum()) < 1e-17


def pin_direction(orc):
    """Under-used experts (n_i < nbar) get a positive step, over-used ones a negative step."""
    n = np.array([1, 9, 4, 6, 0, 12])  # nbar = 32 / 6
    nbar = n.sum() / len(n)
    for mode in ("smebu", "linear", "sign"):
        st = orc.balance_step(n, np.zeros(6), np.zeros(6), mode=mode, lam=LAM, beta=BETA,
                              kappa=KAPPA, gamma=GAMMA)
        assert np.all(np.sign(st.delta_b_raw) == np.sign(nbar - n)), mode


def pin_dead_expert(orc):
    """n_i = 0 gives v_i = 1 and a raw step of lambda * tanh(kappa) = lambda * tanh(2)."""
    st = orc.balance_step(np.array([0, 4, 4, 4]), np.zeros(4), np.zeros(4), mode="smebu",
                          lam=LAM, beta=BETA, kappa=KAPPA)
    _close(st.delta_b_raw[0], LAM * _tanh(2.0), rtol=1e-14, what="lambda tanh 2")
    _close(LAM * _tanh(2.0), 4.8201379003790845e-4, rtol=1e-15, what="constant")


def pin_momentum_closed_form(orc):
    """With m_0 = 0: m_s = (1-beta) sum_r beta^(s-r) db_r and b_s = b_0 + sum_r m_r (eq. (27)-(28))."""
    rng = np.random.default_rng(17)
    n_e = 8
    b0 = rng.standard_normal(n_e) * 0.01
    b, m = b0.copy(), np.zeros(n_e)
    dbs, ms = [], []
    for s in range(6):
        st = orc.balance_step(rng.integers(1, 40, size=n_e), b, m, mode="smebu", lam=LAM, beta=BETA, kappa=KAPPA)
        b, m = st.bias, st.momentum
        dbs.append(st.delta_b)
        ms.append(m)
        want = sum((1 - BETA) * BETA ** (s - r) * dbs[r] for r in range(s + 1))
        _close(m, want, rtol=1e-12, atol=1e-20, what=f"m at step {s}")
        _close(b, b0 + sum(ms), rtol=1e-12, atol=1e-18, what=f"b at step {s}")


def pin_mean_conserved(orc):
    """SMEBU/linear keep mean(b) when sum(m_0) = 0; the sign step leaves mean(b) = 0."""
    rng = np.random.default_rng(19)
    b = rng.standard_normal(16) * 0.02
    mean0 = b.mean()
    m = np.zeros(16)
    for _ in range(10):
        st = orc.balance_step(rng.integers(0, 30, size=16), b, m, mode="smebu", lam=LAM, beta=BETA, kappa=KAPPA)
        b, m = st.bias, st.momentum
        assert abs(b.mean() - mean0) < 1e-16
    st = orc.balance_step(rng.integers(0, 30, size=16), b, m, mode="sign", gamma=GAMMA)
    assert abs(st.bias.mean()) < 1e-17


def pin_sign_step_hand(orc):
    """Sign step: |db| in {0, gamma}; n = [8,4,2,2], b0 = [.01,-.02,.005,.005], gamma = 1e-3.

    db = [-g, 0, g, g]; b0 + db = [.009, -.02, .006, .006], mean .00025;
    b1 = [.00875, -.02025, .00575, .00575].
    """
    b0 = np.array([0.01, -0.02, 0.005, 0.005])
    st = orc.balance_step(np.array([8, 4, 2, 2]), b0, np.zeros(4), mode="sign", gamma=GAMMA)
    _close(st.delta_b_raw, [-GAMMA, 0.0, GAMMA, GAMMA], rtol=0, what="sign step")
    _close(st.bias, [0.00875, -0.02025, 0.00575, 0.00575], rtol=1e-13, atol=1e-18, what="sign bias")


def pin_kappa_limit(orc):
    """kappa -> inf, beta = 0 turns SMEBU into the sign step with gamma = lambda when mean(b0) = 0.

    tanh(kappa v) -> sign(v); SMEBU re-centres db while the sign step re-centres b + db, and
    the two agree exactly when b0 already has zero mean.
    """
    rng = np.random.default_rng(23)
    b0 = rng.standard_normal(10) * 0.01
    b0 -= b0.mean()
    n = np.array([3, 5, 5, 9, 0, 5, 7, 2, 8, 6])  # nbar = 5: exact ties included
    a = orc.balance_step(n, b0, np.zeros(10), mode="smebu", lam=LAM, beta=0.0, kappa=1e9)
    c = orc.balance_step(n, b0, np.zeros(10), mode="sign", gamma=LAM)
    _close(a.bias, c.bias, rtol=1e-12, atol=1e-18, what="kappa limit")


def pin_linear_closed_form(orc):
    """Linear mode, v from exact rationals: db = lambda v (sum v = 0 so (26) is a no-op)."""
    n = [3, 11, 0, 6, 5]
    total = sum(n)
    v = [float(Fraction(total - len(n) * ni, total)) for ni in n]
    b0 = np.array([0.002, -0.001, 0.0, 0.0015, -0.0025])
    m0 = np.array([1e-5, 0.0, -2e-5, 3e-5, 0.0])
    st = orc.balance_step(np.array(n), b0, m0, mode="linear", lam=LAM, beta=BETA)
    m1 = BETA * m0 + (1 - BETA) * LAM * np.array(v)
    _close(st.momentum, m1, rtol=1e-13, atol=1e-20, what="linear m")
    _close(st.bias, b0 + m1, rtol=1e-13, atol=1e-20, what="linear b")


def pin_small_violation(orc):
    """Near balance SMEBU(lambda) ~ linear(lambda kappa): |tanh x - x| <= |x|^3 / 3."""
    n = np.array([1000, 1003, 998, 999, 1000, 1002, 997, 1001])
    a = orc.balance_step(n, np.zeros(8), np.zeros(8), mode="smebu", lam=LAM, beta=BETA, kappa=KAPPA)
    c = orc.balance_step(n, np.zeros(8), np.zeros(8), mode="linear", lam=LAM * KAPPA, beta=BETA)
    vmax = 3.0 / 1000.0
    assert np.all(np.abs(a.delta_b_raw - c.delta_b_raw) <= LAM * (KAPPA * vmax) ** 3 / 3 + 1e-20)
    assert np.any(a.delta_b_raw != 0)


def pin_worked_example(orc):
    """Two SMEBU steps worked by hand from eq. (23)-(28): N_r = 4, n = [8, 4, 2, 2], nbar = 4.

    v = [-1, 0, 1/2, 1/2]; raw db = lambda [-tanh 2, 0, tanh 1, tanh 1];
    mean = lambda (2 tanh 1 - tanh 2) / 4; db = raw - mean;
    m1 = (1 - beta) db; b1 = b0 + m1; same loads again: m2 = beta m1 + (1 - beta) db; b2 = b1 + m2.
    """
    t1, t2 = _tanh(1.0), _tanh(2.0)
    raw = LAM * np.array([-t2, 0.0, t1, t1])
    db = raw - LAM * (2 * t1 - t2) / 4
    b0 = np.array([0.01, -0.02, 0.005, 0.005])
    m1 = (1 - BETA) * db
    b1 = b0 + m1
    m2 = BETA * m1 + (1 - BETA) * db
    b2 = b1 + m2
    n = np.array([8, 4, 2, 2])
    s1 = orc.balance_step(n, b0, np.zeros(4), mode="smebu", lam=LAM, beta=BETA, kappa=KAPPA)
    _close(s1.delta_b_raw, raw, rtol=1e-14, what="raw db")
    _close(s1.delta_b, db, rtol=1e-13, atol=1e-19, what="db")
    _close(s1.momentum, m1, rtol=1e-13, atol=1e-19, what="m1")
    _close(s1.bias, b1, rtol=1e-13, what="b1")
    s2 = orc.balance_step(n, s1.bias, s1.momentum, mode="smebu", lam=LAM, beta=BETA, kappa=KAPPA)
    _close(s2.momentum, m2, rtol=1e-13, atol=1e-19, what="m2")
    _close(s2.bias, b2, rtol=1e-13, what="b2")
    # The same numbers to seven digits, as worked on paper.
    _close(s1.delta_b, [-5.519089e-4, -6.989509e-5, 3.109020e-4, 3.109020e-4], rtol=2e-6, what="db digits")
    _close(s2.bias, [9.310114e-3, -2.008737e-2, 5.388628e-3, 5.388628e-3], rtol=2e-6, what="b2 digits")


def pin_no_tokens(orc):
    """No routed tokens: the update is skipped (our reading; the pages never meet this case)."""
    b = np.array([0.1, -0.1])
    m = np.array([0.01, 0.02])
    for mode in ("smebu", "sign", "linear"):
        st = orc.balance_step(np.zeros(2, dtype=np.int64), b, m, mode=mode)
        assert (st.bias == b).all() and (st.momentum == m).all()


# ------------------------------------------------------------------ z-loss ---------------

def pin_zloss(orc):
    """lse of N equal logits c is c + ln N; one expert gives lse = z; random rows vs math."""
    z = np.full((3, 8), 2.5)
    loss, lse = orc.router_z_loss(z)
    _close(lse, np.full(3, 2.5 + math.log(8)), rtol=1e-15, what="equal logits")
    _close(loss, (2.5 + math.log(8)) ** 2, rtol=1e-15, what="loss equal logits")
    loss, lse = orc.router_z_loss(np.array([[-1.5], [4.0]]))
    _close(lse, [-1.5, 4.0], rtol=0, what="single expert")
    _close(loss, (2.25 + 16.0) / 2, rtol=1e-15, what="single expert loss")
    rng = np.random.default_rng(29)
    z = rng.standard_normal((4, 6)) * 3
    want = [math.log(sum(math.exp(v) for v in row)) for row in z.tolist()]
    loss, lse = orc.router_z_loss(z)
    _close(lse, want, rtol=1e-14, what="lse vs math")
    _close(loss, sum(v * v for v in want) / 4, rtol=1e-14, what="mean square")


def pin_zloss_from_lse(orc):
    """mean of squares of given per-token lse values, against a plain loop."""
    lse = [1.5, -2.0, 0.25, 3.0]
    _close(orc.z_loss_from_lse(np.array(lse)), sum(v * v for v in lse) / 4, rtol=1e-15, what="mean lse^2")
    assert orc.z_loss_from_lse(np.zeros(0)) == 0.0


# ------------------------------------------------------------------ layers ---------------

def pin_layers_independent(orc):
    """L layers updated at once equal L single-layer updates, and a layer's result depends only
    on its own loads: the worked example's layer is unaffected by its neighbours."""
    counts = np.array([[8, 4, 2, 2], [1, 1, 1, 1], [0, 0, 0, 0]])
    b0 = np.array([[0.01, -0.02, 0.005, 0.005], [0.1, 0.2, 0.3, 0.4], [0.5, 0.5, -1.0, 0.0]])
    m0 = np.zeros((3, 4))
    steps = orc.balance_layers(counts, b0, m0)
    t1, t2 = _tanh(1.0), _tanh(2.0)
    db = [LAM * v for v in (-t2, 0.0, t1, t1)]
    mean = sum(db) / 4
    b1 = [b0[0][i] + (1 - BETA) * (db[i] - mean) for i in range(4)]
    _close(steps[0].bias, b1, rtol=1e-14, what="layer 0 worked example")
    _close(steps[1].bias, b0[1], rtol=0, what="uniform layer unchanged")
    _close(steps[2].bias, b0[2], rtol=0, what="empty layer skipped")
    assert len(steps) == 3


# ------------------------------------------------------------------ permute / combine ----

def pin_permute_buckets(orc):
    """The expert-contiguous rows against a bucket loop over (token, slot) in order."""
    rng = np.random.default_rng(31)
    n_e, k = 7, 3
    idx = np.stack([rng.choice(n_e, size=k, replace=False) for _ in range(40)])
    x = rng.integers(0, 2 ** 16, size=(40, 5)).astype(np.uint16)
    want = []
    for e in range(n_e):
        for t in range(40):
            for j in range(k):
                if idx[t, j] == e:
                    want.append(x[t])
    _, perm, _ = orc.dispatch_permutation(idx, n_e)
    got = orc.permute_rows(x, perm, k)
    assert got.dtype == np.uint16 and (got == np.array(want)).all()


def pin_combine_direct(orc):
    """Combine through the permutation equals sum_j g[t,j] * E_{idx[t,j]}(x_t) computed token by
    token, for per-expert affine maps E_e(u) = (e + 1) u + e."""
    rng = np.random.default_rng(37)
    n_e, k, T, d = 6, 2, 25, 4
    idx = np.stack([rng.choice(n_e, size=k, replace=False) for _ in range(T)])
    x = rng.standard_normal((T, d)).astype(np.float32)
    g = rng.random((T, k))
    _, perm, inv = orc.dispatch_permutation(idx, n_e)
    xp = orc.permute_rows(x, perm, k).astype(np.float64)
    e_of_row = idx.ravel()[perm]
    eo = ((e_of_row[:, None] + 1.0) * xp + e_of_row[:, None]).astype(np.float32)
    got = orc.combine(eo, g, inv, k)
    for t in range(T):
        for c in range(d):
            want = 0.0
            for j in range(k):
                e = int(idx[t, j])
                want += g[t, j] * float(np.float32((e + 1.0) * float(x[t, c]) + e))
            assert abs(got[t, c] - want) <= 1e-12 * (1 + abs(want)), (t, c, got[t, c], want)


def pin_combine_identity_experts(orc):
    """Identity experts and normalised gates give back the tokens: sum_j g[t,j] = 1."""
    rng = np.random.default_rng(41)
    n_e, k, T = 9, 4, 30
    idx = np.stack([rng.choice(n_e, size=k, replace=False) for _ in range(T)])
    x = rng.standard_normal((T, 6)).astype(np.float32)
    g = rng.random((T, k))
    g /= g.sum(axis=1, keepdims=True)
    _, perm, inv = orc.dispatch_permutation(idx, n_e)
    y = orc.combine(orc.permute_rows(x, perm, k), g, inv, k)
    _close(y, x.astype(np.float64), rtol=1e-14, atol=1e-15, what="identity experts")


# ------------------------------------------------------------------ backward -------------

def _fd_case(seed, normalize, zc):
    rng = np.random.default_rng(seed)
    T, d, n_e, k = 5, 6, 7, 3
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((n_e, d)) * 0.5
    b = rng.standard_normal(n_e) * 0.05
    G = rng.standard_normal((T, k))
    return x, w, b, k, G, normalize, zc


def pin_backward_finite_differences(orc):
    """dL/dX and dL/dW against central differences of the loss in float64, at a selection whose
    margin is far above the step (normalised and raw gates, with and without the z-loss)."""
    for seed, normalize, zc in ((43, True, 0.0), (47, False, 0.0), (53, True, 0.3), (59, False, 1.0)):
        x, w, b, k, G, normalize, zc = _fd_case(seed, normalize, zc)
        grads = orc.router_backward(x, w, b, k, G, normalize=normalize, zloss_coef=zc)
        assert grads.gap.min() > 1e-4, "pick a seed with a clear selection"
        h = 1e-6
        for arr, got in ((x, grads.dx), (w, grads.dw)):
            num = np.zeros_like(arr)
            for pos in np.ndindex(arr.shape):
                old = arr[pos]
                arr[pos] = old + h
                lp = orc.router_loss(x, w, grads.idx, G, normalize, zc)
                arr[pos] = old - h
                lm = orc.router_loss(x, w, grads.idx, G, normalize, zc)
                arr[pos] = old
                num[pos] = (lp - lm) / (2 * h)
            _close(got, num, rtol=1e-6, atol=1e-8, what=f"finite differences seed {seed}")


def pin_backward_uniform_upstream(orc):
    """Normalised gates sum to 1, so an upstream gradient equal across a token's K slots has zero
    effect; raw gates instead give dL/dz = G * s (1 - s) at the chosen experts."""
    x, w, b, k, G, _, _ = _fd_case(61, True, 0.0)
    Gu = np.repeat(G[:, :1], k, axis=1)
    grads = orc.router_backward(x, w, b, k, Gu, normalize=True)
    _close(grads.dz, np.zeros_like(grads.dz), atol=1e-15, what="normalised, uniform upstream")
    raw = orc.router_backward(x, w, b, k, Gu, normalize=False)
    z = x @ w.T
    for t in range(x.shape[0]):
        for j in range(k):
            i = int(raw.idx[t, j])
            s = 1.0 / (1.0 + math.exp(-z[t, i]))
            _close(raw.dz[t, i], Gu[t, j] * s * (1 - s), rtol=1e-13, what="raw gate derivative")
        others = [i for i in range(w.shape[0]) if i not in raw.idx[t]]
        assert (raw.dz[t, others] == 0).all()


def pin_backward_zloss_rows(orc):
    """The z-loss part alone: each token's row of dL/dz sums to c * 2 lse_t / T (softmax sums to 1)."""
    x, w, b, k, G, _, _ = _fd_case(67, True, 0.0)
    c = 0.7
    grads = orc.router_backward(x, w, b, k, np.zeros_like(G), normalize=True, zloss_coef=c)
    z = x @ w.T
    T = x.shape[0]
    for t in range(T):
        lse = math.log(sum(math.exp(v) for v in z[t]))
        _close(grads.dz[t].sum(), c * 2 * lse / T, rtol=1e-12, what="z-loss row sum")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

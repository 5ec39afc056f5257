"""A seeded random sweep of the bias update against the oracle: expert counts from 1 to 1024
(across the one-wave kernel's lane multiples), load shapes from uniform to a single loaded
expert, no load at all and half the experts dead, every mode, hyperparameters drawn over wide
ranges, random bias and momentum, with and without clearing the counts; 40 draws from a fixed
seed, each checked for b, m, the applied step and both MaxVio forms."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import check_balance, check_maxvio, log, to_dev

pytestmark = pytest.mark.gpu


def draws(n=40, seed=31337):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        n_e = int(rng.choice([1, 2, 3, 7, 64, 65, 255, 256, 257, 512, 1000, 1024]))
        shape = str(rng.choice(["dirichlet", "uniform", "one", "none", "half_dead"]))
        mode = str(rng.choice(["smebu", "sign", "linear"]))
        lam = float(10 ** rng.uniform(-4, np.log10(0.05)))
        beta = float(rng.uniform(0.0, 0.99))
        kappa = float(rng.uniform(0.25, 8.0))
        gamma = float(10 ** rng.uniform(-4, -2))
        clear = bool(rng.random() < 0.5)
        out.append((i, n_e, shape, mode, lam, beta, kappa, gamma, clear))
    return out


def counts_of(rng, n_e, shape):
    total = int(rng.integers(1, 1 << 24))
    if shape == "none":
        return np.zeros(n_e, np.int32)
    if shape == "uniform":
        return np.full(n_e, total // n_e, np.int32)
    if shape == "one":
        c = np.zeros(n_e, np.int32)
        c[int(rng.integers(n_e))] = total
        return c
    c = rng.multinomial(total, rng.dirichlet(np.full(n_e, float(rng.uniform(0.05, 5.0))))).astype(np.int32)
    if shape == "half_dead":
        c[rng.permutation(n_e)[: n_e // 2]] = 0
    return c


@pytest.mark.parametrize("i,n_e,shape,mode,lam,beta,kappa,gamma,clear", draws())
def test_balance_sweep(i, n_e, shape, mode, lam, beta, kappa, gamma, clear):
    log(f"balance sweep {i}: N_r={n_e} loads={shape} mode={mode} lam={lam:.3g} beta={beta:.3g} "
        f"kappa={kappa:.3g} gamma={gamma:.3g} clear={clear}")
    rng = np.random.default_rng(5000 + i)
    c = counts_of(rng, n_e, shape)
    b = (rng.standard_normal(n_e) * 0.05).astype(np.float32)
    m = (rng.standard_normal(n_e) * 1e-3).astype(np.float32)
    cd, bd, md = to_dev(c), to_dev(b), to_dev(m)
    delta, mv = elb.smebu_update(cd, bd, md, mode=mode, lam=lam, beta=beta, kappa=kappa, gamma=gamma,
                                 want_delta=True, clear_counts=clear)
    torch.cuda.synchronize()
    wl = datagen.WORKLOADS["large"].replace(lam=lam, beta=beta, kappa=kappa, gamma=gamma)
    check_balance(mode, c, b, m, bd.cpu().numpy(), md.cpu().numpy(), wl, delta.cpu().numpy())
    check_maxvio(mv.cpu().numpy(), c)
    left = cd.cpu().numpy()
    assert (left == 0).all() if clear else (left == c).all()

"""Golden fixtures: the pages' printed numbers, and the oracle's own tiny-workload outputs."""

import json
import os

import numpy as np

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_workloads_use_the_pages_hyperparameters():
    facts = _load("pages_facts.json")
    hp = facts["smebu_hyperparameters"]
    shape = facts["router_shape"]
    for key, wl in datagen.WORKLOADS.items():
        assert (wl.lam, wl.beta, wl.kappa) == (hp["lambda"], hp["beta"], hp["kappa"]), key
        if key != "tiny":
            assert (wl.n_experts, wl.k) == (shape["n_experts"], shape["k"]), key


def test_overload_violation_from_the_pages():
    fact = _load("pages_facts.json")["overload_violation"]
    for total in fact["batch_tokens"]:
        nbar = total // 4
        counts = np.array([int(fact["load_over_mean"] * nbar), nbar // 2, nbar // 2, nbar])
        assert counts.sum() == total
        assert oracle.normalized_violation(counts)[0] == fact["v"]


def test_maxvio_bands_read_as_ratios():
    bands = _load("pages_facts.json")["maxvio_bands"]
    ratio, _ = oracle.max_violation(np.array([300, 100, 150, 200]))
    assert ratio == bands["ideal_at_most"]
    ratio, _ = oracle.max_violation(np.array([600, 100, 300]))
    assert ratio == bands["late_training_at_most"]


def test_tiny_workload_oracle_fixture():
    g = _load("tiny_oracle.json")
    wl = datagen.WORKLOADS["tiny"]
    assert g["workload"] == wl.label
    x, w = datagen.tokens(wl), datagen.router_weight(wl)
    b, m = datagen.initial_bias(wl), datagen.initial_momentum(wl)
    r = oracle.route(x, w, b, wl.k)
    assert r.idx.tolist() == g["idx"]
    assert np.allclose(r.gates, g["gates"], rtol=1e-13, atol=0)
    n = oracle.expert_loads(r.idx, wl.n_experts)
    assert n.tolist() == g["counts"]
    assert np.allclose(oracle.max_violation(n), g["maxvio"], rtol=1e-15)
    st = oracle.balance_step(n, b, m, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa)
    assert np.allclose(st.bias, g["bias"], rtol=1e-14, atol=0)
    assert np.allclose(st.momentum, g["momentum"], rtol=1e-14, atol=1e-22)

"""The seeded input generator: reproducibility, bf16 rounding, distributions, duplicates."""

import math

import numpy as np
import pytest
import torch

import datagen
from datagen import WORKLOADS


def small(key="large", **kw):
    base = dict(T=3000, d=64)
    base.update(kw)
    return WORKLOADS[key].replace(**base)


def test_reproducible_and_thread_independent():
    wl = small()
    a = datagen.tokens(wl, step=0, threads=1)
    b = datagen.tokens(wl, step=0, threads=4)
    c = datagen.tokens(wl, step=1, threads=4)
    assert a.dtype == np.uint16 and a.shape == (3000, 64)
    assert (a == b).all()
    assert (a != c).any()
    assert (datagen.router_weight(wl) == datagen.router_weight(wl)).all()
    assert (datagen.initial_bias(wl) == datagen.initial_bias(wl)).all()


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    u = x.view(np.uint32).copy()
    u[:1000] = (u[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)  # exact halfway cases
    u[1000:1010] = np.uint32(0x7F7FFFFF)  # rounds up to +inf
    x = u.view(np.float32)
    ours = datagen.to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    back = datagen.bf16_bits_to_f32(ours)
    assert (back == torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()).all()


def test_bias_is_truncated_normal():
    wl = WORKLOADS["large"]
    b = datagen.initial_bias(wl)
    sigma = 0.5 / math.sqrt(wl.d)
    assert b.dtype == np.float32 and b.shape == (256,)
    assert np.all(np.abs(b) <= 2 * sigma)
    # std of N(0, sigma^2) truncated at +-2 sigma is 0.8796 sigma
    assert 0.7 * sigma < b.std() < 1.05 * sigma
    assert (datagen.initial_momentum(wl) == 0).all()


def test_zipf_weights_closed_form():
    for C, p1, plast in ((32, 0.284, 0.0063), (64, 0.250, 0.0026)):
        wl = WORKLOADS["large"].replace(n_clusters=C, d=8)
        _, p = datagen.cluster_model(wl)
        h = sum(c ** -1.1 for c in range(1, C + 1))
        assert abs(p[0] - 1 / h) < 1e-15 and abs(p[-1] - C ** -1.1 / h) < 1e-15
        assert abs(p[0] - p1) < 5e-4 and abs(p[-1] - plast) < 5e-5
        assert abs(p.sum() - 1) < 1e-15


def test_clustered_tokens_sit_near_their_centres():
    wl = small(T=4096, d=256, dtype="f32")
    x = datagen.tokens(wl)
    centres, p = datagen.cluster_model(wl)
    dist = ((x[:, None, :] - centres[None]) ** 2).sum(-1)
    nearest = dist.min(1) / wl.d
    assert abs(np.median(nearest) - 0.25) < 0.02  # within-cluster variance 0.5^2
    share = np.bincount(dist.argmin(1), minlength=len(p)) / len(x)
    assert abs(share[0] - p[0]) < 0.03


def test_duplicates_are_exact_copies():
    wl = WORKLOADS["stress"].replace(T=5000, d=32)
    x = datagen.tokens(wl)
    dst, src = datagen.duplicate_rows(wl)
    assert len(dst) == 250 and len(np.unique(dst)) == 250
    assert not np.isin(src, dst).any()
    assert (x[dst] == x[src]).all()


@pytest.mark.parametrize("key", sorted(WORKLOADS))
def test_recipes(key):
    wl = WORKLOADS[key]
    w = datagen.router_weight(wl)
    assert w.shape == (wl.n_experts, wl.d)
    assert w.dtype == (np.float32 if wl.dtype == "f32" else np.uint16)
    wf = w if wl.dtype == "f32" else datagen.bf16_bits_to_f32(w)
    assert abs(wf.std() - 0.02) < 0.002
    assert wl.k <= wl.n_experts <= 256 and wl.d % 64 == 0

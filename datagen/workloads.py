"""Workload recipes and their seeded generators.

Shapes follow the router of Arcee Trinity Large: 256 routed experts, four chosen per
token (Arcee Trinity Large Technical Report, section 2.3 "Mixture-of-Experts"; the
hotdry blog post on Trinity Large MoE routing, section on sigmoid routing and Top-K).
The pages publish no dataset for the router, so every token batch is synthetic:

* isotropic tokens: every coordinate iid N(0, 1);
* clustered tokens: a fixed set of cluster centres (coordinates iid N(0, 1)), cluster
  popularity p_c proportional to c^-s for c = 1..C (Zipf), and token = centre + 0.5 * N(0, 1)
  noise, so that expert loads are skewed the way a real corpus skews them;
* optional exact duplicates: a seeded fraction of rows overwritten with copies of other
  rows, so identical tokens must receive identical routing wherever they sit in the batch.

Router weights are N(0, 0.02^2).  The expert bias starts from a zero-mean normal with
sigma = 0.5 / sqrt(d) truncated at +-2 sigma by resampling (initialisation advice in the
hotdry blog post, section on production parameters); the momentum buffer starts at 0.

Every random draw comes from numpy's PCG64 seeded through a SeedSequence whose spawn key
names the stream (weights, bias, clusters, duplicates, token chunk), so any piece can be
regenerated on its own and chunks can be drawn in parallel threads.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Spawn-key streams.
_S_WEIGHT, _S_BIAS, _S_CLUSTERS, _S_DUPS, _S_TOKENS = 0, 1, 2, 3, 4
TOKEN_CHUNK = 4096  # rows per independently seeded token chunk


@dataclasses.dataclass(frozen=True)
class Workload:
    """One router workload.  Field names follow the pages' notation where they have one."""

    key: str
    T: int  # tokens per step
    d: int  # hidden size
    n_experts: int  # N_r, routed experts
    k: int  # experts chosen per token
    dtype: str  # "f32" or "bf16": storage type of hidden states and router weights
    token_kind: str = "iid"  # "iid" or "clusters"
    n_clusters: int = 0
    zipf_s: float = 1.1
    cluster_sigma: float = 0.5
    dup_frac: float = 0.0
    w_sigma: float = 0.02
    seed: int = 0
    mode: str = "smebu"  # balance update: "smebu", "sign" or "linear"
    lam: float = 5e-4  # lambda, SMEBU / linear step size
    beta: float = 0.5  # momentum factor
    kappa: float = 2.0  # tanh soft-clamp slope
    gamma: float = 1e-3  # sign-step size
    steps: int = 1  # consecutive routed steps (closed loop when > 1)
    dispatch: bool = False  # whether the step also builds the dispatch permutation
    normalize_gates: bool = True

    @property
    def label(self) -> str:
        parts = [self.mode, self.dtype, f"T{self.T}", f"d{self.d}", f"E{self.n_experts}", f"K{self.k}"]
        if self.token_kind == "clusters":
            parts.append(f"zipf{self.n_clusters}")
        if self.dup_frac:
            parts.append(f"dup{int(round(self.dup_frac * 100))}pct")
        if self.steps > 1:
            parts.append(f"{self.steps}steps")
        return "-".join(parts)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: dict[str, Workload] = {
    # Tiny single step in fp32: one forward, one SMEBU update.
    "tiny": Workload("tiny", T=512, d=256, n_experts=16, k=2, dtype="f32", seed=1001),
    # Nano/Mini-style: isotropic bf16 tokens, sign-step balancing.
    "sign": Workload("sign", T=16384, d=2048, n_experts=256, k=4, dtype="bf16", seed=1002,
                     mode="sign", gamma=1e-3),
    # Large-style single step: one GPU's micro-batch share, 32 Zipf clusters, dispatch.
    "large": Workload("large", T=65536, d=3072, n_experts=256, k=4, dtype="bf16", seed=1003,
                      token_kind="clusters", n_clusters=32, dispatch=True),
    # Closed loop: 300 steps, fixed router weights, fresh clustered tokens each step.
    "loop": Workload("loop", T=32768, d=3072, n_experts=256, k=4, dtype="bf16", seed=1004,
                     token_kind="clusters", n_clusters=32, steps=300),
    # Large-batch stress: 64 clusters plus 5% exact duplicate rows, full path with dispatch.
    "stress": Workload("stress", T=262144, d=4096, n_experts=256, k=4, dtype="bf16", seed=1005,
                       token_kind="clusters", n_clusters=64, dup_frac=0.05, dispatch=True),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=key)))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- bf16 storage ---------

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even; returns the raw 16-bit patterns (uint16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ---------------------------------------------------------------- parameters -----------

def router_weight(wl: Workload) -> np.ndarray:
    """Router weight rows e_i, shape [N_r, d]: fp32 values, or bf16 bit patterns."""
    rng = _rng(wl.seed, _S_WEIGHT)
    w = rng.standard_normal((wl.n_experts, wl.d), dtype=np.float32) * np.float32(wl.w_sigma)
    return _store(w, wl.dtype)


def initial_bias(wl: Workload) -> np.ndarray:
    """Expert bias b at step 0: N(0, (0.5/sqrt(d))^2) truncated at +-2 sigma by resampling."""
    rng = _rng(wl.seed, _S_BIAS)
    sigma = 0.5 / np.sqrt(wl.d)
    b = rng.standard_normal(wl.n_experts) * sigma
    bad = np.abs(b) > 2.0 * sigma
    while bad.any():
        b[bad] = rng.standard_normal(int(bad.sum())) * sigma
        bad = np.abs(b) > 2.0 * sigma
    return b.astype(np.float32)


def initial_momentum(wl: Workload) -> np.ndarray:
    return np.zeros(wl.n_experts, dtype=np.float32)


def cluster_model(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Cluster centres [C, d] (fp32) and Zipf popularity weights [C] (fp64, sums to 1)."""
    rng = _rng(wl.seed, _S_CLUSTERS)
    centres = rng.standard_normal((wl.n_clusters, wl.d), dtype=np.float32)
    ranks = np.arange(1, wl.n_clusters + 1, dtype=np.float64)
    p = ranks ** (-wl.zipf_s)
    return centres, p / p.sum()


def duplicate_rows(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """(dst, src): rows dst[j] are exact copies of rows src[j]; no src row is itself a dst."""
    n_dup = int(round(wl.dup_frac * wl.T))
    if n_dup == 0:
        z = np.zeros(0, dtype=np.int64)
        return z, z
    rng = _rng(wl.seed, _S_DUPS)
    dst = np.sort(rng.choice(wl.T, size=n_dup, replace=False))
    keep = np.setdiff1d(np.arange(wl.T), dst)
    src = rng.choice(keep, size=n_dup, replace=True)
    return dst.astype(np.int64), src.astype(np.int64)


# ---------------------------------------------------------------- tokens ---------------

def tokens(wl: Workload, step: int = 0, threads: int | None = None) -> np.ndarray:
    """Hidden states u_t for one step, shape [T, d]: fp32 values, or bf16 bit patterns.

    Rows are drawn in chunks of TOKEN_CHUNK, each from its own seeded stream (step, chunk),
    in parallel threads; the result does not depend on the thread count.
    """
    out_dtype = np.float32 if wl.dtype == "f32" else np.uint16
    out = np.empty((wl.T, wl.d), dtype=out_dtype)
    model = cluster_model(wl) if wl.token_kind == "clusters" else None
    n_chunks = (wl.T + TOKEN_CHUNK - 1) // TOKEN_CHUNK

    def fill(j: int) -> None:
        lo, hi = j * TOKEN_CHUNK, min(wl.T, (j + 1) * TOKEN_CHUNK)
        rng = _rng(wl.seed, _S_TOKENS, step, j)
        if model is None:
            x = rng.standard_normal((hi - lo, wl.d), dtype=np.float32)
        else:
            centres, p = model
            c = rng.choice(len(p), size=hi - lo, p=p)
            x = rng.standard_normal((hi - lo, wl.d), dtype=np.float32)
            x *= np.float32(wl.cluster_sigma)
            x += centres[c]
        out[lo:hi] = _store(x, wl.dtype)

    n_thr = threads or _threads()
    if n_thr <= 1 or n_chunks == 1:
        for j in range(n_chunks):
            fill(j)
    else:
        with ThreadPoolExecutor(max_workers=n_thr) as ex:
            list(ex.map(fill, range(n_chunks)))
    dst, src = duplicate_rows(wl)
    if len(dst):
        out[dst] = out[src]
    return out

"""Expert loads, MaxVio and the counting-sort dispatch permutation (exact integers).

TEST INFRASTRUCTURE (see the package docstring).

Definitions followed
  * load n_i: tokens routed to expert i this step; mean load nbar = N_r^-1 sum_j n_j
    ("SMEBU Load Balancing", "How it works", the line before eq. (20));
  * MaxVio: the talk defines it as the ratio of the load of the most-routed expert to the
    load of the least-routed one, with <= 3 ideal and > 6 dangerous ("Arcee Halts 400B
    Blackwell Model Collapse With Dynamic Router Biases", section "The MaxVio Metric and
    the Day-4 Crisis").  We also report the relative excess (max n - nbar) / nbar used
    by the aux-loss-free balancing literature the study note builds on; that form is
    not written on the pages;
  * dispatch: the pages define no dispatch; we take the plain counting sort of the
    flattened (token, slot) assignments by expert, stable in flat position t*K + k:
    offsets = [0, cumsum(n)], perm lists flat positions bucket by bucket, inv is its
    inverse.
"""

from __future__ import annotations

import numpy as np


def expert_loads(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """n_i = number of (token, slot) pairs routed to expert i (int64 [N_r])."""
    return np.bincount(np.asarray(idx).ravel(), minlength=n_experts).astype(np.int64)


def max_violation(counts: np.ndarray) -> tuple[float, float]:
    """(max n / min n, (max n - nbar) / nbar).  min n = 0 gives +inf; all-zero loads give NaN."""
    n = np.asarray(counts, dtype=np.int64)
    total = int(n.sum())
    if total == 0:
        return float("nan"), float("nan")
    nmax, nmin = int(n.max()), int(n.min())
    ratio = float("inf") if nmin == 0 else nmax / nmin
    nbar = total / len(n)
    return ratio, (nmax - nbar) / nbar


def dispatch_permutation(idx: np.ndarray, n_experts: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Stable counting sort of flat assignments by expert.

    Returns offsets [N_r + 1] (bucket e is perm[offsets[e]:offsets[e+1]]), perm [T*K]
    (flat positions t*K + k, ascending within each bucket) and inv [T*K] with
    perm[inv[j]] = j.
    """
    flat = np.asarray(idx).ravel()
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm), dtype=np.int64)
    return offsets, perm, inv

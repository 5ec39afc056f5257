"""Expert-side data movement around the router: permute to expert-contiguous rows, and the
gated combine back to token order (float64 where arithmetic happens).

TEST INFRASTRUCTURE (see the package docstring).

What is computed
  * The routed experts' outputs are weighted by the gating scores and summed per token
    (Arcee Trinity Large Technical Report, section 2.3 "Mixture-of-Experts": the gating
    scores multiply the routed experts' outputs; the shared expert is added separately and
    is outside this library).  For token t with chosen experts idx[t, 0..K-1] and gates
    g[t, 0..K-1]:  y_t = sum_j g[t, j] * E_{idx[t, j]}(u_t).
  * Between the two, every expert sees its tokens as one contiguous block.  The pages fix
    no layout; the reading here is the dispatch permutation of loads.dispatch_permutation:
    row p of the expert-contiguous buffer is the token of flat assignment perm[p]
    (token perm[p] // K), and inv[t * K + j] is where assignment (t, j) sits.
"""

from __future__ import annotations

import numpy as np

from .router import widen


def permute_rows(x: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """xp[p] = x[perm[p] // k]: the expert-contiguous copy of the token rows (exact copy,
    same dtype and bit patterns as x)."""
    x = np.asarray(x)
    perm = np.asarray(perm, dtype=np.int64)
    return x[perm // k]


def combine(expert_out: np.ndarray, gates: np.ndarray, inv: np.ndarray, k: int) -> np.ndarray:
    """y[t] = sum_j gates[t, j] * expert_out[inv[t * k + j]], summed over j = 0 .. k-1 in that
    order, in float64 on the exact input values (bf16 as uint16 bit patterns, or fp32)."""
    eo = widen(np.asarray(expert_out))
    g = np.asarray(gates, dtype=np.float64)
    rows = np.asarray(inv, dtype=np.int64).reshape(g.shape[0], k)
    y = np.zeros((g.shape[0], eo.shape[1]))
    for j in range(k):
        y += g[:, j:j + 1] * eo[rows[:, j]]
    return y

"""Router z-loss on the logits (float64).

TEST INFRASTRUCTURE (see the package docstring).

The talk's stabilisation table writes the z-loss as L_z = log^2 sum_i e^{x_i} over the
router logits ("Arcee Halts 400B Blackwell Model Collapse With Dynamic Router Biases",
section "Precision Fallbacks, Loss Stabilization, and MaxVio as Data Telemetry"); the
report summary gives its weight, 1e-4 intended and 1e-6 in effect mid-training (Arcee
Trinity Large Technical Report, section 6 "Discussion").  Reading: per token t,
lse_t = log sum_i exp(z_{t,i}) over all N_r routed experts, and the loss is the mean of
lse_t^2 over the tokens of the batch; the weight is applied by the caller.
"""

from __future__ import annotations

import numpy as np


def router_z_loss(z: np.ndarray) -> tuple[float, np.ndarray]:
    """(mean_t lse_t^2, lse [T]).  lse is evaluated as max + log sum exp(z - max)."""
    z = np.asarray(z, dtype=np.float64)
    if z.shape[0] == 0:
        return 0.0, np.zeros(0)
    zmax = z.max(axis=1, keepdims=True)
    lse = (zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True)))[:, 0]
    return float(np.mean(lse * lse)), lse


def z_loss_from_lse(lse: np.ndarray) -> float:
    """mean_t lse_t^2 from per-token log-sum-exps (the same reading as router_z_loss)."""
    lse = np.asarray(lse, dtype=np.float64)
    return float(np.mean(lse * lse)) if lse.size else 0.0

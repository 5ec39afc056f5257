"""Expert-bias updates: SMEBU, the Nano/Mini sign step, and the linear unclamped step.

TEST INFRASTRUCTURE (see the package docstring).  Float64 throughout.

SMEBU ("SMEBU Load Balancing", "How it works", eq. (23)-(28); Arcee Trinity Large
Technical Report, section 2.3), applied once per optimizer step to that step's loads:
    v_i   = (nbar - n_i) / nbar                      (23)
    vt_i  = tanh(kappa * v_i)                        (24)
    db_i  = lambda * vt_i                            (25)
    db_i <- db_i - mean_j db_j                       (26)  re-centred before momentum
    m_i  <- beta * m_i + (1 - beta) * db_i           (27)
    b_i  <- b_i + m_i                                (28)
Trinity Large used lambda = 5e-4, beta = 0.5, kappa = 2.

Sign step of Trinity Nano/Mini (same note, eq. (20)-(22); report section 2.3):
    db_i = gamma * sign(nbar - n_i),  then b is re-centred.
Reading: the re-centre applies to the updated bias, b <- (b + db) - mean(b + db); the
note calls it the re-centre "of b itself", and re-centring the old b would let mean(b)
drift by mean(db).  sign(0) = 0.  The momentum buffer is untouched in this mode.

Linear unclamped step (same note, last paragraph of "How it works"; report section 2.3):
db_i proportional to v_i.  Reading: only the clamp changes, vt_i = v_i, and steps (25)-(28)
stay as they are.

With no routed tokens at all (nbar = 0) the violation is undefined; the step then leaves
b and m unchanged (our reading; the pages never meet this case).
"""

from __future__ import annotations

import dataclasses

import numpy as np

MODES = ("smebu", "sign", "linear")


def normalized_violation(counts: np.ndarray) -> np.ndarray:
    """v_i = (nbar - n_i) / nbar with nbar = sum_j n_j / N_r   (eq. (23))."""
    n = np.asarray(counts, dtype=np.float64)
    nbar = n.sum() / len(n)
    return (nbar - n) / nbar


@dataclasses.dataclass
class BalanceStep:
    bias: np.ndarray  # b after the step
    momentum: np.ndarray  # m after the step
    delta_b: np.ndarray  # the applied step: re-centred db (smebu/linear), gamma*sign (sign)
    delta_b_raw: np.ndarray  # db before re-centring (smebu/linear), gamma*sign (sign)


def balance_step(counts: np.ndarray, bias: np.ndarray, momentum: np.ndarray, *, mode: str = "smebu",
                 lam: float = 5e-4, beta: float = 0.5, kappa: float = 2.0,
                 gamma: float = 1e-3) -> BalanceStep:
    """One bias update from this step's expert loads n (eq. (20)-(28), see module doc)."""
    if mode not in MODES:
        raise ValueError(f"unknown balance mode {mode!r}")
    n = np.asarray(counts, dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64)
    m = np.asarray(momentum, dtype=np.float64)
    if n.sum() == 0:
        z = np.zeros_like(b)
        return BalanceStep(b.copy(), m.copy(), z, z.copy())
    nbar = n.sum() / len(n)
    if mode == "sign":
        db = gamma * np.sign(nbar - n)
        b_new = b + db
        b_new = b_new - b_new.mean()
        return BalanceStep(b_new, m.copy(), db, db.copy())
    v = (nbar - n) / nbar
    vt = np.tanh(kappa * v) if mode == "smebu" else v
    db_raw = lam * vt
    db = db_raw - db_raw.mean()
    m_new = beta * m + (1.0 - beta) * db
    b_new = b + m_new
    return BalanceStep(b_new, m_new, db, db_raw)


def balance_layers(counts: np.ndarray, bias: np.ndarray, momentum: np.ndarray, **params) -> list[BalanceStep]:
    """One update per MoE layer, each from its own layer's loads: every layer carries its own
    b and m, and no equation on the pages couples layers ("SMEBU Load Balancing", "How it
    works": the update is stated per router).  counts, bias, momentum are [L, N_r]."""
    return [balance_step(counts[l], bias[l], momentum[l], **params) for l in range(len(counts))]

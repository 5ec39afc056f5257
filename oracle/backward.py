"""Router backward: gradients of a loss through the gates and the z-loss (float64).

TEST INFRASTRUCTURE (see the package docstring).

The pages give no backward formula; this is the chain rule applied to the forward of
router.py, with the selection held fixed (Top-K is piecewise constant: the bias b, used only
inside Top-K, receives no gradient, in line with the bias being a non-learned buffer moved by
the balancer in "SMEBU Load Balancing", "How it works").

Loss whose gradient is taken, for upstream gate gradients G [T, K] and a z-loss weight c:
    L = sum_{t, j} G[t, j] * g[t, j]  +  c * mean_t lse_t^2
with g the gates of router.route (normalised over the K chosen, or raw) and lse_t the
log-sum-exp of token t's logits (zloss.py).  Then, for token t, chosen experts i_j with
scores s_j = sigmoid(z_{t, i_j}) and S = sum_j s_j:
    normalised gates: dL/ds_j = (G_j - sum_m G_m g_m) / S      (g_j = s_j / S)
    raw gates:        dL/ds_j = G_j
    dL/dz_{t, i_j}  = dL/ds_j * s_j * (1 - s_j)                 (d sigmoid / dz)
    every expert i:  dL/dz_{t, i} += c * (2 / T) * lse_t * softmax(z_t)_i
and, with z = X W^T:  dL/dX = dZ W,  dL/dW = dZ^T X.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .router import select_topk, sigmoid_scores, widen


@dataclasses.dataclass
class RouterGrads:
    dz: np.ndarray   # [T, N_r] dL/dz
    dx: np.ndarray   # [T, d]   dL/dX
    dw: np.ndarray   # [N_r, d] dL/dW
    idx: np.ndarray  # [T, K] the selection the gradient was taken at
    gap: np.ndarray  # [T] its decision margin


def logit_grads(z: np.ndarray, idx: np.ndarray, dgates: np.ndarray, normalize: bool = True,
                zloss_coef: float = 0.0) -> np.ndarray:
    """dL/dz [T, N_r] from the logits z, the selection idx and the upstream gate gradients."""
    z = np.asarray(z, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    G = np.asarray(dgates, dtype=np.float64)
    T = z.shape[0]
    rows = np.arange(T)[:, None]
    s = sigmoid_scores(z)
    sel = s[rows, idx]
    if normalize:
        S = sel.sum(axis=1, keepdims=True)
        g = sel / S
        ds = (G - (G * g).sum(axis=1, keepdims=True)) / S
    else:
        ds = G
    dz = np.zeros_like(z)
    dz[rows, idx] = ds * sel * (1.0 - sel)
    if zloss_coef != 0.0 and T > 0:
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        lse = zmax + np.log(e.sum(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dz += zloss_coef * (2.0 / T) * lse * p
    return dz


def router_backward(x: np.ndarray, w: np.ndarray, bias: np.ndarray, k: int, dgates: np.ndarray,
                    normalize: bool = True, zloss_coef: float = 0.0) -> RouterGrads:
    """Gradients of L (module docstring) with respect to the logits, X and W."""
    x64, w64 = widen(x), widen(w)
    z = x64 @ w64.T
    q = sigmoid_scores(z) + np.asarray(bias, dtype=np.float64)[None, :]
    idx, gap = select_topk(q, k)
    dz = logit_grads(z, idx, dgates, normalize, zloss_coef)
    return RouterGrads(dz=dz, dx=dz @ w64, dw=dz.T @ x64, idx=idx, gap=gap)


def router_loss(x: np.ndarray, w: np.ndarray, idx: np.ndarray, dgates: np.ndarray, normalize: bool = True,
                zloss_coef: float = 0.0) -> float:
    """L itself (module docstring) at a given selection: the function the gradients differentiate."""
    z = widen(x) @ widen(w).T
    s = sigmoid_scores(z)
    sel = s[np.arange(z.shape[0])[:, None], np.asarray(idx, dtype=np.int64)]
    g = sel / sel.sum(axis=1, keepdims=True) if normalize else sel
    loss = float((np.asarray(dgates, dtype=np.float64) * g).sum())
    if zloss_coef != 0.0 and z.shape[0] > 0:
        zmax = z.max(axis=1, keepdims=True)
        lse = (zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True)))[:, 0]
        loss += zloss_coef * float(np.mean(lse * lse))
    return loss

"""Router forward: logits, sigmoid scores, biased Top-K selection and gates (float64).

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and the
benchmark's CPU baseline use this module.

Definitions followed
  * logit z_{i,t} = u_t^T e_i, one per token and routed expert; the router linear has no
    bias term ("no biases on linear layers": Arcee Trinity Large Technical Report,
    section 2 "Architecture"; dot product u_t^T e_i: hotdry blog post, section on
    sigmoid routing and Top-K selection);
  * score s_{i,t} = sigmoid(z_{i,t}), independent per expert, not normalised across
    experts (same blog section; Technical Report section 2.3 "Mixture-of-Experts");
  * selection: the K experts with the largest s_{i,t} + b_i; the bias is added after
    the sigmoid and only inside Top-K ("SMEBU Load Balancing", "How it works",
    eq. (17); Technical Report section 2.3);
  * gates: from s_{i,t} only, never from b ("SMEBU Load Balancing", "How it works";
    Technical Report section 2.3 "normalized scores").

Readings where the pages leave a step open:
  * the hotdry blog places the bias before the sigmoid; the study note and the report
    summary place it on the score used by Top-K.  We add it after the sigmoid;
  * "normalized scores": by default gates are the selected scores divided by their sum
    over the K chosen experts; ``normalize=False`` returns the raw scores;
  * ties in s + b: the lower expert index wins, and the K outputs are listed in
    descending s + b (stable order on (-q, i)).
"""

from __future__ import annotations

import dataclasses

import numpy as np


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of stored inputs: fp32 arrays as they are, uint16 as bf16 bits."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported input dtype {a.dtype}")


def router_logits(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """z[t, i] = sum_k x[t, k] * w[i, k]  (u_t^T e_i), float64 matrix product."""
    return widen(x) @ widen(w).T


def sigmoid_scores(z: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-z)), elementwise."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def select_topk(q: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """The K largest entries of each row of q, in descending order, ties to the lower index.

    Returns (idx [T, K] int64, gap [T]) where gap is q at the K-th choice minus q at the
    (K+1)-th in that order (+inf when every expert is chosen): the margin by which the
    selection is decided.
    """
    order = np.argsort(-q, axis=1, kind="stable")
    idx = order[:, :k]
    rows = np.arange(q.shape[0])
    if k < q.shape[1]:
        gap = q[rows, order[:, k - 1]] - q[rows, order[:, k]]
    else:
        gap = np.full(q.shape[0], np.inf)
    return idx, gap


def gate_values(s: np.ndarray, idx: np.ndarray, normalize: bool = True) -> np.ndarray:
    """Gates of the chosen experts from the scores alone: s / sum over the K chosen, or s."""
    sel = np.take_along_axis(s, idx, axis=1)
    if normalize:
        return sel / sel.sum(axis=1, keepdims=True)
    return sel


@dataclasses.dataclass
class Route:
    idx: np.ndarray  # [T, K] int64 chosen experts, descending s + b
    gates: np.ndarray  # [T, K] float64
    gap: np.ndarray  # [T] float64 decision margin (see select_topk)
    logits: np.ndarray | None = None  # [T, N_r] float64 when requested
    scores: np.ndarray | None = None  # [T, N_r] float64 when requested


def route(x: np.ndarray, w: np.ndarray, bias: np.ndarray, k: int, *, normalize: bool = True,
          keep: bool = False, chunk: int = 8192) -> Route:
    """Route every token of x: logits -> sigmoid -> Top-K on s + b -> gates from s.

    x: [T, d] fp32 values or bf16 bits; w: [N_r, d] likewise; bias: [N_r].  Tokens are
    processed in row chunks only to bound memory; each row is independent.
    """
    T = x.shape[0]
    b = np.asarray(bias, dtype=np.float64)
    w64 = widen(w)
    idx = np.empty((T, k), dtype=np.int64)
    gates = np.empty((T, k), dtype=np.float64)
    gap = np.empty(T, dtype=np.float64)
    zs = [] if keep else None
    ss = [] if keep else None
    for lo in range(0, T, chunk):
        hi = min(T, lo + chunk)
        z = widen(x[lo:hi]) @ w64.T
        s = sigmoid_scores(z)
        q = s + b[None, :]
        i, g = select_topk(q, k)
        idx[lo:hi] = i
        gap[lo:hi] = g
        gates[lo:hi] = gate_values(s, i, normalize)
        if keep:
            zs.append(z)
            ss.append(s)
    if keep:
        return Route(idx, gates, gap, np.concatenate(zs) if zs else np.zeros((0, len(b))),
                     np.concatenate(ss) if ss else np.zeros((0, len(b))))
    return Route(idx, gates, gap)

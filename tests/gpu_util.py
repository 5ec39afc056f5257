"""Helpers for the GPU parity tests: moving seeded inputs to the device and comparing the
library's outputs with the oracle's under the parity protocol.

Protocol (tolerances stated once, here):
  * expert indices: bit-exact for every token whose oracle decision margin (the gap between
    the K-th and (K+1)-th s + b, fp64) is at least TIE_GAP; tokens below it are counted and
    reported as ties.  Inside the chosen K, an order swap between two experts is excused only
    when their oracle s + b differ by less than order_tol(b), the resolution of the GPU's
    comparison: the MFMA kernel's selection codes resolve 2^(E-22) per code, where 2^E <= 1 +
    max b - min b < 2^(E+1) (two codes of one rounding each: 2^(E-21)); the generic kernel
    compares s + b rounded to fp32 (two roundings of at most half an ulp); the fp32 logit of a
    d-term bf16 product and the fp32 sigmoid add ORDER_TOL_FP32.  Such swaps are counted;
  * gates and logits: |gpu - oracle| <= RTOL |oracle| + ATOL, gates evaluated by the oracle
    at the GPU's own selection;
  * counts, offsets, perm, inv: bit-exact against the oracle run on the GPU's indices;
  * b and m: |gpu - oracle| <= 1e-6 per step, the oracle fed the GPU's counts and the GPU's
    previous b and m.
"""

from __future__ import annotations

import dataclasses
import math
import sys

import numpy as np
import torch

import oracle

TIE_GAP = 1e-3
ORDER_TOL_FP32 = 2e-5
RTOL = 2e-2
ATOL = 1e-6
BM_TOL = 1e-6


def order_tol(bias: np.ndarray) -> float:
    """The largest s + b difference the GPU may order either way for this bias (see above)."""
    b = np.asarray(bias, dtype=np.float64)
    E = math.floor(math.log2(1.0 + float(b.max() - b.min())))
    codes = 2.0 ** (E - 21)
    fp32 = float(np.spacing(np.float32(np.abs(b).max() + 1.0)))
    return max(codes, fp32) + ORDER_TOL_FP32


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclasses.dataclass
class RouteCheck:
    n_tokens: int
    ties: int  # tokens whose decision margin is below TIE_GAP
    tie_mismatch: int  # of those, how many the GPU resolved differently
    order_ties: int  # order swaps inside the selection between experts closer than ORDER_TOL
    max_gate_rel: float
    max_swap_gap: float = 0.0  # largest oracle s + b difference among the excused order swaps
    min_decided_gap: float = float("inf")  # smallest margin among the decided tokens

    def merge(self, o: "RouteCheck") -> "RouteCheck":
        return RouteCheck(self.n_tokens + o.n_tokens, self.ties + o.ties, self.tie_mismatch + o.tie_mismatch,
                          self.order_ties + o.order_ties, max(self.max_gate_rel, o.max_gate_rel),
                          max(self.max_swap_gap, o.max_swap_gap), min(self.min_decided_gap, o.min_decided_gap))

    def __str__(self) -> str:
        return (f"{self.n_tokens} tokens: ties={self.ties} (resolved differently {self.tie_mismatch}), "
                f"order swaps={self.order_ties} (largest gap {self.max_swap_gap:.2e}), smallest decided margin "
                f"{self.min_decided_gap:.2e}, gate rel err {self.max_gate_rel:.2e}")


def _compare_chunk(idx_gpu, gates_gpu, x, w, bias, k, rows, normalize) -> RouteCheck:
    r = oracle.route(x[rows], w, bias, k, normalize=normalize, keep=True)
    g_idx = idx_gpu[rows].astype(np.int64)
    q = r.scores + np.asarray(bias, dtype=np.float64)[None, :]
    ties = r.gap < TIE_GAP
    same_set = np.sort(g_idx, axis=1) == np.sort(r.idx, axis=1)
    bad_set = ~same_set.all(axis=1) & ~ties
    assert not bad_set.any(), (
        f"{int(bad_set.sum())} decided tokens chose a different expert set, e.g. row {rows[np.argmax(bad_set)]}: "
        f"gpu {g_idx[np.argmax(bad_set)]} oracle {r.idx[np.argmax(bad_set)]}")
    # Order inside the selection: descending oracle q, swaps only between experts closer than order_tol.
    qsel = np.take_along_axis(q, g_idx, axis=1)
    order_exact = (g_idx == r.idx).all(axis=1)
    if k > 1:
        worst = np.maximum(qsel[:, 1:] - qsel[:, :-1], 0.0).max(axis=1)  # largest inversion per token
    else:
        worst = np.zeros(len(rows))
    order_ok = worst < order_tol(bias)
    bad_order = ~order_exact & ~order_ok & ~ties
    assert not bad_order.any(), (
        f"{int(bad_order.sum())} tokens list their experts out of order, e.g. row {rows[np.argmax(bad_order)]} "
        f"(inversion {worst[np.argmax(bad_order)]:.3g})")
    swaps = ~order_exact & order_ok & ~ties
    # Gates at the GPU's own selection.
    want = oracle.gate_values(r.scores, g_idx, normalize)
    got = gates_gpu[rows].astype(np.float64)
    err = np.abs(got - want)
    assert (err <= RTOL * np.abs(want) + ATOL).all(), f"gate error {err.max()}"
    rel = float((err / np.maximum(np.abs(want), 1e-30)).max()) if len(rows) else 0.0
    decided = r.gap[~ties]
    return RouteCheck(len(rows), int(ties.sum()), int((~same_set.all(axis=1) & ties).sum()), int(swaps.sum()), rel,
                      float(worst[swaps].max()) if swaps.any() else 0.0,
                      float(decided.min()) if len(decided) else float("inf"))


def compare_route(idx_gpu: np.ndarray, gates_gpu: np.ndarray, x: np.ndarray, w: np.ndarray, bias: np.ndarray,
                  k: int, rows: np.ndarray | None = None, normalize: bool = True,
                  chunk: int = 16384) -> RouteCheck:
    """Check GPU routing of tokens `rows` (every token when None) against the oracle, in chunks of
    rows; raises on failure."""
    if rows is None:
        rows = np.arange(x.shape[0])
    rep = RouteCheck(0, 0, 0, 0, 0.0)
    for lo in range(0, len(rows), chunk):
        rep = rep.merge(_compare_chunk(idx_gpu, gates_gpu, x, w, bias, k, rows[lo:lo + chunk], normalize))
    return rep


def compare_logits(logits_gpu: np.ndarray, x: np.ndarray, w: np.ndarray, rows: np.ndarray | None = None) -> float:
    if rows is None:
        rows = np.arange(x.shape[0])
    z = oracle.router_logits(x[rows], w)
    got = logits_gpu[rows].astype(np.float64)
    err = np.abs(got - z)
    assert (err <= RTOL * np.abs(z) + 1e-4).all(), f"logit error {err.max()}"
    return float(err.max())


def check_counts(counts_gpu: np.ndarray, idx_gpu: np.ndarray, n_experts: int) -> np.ndarray:
    want = oracle.expert_loads(idx_gpu, n_experts)
    assert (counts_gpu.astype(np.int64) == want).all(), "counts differ from the oracle's count of the GPU indices"
    return want


def check_balance(mode: str, counts: np.ndarray, b_prev: np.ndarray, m_prev: np.ndarray, b_gpu: np.ndarray,
                  m_gpu: np.ndarray, wl, delta_gpu: np.ndarray | None = None) -> float:
    st = oracle.balance_step(counts, b_prev, m_prev, mode=mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa,
                             gamma=wl.gamma)
    eb = np.abs(b_gpu.astype(np.float64) - st.bias).max()
    em = np.abs(m_gpu.astype(np.float64) - st.momentum).max()
    assert eb <= BM_TOL and em <= BM_TOL, f"{mode}: |db| {eb:.3g} |dm| {em:.3g}"
    if delta_gpu is not None:
        ed = np.abs(delta_gpu.astype(np.float64) - st.delta_b).max()
        assert ed <= BM_TOL, f"{mode}: |d delta_b| {ed:.3g}"
    return float(max(eb, em))


def check_maxvio(mv_gpu: np.ndarray, counts: np.ndarray) -> None:
    ratio, rel = oracle.max_violation(counts)
    for got, want in ((mv_gpu[0], ratio), (mv_gpu[1], rel)):
        if np.isnan(want):
            assert np.isnan(got)
        elif np.isinf(want):
            assert np.isinf(got) and got > 0
        else:
            assert abs(got - want) <= 1e-6 * abs(want) + 1e-7, (got, want)


def check_dispatch(offsets: np.ndarray, perm: np.ndarray, inv: np.ndarray | None, idx_gpu: np.ndarray,
                   n_experts: int) -> None:
    o, p, i = oracle.dispatch_permutation(idx_gpu, n_experts)
    assert (offsets.astype(np.int64) == o).all(), "offsets differ"
    assert (perm.astype(np.int64) == p).all(), "perm differs"
    if inv is not None:
        assert (inv.astype(np.int64) == i).all(), "inv differs"


def sample_rows(T: int, n: int, seed: int, extra=()) -> np.ndarray:
    """A seeded sample of n token rows plus the first, last, ragged-tail and any extra rows."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows.update([0, T - 1] + list(range(max(0, T - 37), T)))
    rows.update(int(r) for r in extra)
    return np.array(sorted(rows), dtype=np.int64)


def check_dispatch_device(offs: torch.Tensor, perm: torch.Tensor, inv: torch.Tensor, flat: torch.Tensor,
                          n_experts: int, chunk: int = 1 << 27) -> None:
    """The stable counting sort of the flat ids `flat` checked on the device, in chunks, for sizes
    the host cannot sort: bucket sizes = id histogram, perm[inv] = identity, ids non-decreasing
    along perm, flat positions ascending inside a bucket.  Together these leave exactly one perm."""
    n = flat.numel()
    hist = torch.zeros(n_experts, dtype=torch.int64, device=flat.device)
    for lo in range(0, n, chunk):
        hist += torch.bincount(flat[lo:lo + chunk].long(), minlength=n_experts)
    o = offs.long()
    assert o[0].item() == 0 and o[-1].item() == n
    assert torch.equal(o[1:] - o[:-1], hist), "bucket sizes differ from the id histogram"
    for lo in range(0, n, chunk):
        hi = min(lo + chunk, n)
        back = perm[inv[lo:hi].long()].long()
        assert torch.equal(back, torch.arange(lo, hi, device=flat.device)), f"perm[inv] differs near {lo}"
    for lo in range(0, n, chunk):  # each chunk together with the first entry of the next
        p = perm[lo:min(lo + chunk + 1, n)].long()
        e = flat[p]
        de = e[1:] - e[:-1]
        assert bool((de >= 0).all()), f"ids decrease along perm near {lo}"
        same = de == 0
        assert bool((p[1:][same] > p[:-1][same]).all()), f"unstable bucket near {lo}"

"""Plant plausible slips in a private copy of the oracle and check that a pin catches each.

The mutation happens on the CPU, in a temporary copy of the oracle package; the real
oracle is never modified.  A mutant that every pin lets through marks a hole in the pins.
"""

import importlib
import os
import shutil
import sys

import pytest

import pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

# (file, original text, planted slip, what the slip means)
MUTANTS = [
    ("router.py", "q = s + b[None, :]", "q = sigmoid_scores(z + b[None, :])", "bias inside the sigmoid"),
    ("router.py", "gates[lo:hi] = gate_values(s, i, normalize)", "gates[lo:hi] = gate_values(q, i, normalize)",
     "gates from s + b"),
    ("router.py", 'order = np.argsort(-q, axis=1, kind="stable")', 'order = np.argsort(q, axis=1, kind="stable")[:, ::-1]',
     "ties to the higher index"),
    ("router.py", "q = s + b[None, :]", "q = s - b[None, :]", "bias subtracted"),
    ("router.py", "return widen(x) @ widen(w).T", "return widen(x)[:, :-1] @ widen(w)[:, :-1].T", "dropped last term"),
    ("router.py", "1.0 / (1.0 + np.exp(-z))", "1.0 / (1.0 + np.exp(z))", "sigmoid sign"),
    ("router.py", "gap = q[rows, order[:, k - 1]] - q[rows, order[:, k]]",
     "gap = q[rows, order[:, 0]] - q[rows, order[:, k]]", "gap from the first choice"),
    ("router.py", "return sel / sel.sum(axis=1, keepdims=True)", "return sel / s.sum(axis=1, keepdims=True)",
     "normalised over every expert"),
    ("router.py", "z = widen(x[lo:hi]) @ w64.T", "z = widen(x[lo:hi]) @ w64[::-1].T", "expert rows reversed"),
    ("balance.py", "db = db_raw - db_raw.mean()", "db = db_raw", "no re-centre"),
    ("balance.py", "m_new = beta * m + (1.0 - beta) * db", "m_new = beta * m + db", "momentum without (1-beta)"),
    ("balance.py", "b_new = b + m_new", "b_new = b + db", "bias stepped by db, not m"),
    ("balance.py", "v = (nbar - n) / nbar", "v = (n - nbar) / nbar", "violation sign"),
    ("balance.py", "np.tanh(kappa * v)", "np.tanh(v)", "dropped kappa"),
    ("balance.py", "b_new = b_new - b_new.mean()", "b_new = b_new - b.mean()", "sign mode re-centres the old b"),
    ("balance.py", "m_new = beta * m + (1.0 - beta) * db\n", "m_new = beta * m + (1.0 - beta) * db_raw\n",
     "re-centre after momentum"),
    ("balance.py", "db = gamma * np.sign(nbar - n)", "db = gamma * np.sign(nbar - n + 0.5)", "sign(0) taken as +1"),
    ("balance.py", 'vt = np.tanh(kappa * v) if mode == "smebu" else v', "vt = np.tanh(kappa * v)",
     "linear mode through tanh"),
    ("balance.py", "return BalanceStep(b_new, m.copy(), db, db.copy())",
     "return BalanceStep(b_new, beta * m + (1.0 - beta) * db, db, db.copy())", "sign mode moves the momentum"),
    ("balance.py", "nbar = n.sum() / len(n)\n    if mode", "nbar = n.sum() / (len(n) - 1)\n    if mode",
     "mean load over N_r - 1"),
    ("loads.py", "offsets = np.concatenate([[0], np.cumsum(counts)])",
     "offsets = np.concatenate([np.cumsum(counts), [counts.sum()]])", "inclusive bucket offsets"),
    ("loads.py", "inv[perm] = np.arange(len(perm), dtype=np.int64)", "inv[:] = perm", "inv taken as perm"),
    ("zloss.py", "np.exp(z - zmax).sum(axis=1", "np.exp(z - zmax).mean(axis=1", "log-mean-exp"),
    ("loads.py", 'np.argsort(flat, kind="stable")', 'np.argsort(flat, kind="quicksort")', "unstable dispatch"),
    ("loads.py", "ratio = float(\"inf\") if nmin == 0 else nmax / nmin",
     "ratio = float(\"inf\") if nmin == 0 else nmax / nbar", "MaxVio over the mean"),
    ("loads.py", "return ratio, (nmax - nbar) / nbar", "return ratio, (nmax - nmin) / nbar", "excess over min"),
    ("zloss.py", "lse = (zmax + np.log(", "lse = (np.log(", "dropped max shift"),
    ("zloss.py", "return float(np.mean(lse * lse)) if lse.size", "return float(np.mean(lse) ** 2) if lse.size",
     "square of the mean"),
    ("balance.py", "balance_step(counts[l], bias[l], momentum[l]", "balance_step(counts[0], bias[l], momentum[l]",
     "every layer fed layer 0's loads"),
    ("moe.py", "return x[perm // k]", "return x[perm % len(x)]", "flat index taken as the token"),
    ("moe.py", "y += g[:, j:j + 1] * eo[rows[:, j]]", "y += g[:, j:j + 1] * eo[rows[:, 0]]", "every slot reads slot 0"),
    ("moe.py", "rows = np.asarray(inv, dtype=np.int64).reshape(g.shape[0], k)",
     "rows = np.asarray(inv, dtype=np.int64).reshape(k, g.shape[0]).T", "inv read slot-major"),
    ("backward.py", "ds = (G - (G * g).sum(axis=1, keepdims=True)) / S", "ds = G / S",
     "normalisation coupling dropped"),
    ("backward.py", "dz[rows, idx] = ds * sel * (1.0 - sel)", "dz[rows, idx] = ds * sel", "sigmoid derivative s, not s(1-s)"),
    ("backward.py", "dz += zloss_coef * (2.0 / T) * lse * p", "dz += zloss_coef * (1.0 / T) * lse * p",
     "z-loss factor 2 dropped"),
    ("backward.py", "return RouterGrads(dz=dz, dx=dz @ w64, dw=dz.T @ x64",
     "return RouterGrads(dz=dz, dx=dz @ w64, dw=dz.T @ x64[::-1]", "tokens reversed in dW"),
    ("backward.py", "return RouterGrads(dz=dz, dx=dz @ w64,", "return RouterGrads(dz=dz, dx=dz @ w64[::-1],",
     "expert rows reversed in dX"),
]


def _load_mutant(tmp_path, i, fname, old, new):
    pkg = f"oracle_mutant_{i}"
    dst = tmp_path / pkg
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("__pycache__"))
    path = dst / fname
    src = path.read_text()
    assert src.count(old) == 1, f"mutation anchor not unique in {fname}: {old!r}"
    path.write_text(src.replace(old, new))
    sys.path.insert(0, str(tmp_path))
    try:
        return importlib.import_module(pkg)
    finally:
        sys.path.remove(str(tmp_path))


@pytest.mark.parametrize("i", range(len(MUTANTS)), ids=[m[3] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, i):
    fname, old, new, what = MUTANTS[i]
    mod = _load_mutant(tmp_path, i, fname, old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin catches the planted slip: {what}"

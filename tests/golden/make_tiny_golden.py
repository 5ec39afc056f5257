"""Write tests/golden/tiny_oracle.json: the oracle's outputs on the tiny fp32 workload.

Calls only the seeded input generator and the CPU oracle.  The fixture pins the oracle
against unintended changes of its own arithmetic; a deliberate change must regenerate it
and say why in the commit message.

    python tests/golden/make_tiny_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle  # noqa: E402


def build():
    wl = datagen.WORKLOADS["tiny"]
    x, w = datagen.tokens(wl), datagen.router_weight(wl)
    b, m = datagen.initial_bias(wl), datagen.initial_momentum(wl)
    r = oracle.route(x, w, b, wl.k)
    n = oracle.expert_loads(r.idx, wl.n_experts)
    ratio, rel = oracle.max_violation(n)
    st = oracle.balance_step(n, b, m, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa)
    return {
        "_about": "oracle outputs on the tiny fp32 workload (T=512, d=256, N_r=16, K=2, SMEBU); "
                  "written by tests/golden/make_tiny_golden.py",
        "workload": wl.label,
        "idx": r.idx.tolist(),
        "gates": [[float(v) for v in row] for row in r.gates],
        "counts": n.tolist(),
        "maxvio": [ratio, rel],
        "bias": st.bias.tolist(),
        "momentum": st.momentum.tolist(),
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(out, "w") as f:
        json.dump(build(), f, separators=(",", ":"))
    print("wrote", out)

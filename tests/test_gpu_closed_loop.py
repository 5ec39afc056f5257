"""Closed loop: 300 consecutive steps with fixed router weights and fresh clustered tokens each
step; b and m persist on the GPU.  The same token stream drives three balancers side by side
(SMEBU, the Nano/Mini sign step and the linear unclamped step).

Every step is teacher-forced: the oracle routes that step's tokens with the GPU's own
pre-step bias (every token at steps 0, 25, 50, ... and the last step, for all three modes; a
seeded sample plus the ragged tail otherwise), counts the GPU's indices, and applies its
update to the GPU's counts and pre-step b, m; b and m must agree within 1e-6.  Near-ties of the
whole-batch checks are counted and reported per mode.  (A free-running oracle would
drift by design: one excused near-tie moves a load by one, which moves the step by about
lambda kappa / nbar.)  A resume check restarts SMEBU from a copy of (b, m) taken 50 steps
before the end and must land on the same bits."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import check_balance, check_counts, compare_route, log, sample_rows, to_dev

pytestmark = pytest.mark.gpu

MODES = ("smebu", "sign", "linear")


@pytest.mark.timeout(900)
def test_closed_loop_three_balancers():
    wl = datagen.WORKLOADS["loop"]
    w = datagen.router_weight(wl)
    b0 = datagen.initial_bias(wl)
    wd = to_dev(w)
    state = {m: (to_dev(b0), torch.zeros(wl.n_experts, dtype=torch.float32, device="cuda")) for m in MODES}
    maxvio = {m: [] for m in MODES}
    worst = {m: 0.0 for m in MODES}
    ties = 0
    full = {m: None for m in MODES}  # merged whole-batch checks per mode
    resume_at = wl.steps - 50
    saved = None
    for step in range(wl.steps):
        x = datagen.tokens(wl, step=step)
        xd = to_dev(x)
        whole = step % 25 == 0 or step == wl.steps - 1
        rows = None if whole else sample_rows(wl.T, 48, seed=step)
        for mode in MODES:
            bd, md = state[mode]
            b_prev, m_prev = bd.cpu().numpy(), md.cpu().numpy()
            if mode == "smebu" and step == resume_at:
                saved = (b_prev.copy(), m_prev.copy())
            idx, gates, counts = elb.router_forward(xd, wd, bd, wl.k)
            _, mv = elb.smebu_update(counts, bd, md, mode=mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa,
                                     gamma=wl.gamma)
            torch.cuda.synchronize()
            idx_h, counts_h = idx.cpu().numpy(), counts.cpu().numpy()
            rep = compare_route(idx_h, gates.cpu().numpy(), x, w, b_prev, wl.k, rows)
            ties += rep.ties
            if whole:
                assert rep.n_tokens == wl.T
                full[mode] = rep if full[mode] is None else full[mode].merge(rep)
            c64 = check_counts(counts_h, idx_h, wl.n_experts)
            worst[mode] = max(worst[mode], check_balance(mode, c64, b_prev, m_prev, bd.cpu().numpy(),
                                                         md.cpu().numpy(), wl))
            maxvio[mode].append(float(mv.cpu().numpy()[0]))
        if step % 50 == 0 or step == wl.steps - 1:
            log(f"step {step}: MaxVio " + ", ".join(f"{m} {maxvio[m][-1]:.2f}" for m in MODES))
    for m in MODES:
        log(f"{m}: max |b,m error| {worst[m]:.2e}; MaxVio first {maxvio[m][0]:.2f} "
            f"mean of last 50 {np.mean(maxvio[m][-50:]):.2f}")
    log(f"near-ties, all checked tokens: {ties}")
    for m in MODES:
        log(f"{m}, whole batches at every 25th step: {full[m]}")

    # Resume: restart SMEBU from the saved (b, m) and replay the second half; bit-exact.
    bd, md = to_dev(saved[0]), to_dev(saved[1])
    for step in range(resume_at, wl.steps):
        xd = to_dev(datagen.tokens(wl, step=step))
        _, _, counts = elb.router_forward(xd, wd, bd, wl.k)
        elb.smebu_update(counts, bd, md, mode="smebu", lam=wl.lam, beta=wl.beta, kappa=wl.kappa)
    torch.cuda.synchronize()
    sb, sm = state["smebu"]
    assert (bd.cpu().numpy().view(np.uint32) == sb.cpu().numpy().view(np.uint32)).all()
    assert (md.cpu().numpy().view(np.uint32) == sm.cpu().numpy().view(np.uint32)).all()

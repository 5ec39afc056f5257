"""The fused routed step at the largest batch its int32 positions allow: T = 268,435,455 tokens
(d = 64, N_r = 256, K = 8), so idx and gates (8.6 GB each), perm and inv pass 4 GiB of byte
offsets, the MFMA router runs 1,048,576 workgroups and fills a loads table of as many tiles,
and every per-expert count sits near 2^23.  Routing is checked against the oracle on sampled
rows (around the first token whose outputs start past 4 GiB, and the ragged tail); the counts
against the histogram of the indices, the dispatch through its defining properties, and the
bias update against the oracle, all on the whole batch."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import check_balance, check_dispatch_device, check_maxvio, compare_route, log, sample_rows, to_dev

pytestmark = pytest.mark.gpu

T, D, N_E, K = (1 << 31) // 8 - 1, 64, 256, 8
CHUNK = 1 << 24  # tokens per chunk of the on-device checks


def test_routed_step_at_the_int32_position_limit():
    wl = datagen.WORKLOADS["large"].replace(T=T, d=D, k=K, seed=43)
    log(f"max routed step: T={T} d={D} N_r={N_E} K={K}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    xd = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    for lo in range(0, T, CHUNK):
        hi = min(lo + CHUNK, T)
        # x 8 (exact in bf16): at d = 64 this scale puts the fewest selections in the tie band
        # (~13% against ~25% unscaled, on the oracle: the 8th and 9th of 256 scores lie close)
        xd[lo:hi] = (8.0 * torch.randn((hi - lo, D), generator=gen, device="cuda")).to(torch.bfloat16)
    w, b0, m0 = datagen.router_weight(wl), datagen.initial_bias(wl), datagen.initial_momentum(wl)
    bd, md = to_dev(b0), to_dev(m0)
    step = elb.RouterStep(to_dev(w), bd, md, K, T, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa,
                          gamma=wl.gamma, want_delta=True, clear_counts=False)
    out = step(xd)
    torch.cuda.synchronize()
    idx, gates = out.topk_idx, out.gates

    # Whole batch, on the device: ids in range and distinct per token, gates normalised, counts
    # equal to the histogram of the ids.
    hist = torch.zeros(N_E, dtype=torch.int64, device="cuda")
    for lo in range(0, T, CHUNK):
        hi = min(lo + CHUNK, T)
        s = torch.sort(idx[lo:hi], dim=1).values
        assert int(s[:, 0].min()) >= 0 and int(s[:, -1].max()) < N_E
        assert bool((s[:, 1:] > s[:, :-1]).all()), f"a token lists an expert twice near {lo}"
        g = gates[lo:hi].double().sum(dim=1)
        assert float((g - 1.0).abs().max()) <= 4e-6, f"gates not normalised near {lo}"
        hist += torch.bincount(idx[lo:hi].reshape(-1).long(), minlength=N_E)
    counts64 = out.counts.cpu().numpy().astype(np.int64)
    assert (counts64 == hist.cpu().numpy()).all(), "counts differ from the histogram of the ids"

    # Sampled rows against the oracle: around the first token whose idx/gates bytes start past
    # 4 GiB, and the ragged tail.
    mark = 2 ** 32 // (K * 4)
    rows = sample_rows(T, 1500, seed=11, extra=range(mark - 8, mark + 8))
    rows_t = torch.from_numpy(rows).to("cuda")
    xs = xd[rows_t].view(torch.int16).cpu().numpy().view(np.uint16)
    rep = compare_route(idx[rows_t].cpu().numpy(), gates[rows_t].cpu().numpy(), xs, w, b0, K)
    log(f"  routing: {rep.n_tokens} sampled tokens, ties {rep.ties}, gate rel err {rep.max_gate_rel:.2e}")

    # The dispatch of the whole batch and the bias update from its counts.
    del xd
    check_dispatch_device(out.offsets, out.perm, out.inv_perm, idx.view(-1), N_E)
    check_balance(wl.mode, counts64, b0, m0, bd.cpu().numpy(), md.cpu().numpy(), wl, out.delta_b.cpu().numpy())
    check_maxvio(out.maxvio.cpu().numpy(), counts64)
    log(f"  counts, dispatch of {T * K} assignments and the bias update hold")

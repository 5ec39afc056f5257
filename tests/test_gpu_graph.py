"""The routed step captured once in a HIP graph and replayed (the form a serving loop or a
graph-captured training step uses): every replay must give exactly what the same step run
eagerly gives from the same state.  The step's kernels are launched through plain kernel
launches (no memset nodes, no allocation inside the call), so each replay runs them again on
the captured buffers: the bias and momentum move every replay, and the eager twin follows them.
Replays are separated by the program's own eager work and synchronisations, and every replay
is compared, not only the first."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d,dispatch,mode", [
    (40000, 256, True, "smebu"),   # 256-token tiles: router, then the dispatch launch with the update in it
    (20000, 256, True, "linear"),  # 128-token tiles: the dispatch counts the loads itself
    (700, 256, True, "smebu"),     # 64-token tiles, ragged tail
    (2048, 256, False, "sign"),    # 64-token tiles: router, then the update launch
])
def test_replayed_step_matches_eager(T, d, dispatch, mode):
    log(f"graph replay T={T} d={d} dispatch={dispatch} mode={mode}")
    wl = datagen.WORKLOADS["large"].replace(T=T, d=d, seed=11, n_clusters=8, gamma=1e-3)
    w = to_dev(datagen.router_weight(wl))
    b0 = datagen.initial_bias(wl)
    m0 = np.zeros(wl.n_experts, dtype=np.float32)
    rng = np.random.default_rng(5)
    batches = [to_dev(datagen.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))) for _ in range(4)]

    def make_step(b, m):
        return elb.RouterStep(w, b, m, wl.k, T, mode=mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa,
                              gamma=wl.gamma, want_delta=True, dispatch=dispatch)

    b_e, m_e = to_dev(b0), to_dev(m0)
    b_g, m_g = to_dev(b0), to_dev(m0)
    eager, graphed = make_step(b_e, m_e), make_step(b_g, m_g)
    x_static = torch.empty_like(batches[0])
    # A throwaway step of the same shapes first, so that no kernel is loaded for the first time
    # inside the capture.
    make_step(to_dev(b0), to_dev(m0))(batches[0])
    torch.cuda.synchronize()

    # Capture on a side stream, as torch requires; nothing runs during the capture itself.
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            out_g = graphed(x_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def host(out, b, m):
        vals = [out.topk_idx, out.gates, out.counts, out.delta_b, out.maxvio, b, m]
        if dispatch:
            vals += [out.offsets, out.perm, out.inv_perm]
        return [v.cpu().numpy().copy() for v in vals]

    for i, x in enumerate(batches):
        x_static.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        got = host(out_g, b_g, m_g)
        out_e = eager(x)
        torch.cuda.synchronize()
        want = host(out_e, b_e, m_e)
        for gv, wv in zip(got, want):
            assert np.array_equal(gv, wv, equal_nan=True), f"replay {i} differs from the eager step"
        _ = (x.float().sum() * 0).item()  # unrelated eager work between replays
    log(f"  {len(batches)} replays bit-identical to the eager steps; bias moved by "
        f"{float(np.abs(b_g.cpu().numpy() - b0).max()):.3g}")

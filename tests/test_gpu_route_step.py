"""GPU parity of the fused routed step (elb_route_step / RouterStep): forward, dispatch and the
bias update in three kernels must give exactly what the three separate calls give, which the
other GPU tests hold to the oracle; the first step is also checked against the oracle here."""

import numpy as np
import pytest
import torch

import datagen
import expert_load_balancing_amd as elb
from gpu_util import check_balance, check_counts, check_dispatch, check_maxvio, compare_route, log, to_dev

pytestmark = pytest.mark.gpu


def make(T, d, n_e, k, dtype="bf16", seed=3):
    wl = datagen.WORKLOADS["large"].replace(T=T, d=d, n_experts=n_e, k=k, dtype=dtype, seed=seed, n_clusters=8)
    return wl, datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)


def separate_step(x, w, b, m, k, mode, wl, counts, force_generic):
    """The same step from the three separate entry points; returns host copies."""
    idx, gates, counts = elb.router_forward(x, w, b, k, counts=counts, accumulate=True, force_generic=force_generic)
    offs, perm, inv = elb.router_dispatch(idx, w.shape[0])
    c = counts.clone()
    delta, mv = elb.smebu_update(counts, b, m, mode=mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa, gamma=wl.gamma,
                                 want_delta=True, clear_counts=True)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (idx, gates, c, offs, perm, inv, b, m, delta, mv)]


@pytest.mark.parametrize("T,d,n_e,k,dtype,kernel", [
    (700, 256, 256, 4, "bf16", "mfma"),      # 3 tiles, ragged tail
    (4096, 512, 256, 4, "bf16", "mfma"),
    (1300, 256, 64, 8, "bf16", "mfma"),      # padded experts, K = 8
    (513, 128, 200, 3, "bf16", "mfma"),
    (257, 64, 16, 1, "bf16", "mfma"),
    (300, 96, 32, 2, "f32", "generic"),      # fp32: the generic kernel plus a counting pass
    (1000, 256, 256, 4, "bf16", "generic"),
])
@pytest.mark.parametrize("mode", ["smebu", "sign", "linear"])
def test_step_matches_separate_calls(T, d, n_e, k, dtype, kernel, mode):
    log(f"route_step T={T} d={d} N_r={n_e} K={k} {dtype} kernel={kernel} mode={mode}")
    wl, x, w, b0 = make(T, d, n_e, k, dtype)
    wl = wl.replace(gamma=1e-3)
    xd, wd = to_dev(x), to_dev(w)
    m0 = np.zeros(n_e, dtype=np.float32)
    b_sep, m_sep, c_sep = to_dev(b0), to_dev(m0), torch.zeros(n_e, dtype=torch.int32, device="cuda")
    b_fus, m_fus = to_dev(b0), to_dev(m0)
    step = elb.RouterStep(wd, b_fus, m_fus, k, T, mode=mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa,
                          gamma=wl.gamma, want_delta=True, force_generic=(kernel == "generic"))
    for it in range(3):  # the bias moves between steps, so later steps route differently
        b_prev, m_prev = b_fus.cpu().numpy(), m_fus.cpu().numpy()
        want = separate_step(xd, wd, b_sep, m_sep, k, mode, wl, c_sep, kernel == "generic")
        out = step(xd)
        torch.cuda.synchronize()
        got = [t.cpu().numpy() for t in (out.topk_idx, out.gates)]
        counts_after = out.counts.cpu().numpy()
        got += [None] + [t.cpu().numpy() for t in (out.offsets, out.perm, out.inv_perm, b_fus, m_fus, out.delta_b,
                                                   out.maxvio)]
        names = ["idx", "gates", "counts", "offsets", "perm", "inv", "bias", "momentum", "delta_b", "maxvio"]
        for name, g, s in zip(names, got, want):
            if g is not None:
                assert np.array_equal(g, s, equal_nan=True), f"step {it}: {name} differs from the separate calls"
        assert (counts_after == 0).all(), "the step must leave the loads cleared"
        if it == 0:
            rep = compare_route(got[0], got[1], x, w, b_prev, k)
            counts = check_counts(want[2], got[0], n_e)
            check_dispatch(got[3], got[4], got[5], got[0], n_e)
            check_balance(mode, counts, b_prev, m_prev, got[6], got[7], wl, got[8])
            check_maxvio(got[9], counts)
            log(f"  ties={rep.ties} gate rel err={rep.max_gate_rel:.2e}")


def test_step_accumulates_micro_batches():
    """Without the update the loads add up over calls; an update with clear then consumes them."""
    T, d, n_e, k = 600, 256, 256, 4
    wl, x, w, b0 = make(T, d, n_e, k, seed=9)
    xd, wd = to_dev(x), to_dev(w)
    bd = to_dev(b0)
    step = elb.RouterStep(wd, bd, None, k, T, update=False)
    total = np.zeros(n_e, dtype=np.int64)
    for lo, hi in ((0, 256), (256, 600), (100, 101)):
        out = step(xd[lo:hi].contiguous())
        torch.cuda.synchronize()
        total += np.bincount(out.topk_idx.cpu().numpy().ravel(), minlength=n_e)
        assert (out.counts.cpu().numpy() == total).all()
        assert out.maxvio is None and out.delta_b is None
        check_dispatch(out.offsets.cpu().numpy(), out.perm.cpu().numpy(), out.inv_perm.cpu().numpy(),
                       out.topk_idx.cpu().numpy(), n_e)
    assert (bd.cpu().numpy() == b0).all(), "no update was asked for"
    md = torch.zeros(n_e, dtype=torch.float32, device="cuda")
    b_prev = bd.cpu().numpy()
    _, mv = elb.smebu_update(step.counts, bd, md, clear_counts=True)
    torch.cuda.synchronize()
    check_balance("smebu", total, b_prev, np.zeros(n_e, np.float32), bd.cpu().numpy(), md.cpu().numpy(), wl)
    check_maxvio(mv.cpu().numpy(), total)
    assert (step.counts.cpu().numpy() == 0).all()


def test_step_empty_batch_still_updates():
    """T = 0: nothing is routed, offsets are zero, and the update runs on the loads so far."""
    n_e, k, d = 64, 2, 128
    wl, x, w, b0 = make(300, d, n_e, k, seed=4)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b0)
    md = torch.zeros(n_e, dtype=torch.float32, device="cuda")
    acc = elb.RouterStep(wd, bd, md, k, 300, update=False)
    acc(xd)
    torch.cuda.synchronize()
    counts = acc.counts.cpu().numpy().astype(np.int64)
    fused = elb.RouterStep(wd, bd, md, k, 300)
    fused.counts.copy_(acc.counts)
    out = fused(xd[:0])
    torch.cuda.synchronize()
    check_balance("smebu", counts, b0, np.zeros(n_e, np.float32), bd.cpu().numpy(), md.cpu().numpy(), wl)
    assert (out.offsets.cpu().numpy() == 0).all() and out.perm.numel() == 0
    assert (out.counts.cpu().numpy() == 0).all()
    # And with no loads at all the update is skipped.
    b1 = bd.cpu().numpy()
    out = fused(xd[:0])
    torch.cuda.synchronize()
    assert (bd.cpu().numpy() == b1).all() and np.isnan(out.maxvio.cpu().numpy()).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])  # the MFMA kernel and the generic one
def test_step_timing_events(dtype):
    """Events handed to the step bracket the router kernel; the routing is the same with and
    without them, and an empty batch gives a (near) empty interval."""
    T, d, n_e, k = 1024, 512, 256, 4
    _, x, w, b0 = make(T, d, n_e, k, dtype=dtype, seed=2)
    xd = to_dev(x)
    outs = []
    for timed in (True, False):
        step = elb.RouterStep(to_dev(w), to_dev(b0), torch.zeros(n_e, device="cuda"), k, T, update=False)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if timed:
            step.set_timing(start, stop)
        out = step(xd)
        torch.cuda.synchronize()
        if timed:
            ms = start.elapsed_time(stop)
            assert 0.0 < ms < 100.0, ms
            step(xd[:0])
            torch.cuda.synchronize()
            assert 0.0 <= start.elapsed_time(stop) < 100.0
            # One event per call: from before the first router kernel to the end of the second.
            step.set_timing(start, None)
            step(xd)
            step.set_timing(None, stop)
            step(xd)
            torch.cuda.synchronize()
            assert 0.0 < start.elapsed_time(stop) < 200.0
            step.set_timing()
            out = step(xd)
            torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (out.topk_idx, out.gates)])
    for a, b in zip(*outs):
        assert (a == b).all()


def test_route_step_without_dispatch_matches():
    """offsets, perm and inv_perm all NULL: the step routes and updates exactly as with the
    dispatch (same idx, gates, counts, bias, momentum), and produces no permutation."""
    for T in (5000, 40000):  # a 128-token tile batch and a 256-token tile batch
        wl = datagen.WORKLOADS["large"].replace(T=T, d=512, seed=T, n_clusters=8)
        x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
        res = []
        for dispatch in (True, False):
            bd, md = to_dev(b), torch.zeros(wl.n_experts, device="cuda")
            step = elb.RouterStep(to_dev(w), bd, md, wl.k, T, dispatch=dispatch, want_delta=True)
            out = step(to_dev(x))
            torch.cuda.synchronize()
            res.append((out.topk_idx.cpu().numpy(), out.gates.cpu().numpy(), out.delta_b.cpu().numpy(),
                        bd.cpu().numpy(), md.cpu().numpy(), out.maxvio.cpu().numpy()))
            if not dispatch:
                assert out.offsets is None and out.perm is None and out.inv_perm is None
        for a, c in zip(res[0], res[1]):
            assert np.array_equal(a, c)
        log(f"T={T}: identical with and without dispatch")


@pytest.mark.parametrize("T", [16384, 16385, 32768, 32769, 40000, 65535, 65536, 65537])
def test_route_step_dispatch_at_tile_switch(T):
    """The fused step's dispatch on either side of the tile-size switch: 128-token router tiles
    (the dispatch counts the loads itself) and 256-token tiles with a ragged tail (the router
    fills the loads table), up to the large workload's 65,536 tokens and one token past it."""
    wl = datagen.WORKLOADS["large"].replace(T=T, d=256, seed=T + 3, n_clusters=8)
    x, w, b = datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl)
    step = elb.RouterStep(to_dev(w), to_dev(b), torch.zeros(wl.n_experts, device="cuda"), wl.k, T, update=False)
    out = step(to_dev(x))
    torch.cuda.synchronize()
    idx = out.topk_idx.cpu().numpy()
    check_counts(out.counts.cpu().numpy(), idx, wl.n_experts)
    check_dispatch(out.offsets.cpu().numpy(), out.perm.cpu().numpy(), out.inv_perm.cpu().numpy(), idx, wl.n_experts)
    log(f"T={T}: dispatch matches the oracle")


@pytest.mark.parametrize("dispatch,update,zloss", [(True, True, False), (False, True, False), (False, False, True),
                                                   (False, False, False), (True, False, True)])
def test_step_end_event(dispatch, update, zloss):
    """The third timing event takes the end of the step's last kernel (the scatter, the update,
    the z-loss, or an empty kernel after a lone router kernel): it is never before the router
    kernel's end, and timing changes no output."""
    T, d, n_e, k = 3000, 512, 256, 4
    _, x, w, b0 = make(T, d, n_e, k, seed=3)
    xd = to_dev(x)
    outs = []
    for timed in (True, False):
        step = elb.RouterStep(to_dev(w), to_dev(b0), torch.zeros(n_e, device="cuda"), k, T, update=update,
                              dispatch=dispatch, want_zloss=zloss)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        if timed:
            step.set_timing(*ev)
        out = step(xd)
        torch.cuda.synchronize()
        if timed:
            r, e = ev[0].elapsed_time(ev[1]), ev[0].elapsed_time(ev[2])
            log(f"  dispatch={dispatch} update={update} zloss={zloss}: router {r * 1e3:.1f} us, step {e * 1e3:.1f} us")
            assert 0.0 < r <= e < 100.0, (r, e)
        got = [t.cpu().numpy() for t in (out.topk_idx, out.gates, step.bias)]
        if dispatch:
            got += [out.perm.cpu().numpy()]
        outs.append(got)
    for a, b in zip(*outs):
        assert (a == b).all()


@pytest.mark.parametrize("T,dtype", [(3000, "bf16"), (20000, "bf16"), (40000, "bf16"), (1000, "f32"), (0, "bf16")])
def test_step_counts_without_accumulate(T, dtype):
    """Without ELB_ACCUMULATE_COUNTS a step with a dispatch sets the loads to this batch's (its
    scan writes them over whatever `counts` held; an empty batch leaves zeros), on the 256-token
    tile that fills the loads table, on the 64- and 128-token tiles and on the fp32 generic kernel."""
    n_e, k = 256, 4
    wl = datagen.WORKLOADS["large"].replace(T=max(T, 1), d=128, n_experts=n_e, k=k, dtype=dtype, seed=T + 11,
                                            n_clusters=8)
    x, w, b = datagen.tokens(wl)[:T], datagen.router_weight(wl), datagen.initial_bias(wl)
    step = elb.RouterStep(to_dev(w), to_dev(b), None, k, max(T, 1), update=False)
    step._args.flags &= ~elb.ELB_ACCUMULATE_COUNTS
    for it in range(2):
        step.counts.fill_(12345 + it)  # stale loads that the step must not add to
        out = step(to_dev(x).contiguous())
        torch.cuda.synchronize()
        idx = out.topk_idx.cpu().numpy()
        got = out.counts.cpu().numpy()
        assert np.array_equal(got, np.bincount(idx.ravel(), minlength=n_e)), f"call {it}: loads differ"
        if T > 0:
            check_dispatch(out.offsets.cpu().numpy(), out.perm.cpu().numpy(), out.inv_perm.cpu().numpy(), idx, n_e)
        else:
            assert (got == 0).all() and (out.offsets.cpu().numpy() == 0).all()
    log(f"T={T} {dtype}: loads set, not accumulated")

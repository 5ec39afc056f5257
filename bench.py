"""Benchmark: routed tokens/s of the full router step on one MI355X.

One step = router forward (logits, sigmoid, biased Top-4, gates, expert loads) + dispatch
permutation + SMEBU bias update with MaxVio: one elb_route_step call (three kernels) on one
stream, inputs resident in HBM.  Default workload: one GPU's micro-batch share of the Large-style
step, T = 65536 tokens, d = 3072, N_r = 256, K = 4, 32 Zipf clusters (synthetic).

    python bench.py [--steps K] [--warmup W] [--workload large] [--no-cpu]

Prints one JSON line: throughput, the router kernel's roofline position (algorithmic HBM
bytes over its average duration across 200 back-to-back launches on the same stream, between
fence-free HIP events bound to the kernels), HBM traffic from the committed rocprofv3 counter
summary when it matches the current kernel source, the dispatch's achieved bytes, the rows
beside the hot path, and the CPU oracle timed on the host on the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
METRIC = "routed tokens/s (logits+top-4+counts+SMEBU) at N_r=256,K=4; % roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "router_mfma_traffic.json")
KERNEL_SOURCES = ["expert_load_balancing_amd/csrc/router_mfma.hip", "expert_load_balancing_amd/csrc/mfma_tile.hpp",
                  "expert_load_balancing_amd/csrc/device_common.hpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence, through the HIP runtime torch
    already loaded.  Handed to a kernel launch as its stop event, it takes the kernel's own end
    time stamp (no marker packet, no cache write-back or invalidation), as a profiler's kernel
    trace sees it.  Duck-types the parts of torch.cuda.Event that RouterStep.set_timing and the
    bench use."""

    _hip = None

    def __init__(self) -> None:
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so.7")  # resolves to the copy already loaded
        h = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(0x20000000))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self, stream) -> None:
        rc = self._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                           ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self) -> None:
        if TimingEvent._hip is not None and getattr(self, "cuda_event", None):
            TimingEvent._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def router_kernel_name(T: int, n_e: int, k: int) -> str:
    """The MFMA router instantiation a forward of T tokens runs, as the profiler names it:
    <K, all 256 experts, no logits/lse copy, 32-token blocks per wave pair, waves / 2> with the
    256-token tile above 128 x 256 tokens, the 128-token tile above 64 x 256, else the 64-token."""
    nb, tg = (2, 4) if T > 128 * 256 else (1, 4) if T > 64 * 256 else (1, 2)
    return f"router_mfma_kernel<{k}, {'true' if n_e == 256 else 'false'}, false, {nb}, {tg}>"


def dispatch_alg_bytes(T: int, n_e: int, k: int) -> int:
    """HBM bytes the dispatch must move: idx in once, perm and inv out, offsets out."""
    return T * k * 4 * 3 + (n_e + 1) * 4


def router_alg_bytes(T: int, d: int, n_e: int, k: int) -> int:
    """HBM bytes the router forward must move: X once, W once, idx + gates out, b in, counts."""
    return T * (2 * d + 8 * k) + n_e * 2 * d + n_e * 4 + n_e * 4


def traffic_from_profile(T: int) -> float | None:
    """Counter-measured HBM bytes per router launch, if taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("T") != T:
        return None
    return float(rec["traffic_bytes_per_launch"])


def summarize_traffic(fetch_csv: str, write_csv: str, copy_mib: int, T: int, launches: int) -> dict:
    """HBM bytes per router launch from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE).

    Both counters report KiB per dispatch, summed here over the counter's instances, and are
    averaged over the last `launches` router launches: the back-to-back launches the roofline
    times.  (Inside a step the counters of the router launch also take in the write-back of the
    permutation the previous step's scatter left in the cache, 2 MiB more.)  Each is scaled by
    what it reads for the plain device-to-device copy of known size that ``--calibrate-copy``
    runs in the same program (the copy reads and writes copy_mib MiB).
    """
    import csv
    from collections import defaultdict

    def per_kernel(path, counter, key, last=None):
        acc = defaultdict(float)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and key in r["Kernel_Name"]:
                    acc[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        ids = sorted(acc)[-last:] if last else sorted(acc)
        return sum(acc[i] for i in ids) / len(ids)

    # The calibration copies are the last three blits of the program (earlier blits are the
    # host-to-device uploads of the inputs).
    copy_bytes = copy_mib * 1024 * 1024
    f_router = per_kernel(fetch_csv, "FETCH_SIZE", "router_mfma_kernel", last=launches)
    w_router = per_kernel(write_csv, "WRITE_SIZE", "router_mfma_kernel", last=launches)
    f_copy = per_kernel(fetch_csv, "FETCH_SIZE", "copyBuffer", last=3)
    w_copy = per_kernel(write_csv, "WRITE_SIZE", "copyBuffer", last=3)
    f_scale, w_scale = copy_bytes / (f_copy * 1024), copy_bytes / (w_copy * 1024)
    return {
        "kernel_source_sha256": kernel_source_hash(), "T": T, "launches_averaged": launches,
        "fetch_kib_per_launch": f_router, "write_kib_per_launch": w_router,
        "copy_mib": copy_mib, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "traffic_bytes_per_launch": f_router * 1024 * f_scale + w_router * 1024 * w_scale,
    }


def cpu_baseline(wl, x, w, b, m, min_seconds: float = 10.0, max_seconds: float = 30.0) -> dict:
    """The oracle (untuned) on the whole step of the same workload, repeated for >= min_seconds."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    cores = min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=cores):
        reps, t0 = 0, time.perf_counter()
        while True:
            r = oracle.route(x, w, b, wl.k)
            n = oracle.expert_loads(r.idx, wl.n_experts)
            oracle.max_violation(n)
            if wl.dispatch:
                oracle.dispatch_permutation(r.idx, wl.n_experts)
            oracle.balance_step(n, b, m, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa, gamma=wl.gamma)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or el * (reps + 1) / reps > max_seconds:
                break
    return {"value": reps * wl.T / el, "unit": "routed tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full step of {wl.label} (route + loads + MaxVio"
                      f"{' + dispatch' if wl.dispatch else ''} + {wl.mode} update), {reps} repetition(s), "
                      f"fp64 numpy, BLAS threads={cores}",
            "seconds": round(el, 2)}


def time_events(fn, reps: int, stream, per_call: bool = False) -> float:
    """Average ms of fn() over reps runs between HIP events on `stream`: back to back between two
    events, or (per_call, for kernels of a few microseconds, whose back-to-back rate is the
    host's launch rate) bracketed one by one with fence-free events."""
    import torch

    fn()
    torch.cuda.synchronize()
    if per_call:
        ev = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / reps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def bench_next_rows(elb, wl, x, w, out, stream, reps: int = 20) -> dict:
    """The rows beside the hot path, on the same workload and stream: router z-loss reduction,
    a 60-layer batched bias update, the router backward, the expert-contiguous permute and the
    gated combine."""
    import torch

    T, d, k, n_e = wl.T, wl.d, wl.k, wl.n_experts
    res = {}
    lse = torch.randn(T, device=x.device) + 6.0
    res["zloss_us"] = round(time_events(lambda: elb.zloss(lse), reps, stream, per_call=True) * 1e3, 2)
    L = 60
    counts = torch.randint(0, 4 * T // n_e * 2, (L, n_e), dtype=torch.int32, device=x.device)
    bl, ml = torch.zeros((L, n_e), device=x.device), torch.zeros((L, n_e), device=x.device)
    res["update_60_layers_us"] = round(time_events(lambda: elb.smebu_update_layers(counts, bl, ml), reps, stream,
                                                         per_call=True) * 1e3, 2)
    # The permutation of this batch (from the step, or from a dispatch call when the step has none).
    inv = out.inv_perm.clone() if out.inv_perm is not None else elb.router_dispatch(out.topk_idx, n_e)[2]
    gates = out.gates.clone()
    xp = torch.empty((T * k, d), dtype=x.dtype, device=x.device)
    y = torch.empty((T, d), dtype=torch.float32, device=x.device)
    ms_p = time_events(lambda: elb.permute_rows(x, inv, k, out=xp), reps, stream)
    ms_c = time_events(lambda: elb.unpermute_combine(xp, gates, inv, out=y), reps, stream)
    # Router backward with the z-loss (recomputed logits, dL/dz, dX = dZ W, dW = dZ^T X).
    dg = torch.randn((T, k), device=x.device)
    ws_b = torch.empty(elb.backward_workspace_bytes(T, d, n_e), dtype=torch.uint8, device=x.device)
    ms_b = time_events(lambda: elb.router_backward(x, w, out.topk_idx, dg, zloss_coef=1e-3, workspace=ws_b),
                       max(3, reps // 4), stream)
    ms_b16 = time_events(lambda: elb.router_backward(x, w, out.topk_idx, dg, zloss_coef=1e-3, workspace=ws_b,
                                                     dx_dtype=torch.bfloat16), max(3, reps // 4), stream)
    fl = 3 * 2.0 * T * n_e * d
    for name, ms in (("backward", ms_b), ("backward_bf16_dx", ms_b16)):
        res[name] = {"us": round(ms * 1e3, 2), "flops": fl, "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                     "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    esz = x.element_size()
    bytes_p = T * d * esz + T * k * d * esz + T * k * 4
    bytes_c = T * k * d * esz + T * k * 8 + T * d * 4
    for name, ms, nbytes in (("permute", ms_p, bytes_p), ("combine", ms_c, bytes_c)):
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "alg_bytes": nbytes, "achieved_GBps": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-next", action="store_true", help="skip the rows beside the hot path")
    ap.add_argument("--router-launches", type=int, default=200, metavar="R",
                    help="back-to-back router launches timed for the roofline")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a device-to-device copy of MIB MiB (the byte-counter reference)")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_MIB"),
                    help="write the HBM traffic record from two rocprofv3 counter runs and exit")
    args = ap.parse_args()
    if args.summarize_traffic:
        import datagen

        rec = summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], int(args.summarize_traffic[2]),
                                datagen.WORKLOADS[args.workload].T, max(1, args.router_launches))
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import datagen
    import expert_load_balancing_amd as elb

    wl = datagen.WORKLOADS[args.workload]
    elb.lib()  # fails loudly when libelb.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x = datagen.tokens(wl)
    w = datagen.router_weight(wl)
    b0, m0 = datagen.initial_bias(wl), datagen.initial_momentum(wl)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # Two copies of the tokens, alternated step by step, so no step reads its input out of the
    # 256 MB last-level cache that the previous step filled.
    xs = [to_dev(x), to_dev(x)]
    wd, bd, md = to_dev(w), to_dev(b0), to_dev(m0)
    T, d, n_e, k = wl.T, wl.d, wl.n_experts, wl.k
    # One library call per step (elb_route_step): router kernel, dispatch scan, scatter with the
    # bias update beside it (workloads without dispatch: router kernel, then the update).
    # The loads accumulate into counts and the update clears them.
    step = elb.RouterStep(wd, bd, md, k, T, mode=wl.mode, lam=wl.lam, beta=wl.beta, kappa=wl.kappa, gamma=wl.gamma,
                          dispatch=wl.dispatch)
    stream = torch.cuda.current_stream(dev)

    for i in range(args.warmup):
        step(xs[i & 1])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        out = step(xs[i & 1])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    value = T / (ms * 1e-3)
    mv = out.maxvio

    # The router kernel's average launch duration, for the roofline: R launches of it back to
    # back on the same stream (a step with neither dispatch nor update; the counts accumulate),
    # from the end of an empty kernel launched just before the first to the end of the last.
    # The events are fence-free and bound to those two kernels, so no marker sits between the
    # launches; the one dispatch gap after the empty kernel is spread over the R launches.  (A
    # marker beside every launch would add its own ~5 us dispatch gap to each.)  The clock of a
    # power-limited part wanders over milliseconds, so R spans about as long as the steps do.
    solo = elb.RouterStep(wd, bd, None, k, T, update=False, dispatch=False)
    t0, t1 = TimingEvent(), TimingEvent()
    n_solo = max(1, args.router_launches)
    for i in range(2):
        solo(xs[i & 1])
    torch.cuda.synchronize()
    for i in range(n_solo):
        solo.set_timing(t0 if i == 0 else None, t1 if i == n_solo - 1 else None)
        solo(xs[i & 1])
    torch.cuda.synchronize()
    router_ms = t0.elapsed_time(t1) / n_solo

    # The dispatch (a6) through its own entry point, on the last step's indices, back to back:
    # the counting pass, the scan and the scatter (inside the step the router kernel has done the
    # counting).  It moves ~1% of the router's bytes and is bound by latency, not bandwidth.
    dispatch = None
    if wl.dispatch:
        ws_d = torch.empty(elb.dispatch_workspace_bytes(T, k, n_e), dtype=torch.uint8, device=dev)
        idx_last = out.topk_idx.clone()
        outs = (torch.empty(n_e + 1, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev),
                torch.empty(T * k, dtype=torch.int32, device=dev))
        ms_d = time_events(lambda: elb.router_dispatch(idx_last, n_e, workspace=ws_d, out=outs), 50, stream)
        alg_d = dispatch_alg_bytes(T, n_e, k)
        dispatch = {"us": round(ms_d * 1e3, 2), "kernels": 3, "alg_bytes": alg_d,
                    "achieved_GBps": round(alg_d / (ms_d * 1e-3) / 1e9, 1),
                    "frac": round(alg_d / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    alg = router_alg_bytes(T, d, n_e, k)
    achieved = alg / (router_ms * 1e-3) / 1e9
    flops = 2.0 * T * d * n_e
    tflops = flops / (router_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(T)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "routed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.label, "T": T, "d": d, "n_experts": n_e, "k": k, "balance": wl.mode,
                   "dispatch": wl.dispatch, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": router_kernel_name(T, n_e, k), "alg_bytes_per_launch": alg, "launches_timed": n_solo,
                     "kernel_us": round(router_ms * 1e3, 2),
                     "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
        "breakdown_us": {"step": round(ms * 1e3, 2), "router_back_to_back": round(router_ms * 1e3, 2)},
        "dispatch": dispatch,
        "maxvio_last": float(mv.cpu()[0]),
    }
    if not args.no_next:
        line["next_rows"] = bench_next_rows(elb, wl, xs[0], wd, out, stream)
    if args.calibrate_copy:
        n = args.calibrate_copy * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)  # a device-to-device blit of known size
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, x, w, b0, m0)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

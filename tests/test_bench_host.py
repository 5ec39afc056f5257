"""Host logic of bench.py, on the CPU: the refusal of several GPUs, the algorithmic byte count of
the router launch, and the HBM traffic record built from two counter runs (synthetic counter
tables in rocprofv3's CSV layout)."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_router_alg_bytes_large_workload():
    # X once (bf16), idx + gates out, W once (bf16), b in, counts out.
    T, d, n_e, k = 65536, 3072, 256, 4
    assert bench.router_alg_bytes(T, d, n_e, k) == T * 2 * d + T * k * 8 + n_e * d * 2 + n_e * 4 * 2
    assert bench.router_alg_bytes(T, d, n_e, k) == 406_325_248


def test_router_kernel_name_follows_the_tile_switch():
    # The names the profiler prints for the three tiles (see profiles/).
    assert bench.router_kernel_name(65536, 256, 4) == "router_mfma_kernel<4, true, false, 2, 4>"
    assert bench.router_kernel_name(32768, 256, 4) == "router_mfma_kernel<4, true, false, 1, 4>"
    assert bench.router_kernel_name(16384, 200, 2) == "router_mfma_kernel<2, false, false, 1, 2>"
    assert bench.router_kernel_name(512, 16, 2, "f32") == "router_generic_kernel<float, 4>"
    assert bench.router_kernel_name(512, 100, 2, "f32") == "router_generic_kernel<float, 2>"
    assert bench.router_kernel_name(512, 256, 2, "f32") == "router_generic_kernel<float, 1>"


def test_dispatch_alg_bytes_large_workload():
    # idx in (16 B per token at K = 4), perm and inv out (32 B per token), offsets out.
    T, n_e, k = 65536, 256, 4
    assert bench.dispatch_alg_bytes(T, n_e, k) == T * 16 + T * 32 + (n_e + 1) * 4


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, [values of the counter's instances])."""
    fields = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for did, name, values in rows:
            for v in values:
                w.writerow({"Correlation_Id": did, "Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


ROUTER = "void elb::(anonymous namespace)::router_mfma_kernel<4, true, false, 2, 4>(unsigned short const*, ...)"


def test_summarize_traffic_scales_and_averages_the_last_launches(tmp_path):
    mib = 4
    copy_kib = mib * 1024
    # Uploads (blits) first; then two step launches whose write counter also takes in another
    # kernel's write-back; then three back-to-back launches; then the three calibration copies,
    # whose counters read half (fetch) and exactly (write) the bytes moved.
    fetch_rows = [(1, "__amd_rocclr_copyBuffer", [10.0]), (2, "__amd_rocclr_copyBuffer", [20.0]),
                  (3, ROUTER, [500.0, 500.0]), (4, ROUTER, [500.0, 500.0]),
                  (5, ROUTER, [400.0, 600.0]), (6, ROUTER, [450.0, 550.0]), (7, ROUTER, [500.0, 500.0]),
                  (8, "__amd_rocclr_copyBuffer", [copy_kib / 2]), (9, "__amd_rocclr_copyBuffer", [copy_kib / 2]),
                  (10, "__amd_rocclr_copyBuffer", [copy_kib / 2])]
    write_rows = [(1, "__amd_rocclr_copyBuffer", [5.0]), (2, "__amd_rocclr_copyBuffer", [5.0]),
                  (3, ROUTER, [300.0]), (4, ROUTER, [300.0]),
                  (5, ROUTER, [100.0]), (6, ROUTER, [100.0]), (7, ROUTER, [100.0]),
                  (8, "__amd_rocclr_copyBuffer", [copy_kib]), (9, "__amd_rocclr_copyBuffer", [copy_kib]),
                  (10, "__amd_rocclr_copyBuffer", [copy_kib])]
    fpath, wpath = str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv")
    _counter_csv(fpath, "FETCH_SIZE", fetch_rows)
    _counter_csv(wpath, "WRITE_SIZE", write_rows)
    rec = bench.summarize_traffic(fpath, wpath, mib, T=123, launches=3)
    assert rec["T"] == 123 and rec["launches_averaged"] == 3
    assert rec["fetch_kib_per_launch"] == pytest.approx(1000.0)  # instances summed, last 3 launches
    assert rec["write_kib_per_launch"] == pytest.approx(100.0)   # the step launches are left out
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["traffic_bytes_per_launch"] == pytest.approx((1000.0 * 2.0 + 100.0) * 1024)
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()


def test_traffic_record_applies_only_to_its_source_and_size(tmp_path, monkeypatch):
    path = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.traffic_from_profile(65536) is None  # no record
    rec = {"kernel_source_sha256": bench.kernel_source_hash(), "T": 65536, "traffic_bytes_per_launch": 4.2e8}
    with open(path, "w") as f:
        json.dump(rec, f)
    assert bench.traffic_from_profile(65536) == pytest.approx(4.2e8)
    assert bench.traffic_from_profile(32768) is None  # another size
    rec["kernel_source_sha256"] = "0" * 64
    with open(path, "w") as f:
        json.dump(rec, f)
    assert bench.traffic_from_profile(65536) is None  # taken on another kernel source


def test_committed_traffic_record_is_near_the_algorithmic_bytes():
    """The record in profiles/ (when taken on the current router source): counted HBM bytes of a
    launch of its workload within 10% above its algorithmic bytes."""
    import datagen

    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec["kernel_source_sha256"] != bench.kernel_source_hash():
        pytest.skip("the traffic record predates the router source (the bench reports traffic null)")
    wl = datagen.WORKLOADS[rec.get("workload", "large")]
    assert wl.T == rec["T"]
    alg = bench.router_alg_bytes(wl.T, wl.d, wl.n_experts, wl.k)
    assert 1.0 <= rec["traffic_bytes_per_launch"] / alg < 1.1


def test_stress_workload_is_the_default_and_its_bytes():
    """The headline is the largest single-GPU workload: T = 262144, d = 4096 (2.158 GB per launch)."""
    import datagen

    wl = datagen.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (wl.T, wl.d, wl.n_experts, wl.k) == (262144, 4096, 256, 4)
    assert bench.router_alg_bytes(wl.T, wl.d, wl.n_experts, wl.k) == 2_157_971_456


def test_oracle_threads_follow_the_affinity_mask_and_the_host_share(monkeypatch):
    aff = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    assert bench.oracle_threads() == (aff, aff)
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.oracle_threads() == (1, aff)
    monkeypatch.setenv("OMP_NUM_THREADS", str(aff + 100))
    assert bench.oracle_threads() == (aff, aff)


def test_cpu_baseline_reports_cores_and_single_thread_samples():
    """The CPU leg on a small workload: all cores of the affinity mask, then one-thread samples."""
    import datagen

    wl = datagen.WORKLOADS["tiny"]
    res = bench.cpu_baseline(wl, datagen.tokens(wl), datagen.router_weight(wl), datagen.initial_bias(wl),
                             datagen.initial_momentum(wl), min_seconds=0.2, max_seconds=1.0, single_thread=False)
    assert res["kind"] == "oracle" and res["value"] > 0
    assert res["cores"] == bench.oracle_threads()[0] and res["affinity_cores"] == len(os.sched_getaffinity(0))

"""Host-side logic of bench.py, no GPU: the one-GPU guard and the conversion of rocprofv3
counter dumps into HBM bytes per launch (calibrated on a copy of known size)."""
import argparse
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _csv(path, rows):
    with open(path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for did, name, val in rows:
            f.write(f'{did},"{name}","X",{val}\n')


def test_traffic_from_scales_each_counter_by_the_calibration_copy(tmp_path):
    import bench
    kern = "void cpattn::(anonymous namespace)::bwd_fused_kernel<64, 4, 4, 2>(cpattn::BwdArgs, int, int, int, int)"
    copy = "__amd_rocclr_copyBuffer"
    mib512 = 512 * 1024  # KiB in 512 MiB
    # FETCH_SIZE reports half of what the copy reads; WRITE_SIZE all of what it writes
    _csv(tmp_path / "fetch.csv", [(1, kern, 1000.0), (2, kern, 1200.0), (3, copy, mib512 / 2), (4, copy, mib512 / 2),
                                  (5, copy, mib512 / 2)])
    _csv(tmp_path / "write.csv", [(1, kern, 300.0), (2, kern, 500.0), (3, copy, mib512), (4, copy, mib512),
                                  (5, copy, mib512)])
    out = tmp_path / "traffic.json"
    args = argparse.Namespace(workload="gpt2s", split_bwd=False, traffic=str(out), traffic_kernel=None,
                              traffic_from=[str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv")])
    bench.traffic_from(args)
    t = json.load(open(out))
    assert t["kernel"] == "block_bwd" and t["workload"] == "gpt2s"
    assert t["fetch"]["factor"] == pytest.approx(2.0) and t["write"]["factor"] == pytest.approx(1.0)
    assert t["fetch"]["bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 2)
    assert t["write"]["bytes_per_launch"] == pytest.approx(400.0 * 1024)
    assert t["bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 2 + 400.0 * 1024)
    assert t["source_hash"] == bench.kernel_source_hash("block_bwd")


def test_traffic_from_needs_the_calibration_copies(tmp_path):
    import bench
    _csv(tmp_path / "f.csv", [(1, "bwd_fused_kernel<64>", 1.0)])
    args = argparse.Namespace(workload="gpt2s", split_bwd=False, traffic=str(tmp_path / "t.json"),
                              traffic_kernel=None, traffic_from=[str(tmp_path / "f.csv"), str(tmp_path / "f.csv")])
    with pytest.raises(SystemExit):
        bench.traffic_from(args)


def test_source_hash_follows_the_kernel_sources():
    import bench
    # each kernel hashes its own device sources (and the shared headers), so the backward's
    # hash differs from the merge's
    assert bench.kernel_source_hash("block_bwd") != bench.kernel_source_hash("lse_merge")
    assert bench.kernel_source_hash("block_bwd") == bench.kernel_source_hash("block_bwd")


def test_traffic_of_the_forward_and_the_merge(tmp_path):
    import bench
    fwd = "void cpattn::(anonymous namespace)::fwd_bf16_kernel<128, 2, 1>(cpattn::FwdArgs, int)"
    mrg = "void cpattn::(anonymous namespace)::merge_kernel<128>(cpattn::MergeArgs)"
    copy = "__amd_rocclr_copyBuffer"
    mib512 = 512 * 1024
    for kern, name, wl in ((fwd, None, "win32k"), (mrg, "lse_merge", "merge_hbm_16k")):
        _csv(tmp_path / "f.csv", [(1, kern, 100.0), (2, kern, 300.0)] + [(3 + i, copy, mib512 / 2) for i in range(3)])
        _csv(tmp_path / "w.csv", [(1, kern, 50.0), (2, kern, 50.0)] + [(3 + i, copy, mib512) for i in range(3)])
        out = tmp_path / "t.json"
        args = argparse.Namespace(workload="win32k", split_bwd=False, traffic=str(out), traffic_kernel=name,
                                  traffic_from=[str(tmp_path / "f.csv"), str(tmp_path / "w.csv")])
        bench.traffic_from(args)
        t = json.load(open(out))
        assert t["kernel"] == (name or "block_fwd") and t["workload"] == wl
        assert t["bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2 + 50.0 * 1024)


def test_kernel_families_pool_the_forward_launches():
    import bench
    s = {"block_fwd": {"bound": "mfma", "launches": 2, "total_ms": 2.0, "work_per_launch": 1e12,
                       "unit": "TFLOP/s", "peak": 2500.0},
         "block_fwd_merge": {"bound": "mfma", "launches": 2, "total_ms": 1.0, "work_per_launch": 0.5e12,
                             "unit": "TFLOP/s", "peak": 2500.0},
         "rope_rotate": {"bound": "hbm", "launches": 6, "total_ms": 0.2, "work_per_launch": 1e8,
                         "unit": "GB/s", "peak": 8000.0}}
    fam = bench.EventLog().families(s)
    f = fam["block_fwd"]
    assert f["launches"] == 4 and f["total_ms"] == pytest.approx(3.0)
    assert f["achieved"] == pytest.approx(3e12 / 3e-3 / 1e12)  # total work over total time
    assert f["avg_us"] == pytest.approx(750.0) and f["work_per_launch"] == pytest.approx(0.75e12)
    assert fam["rope_rotate"]["achieved"] == pytest.approx(6e8 / 0.2e-3 / 1e9)


def test_headline_is_the_32k_window_forward():
    import bench
    from workloads import BY_NAME
    args = bench.argparse.Namespace(bwd="auto")
    assert bench.HEADLINE == "win32k"
    assert not bench._do_bwd(args, BY_NAME["win32k"]) and bench._do_bwd(args, BY_NAME["gpt2s"])
    assert bench.DOMINANT["win32k"] == "block_fwd"


@pytest.mark.parametrize("name", ["traffic_block_fwd_win32k.json", "traffic_block_bwd_bwd16k.json",
                                  "traffic_merge_hbm_16k.json", "traffic_block_bwd_gpt2s.json"])
def test_committed_traffic_matches_the_kernel_sources(name):
    """The HBM bytes committed for the headline kernel, the backward kernels and the merge were
    counted on the sources as they stand: a kernel edited since then needs its counters taken
    again (the bench line would otherwise report no traffic)."""
    import bench
    t = json.load(open(os.path.join(ROOT, "profiles", name)))
    assert t["source_hash"] == bench.kernel_source_hash(t["kernel"]), name
    assert t["bytes_per_launch"] > 0

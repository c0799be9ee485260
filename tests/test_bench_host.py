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
    args = argparse.Namespace(workload="gpt2s", split_bwd=False, traffic=str(out),
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
                              traffic_from=[str(tmp_path / "f.csv"), str(tmp_path / "f.csv")])
    with pytest.raises(SystemExit):
        bench.traffic_from(args)


def test_source_hash_follows_the_kernel_sources():
    import bench
    # each kernel hashes its own device sources (and the shared headers), so the backward's
    # hash differs from the merge's
    assert bench.kernel_source_hash("block_bwd") != bench.kernel_source_hash("lse_merge")
    assert bench.kernel_source_hash("block_bwd") == bench.kernel_source_hash("block_bwd")

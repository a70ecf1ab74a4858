"""Host-side pieces of bench.py that need no GPU: the one-GPU guard, the
scaling of the HBM byte counters, and the kernel-source check that keeps a
stale traffic record out of the bench line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""  # no bench line


def _csv(path, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for k, c, v in rows:
            f.write(f'"{k}",{c},{v}\n')


def test_pmc_summary_scales_each_counter_by_its_calibration_copy(tmp_path):
    # The calibration copy moves CALIB_BYTES; a counter that reads half of that
    # for it is scaled by 2, one that reads all of it by 1.  Only the largest
    # copy dispatch is the calibration; other copies and kernels are ignored.
    half_kib = bench.CALIB_BYTES // 2048
    full_kib = bench.CALIB_BYTES // 1024
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _csv(fetch, [("void moe::k_moe_layer<1, true, 4>(moe::LayerParams)", "FETCH_SIZE", 100.0),
                 ("void moe::k_moe_layer<1, true, 4>(moe::LayerParams)", "FETCH_SIZE", 300.0),
                 ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 10.0),
                 ("__amd_rocclr_copyBuffer", "FETCH_SIZE", float(half_kib)),
                 ("other_kernel", "FETCH_SIZE", 5e6)])
    _csv(write, [("void moe::k_moe_layer<1, true, 4>(moe::LayerParams)", "WRITE_SIZE", 40.0),
                 ("void moe::k_moe_layer<1, true, 4>(moe::LayerParams)", "WRITE_SIZE", 60.0),
                 ("__amd_rocclr_copyBuffer", "WRITE_SIZE", float(full_kib))])
    s = bench.pmc_summary(str(fetch), str(write))
    assert s["fetch_scale"] == pytest.approx(2.0)
    assert s["write_scale"] == pytest.approx(1.0)
    assert s["fetch_bytes"] == 200 * 1024 * 2
    assert s["write_bytes"] == 50 * 1024
    assert s["traffic_bytes_per_launch"] == 200 * 1024 * 2 + 50 * 1024
    assert s["dispatches"] == 2
    assert s["kernel_source_hash"] == bench.kernel_source_hash()


def test_traffic_record_is_used_only_for_the_same_kernel_sources(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.txt"
    rec.write_text("# header\ntraffic_bytes_per_launch = 12345\nkernel_source_hash = %s\n" % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic() == 12345
    rec.write_text("# header\ntraffic_bytes_per_launch = 12345\nkernel_source_hash = 0000000000000000\n")
    assert bench.recorded_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.recorded_traffic() is None


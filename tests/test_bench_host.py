"""Host logic of bench.py (no GPU): the one-GPU rule, the counter-to-traffic
conversion and the kernel-source hash that ties profiles/traffic.json to the
sources it was measured on."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_counters(tmp_path, monkeypatch):
    """Counters in KiB per dispatch, scaled so the calibration copy moves CALIB_BYTES,
    averaged per kernel and summed per entry point; entry points absent from the run
    are left out."""
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    calib_kib = bench.CALIB_BYTES / 1024
    lm = "void qg::k_affine<8, 2, true, true>(QgAffineArgs)"
    fin = "qg::k_lmhead_finalize(QgAffineArgs, int)"
    moe_gu, moe_dn = "qg::k_moe_gateup(QgMoeArgs)", "qg::k_moe_down(QgMoeArgs)"
    fetch = [("void at::native::elementwise_kernel<bitwise_not>", calib_kib / 2)] * 2 + [
        (lm, 40000.0), (lm, 42000.0), (fin, 20.0), (moe_gu, 7000.0), (moe_dn, 3500.0)]
    write = [("void at::native::elementwise_kernel<bitwise_not>", calib_kib)] + [
        (lm, 16.0), (fin, 0.0), (moe_gu, 6.0), (moe_dn, 2.0)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    t = json.loads(out.read_text())
    assert t["fetch_factor"] == pytest.approx(2.0) and t["write_factor"] == pytest.approx(1.0)
    assert t["source_hash"] == bench.kernel_source_hash()
    lmh = t["kernels"]["lmhead_argmax"]
    assert lmh["kernels"][lm] == {"fetch_bytes": round(41000.0 * 1024 * 2), "write_bytes": 16 * 1024}
    assert lmh["bytes_per_launch"] == round((41000.0 * 2 + 16 + 20.0 * 2) * 1024)
    assert t["kernels"]["moe_expert_qgemv"]["bytes_per_launch"] == round((7000 * 2 + 6 + 3500 * 2 + 2) * 1024)
    assert "mlp_block" not in t["kernels"] and "qgemv_affine4" not in t["kernels"]


def test_traffic_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [("qg::k_moe_down(QgMoeArgs)", 1.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [("qg::k_moe_down(QgMoeArgs)", 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))


def test_source_hash_covers_every_kernel_source():
    """Every HIP source and header the library is built from takes part in the hash, so a
    changed kernel invalidates the stored traffic figures."""
    from bit_quantized_decode_group_amd import build
    hashed = {os.path.basename(p) for p in bench.KERNEL_SOURCES}
    csrc = os.path.join(ROOT, "bit_quantized_decode_group_amd", "csrc")
    on_disk = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))}
    assert set(build.SOURCES) <= hashed
    assert on_disk <= hashed

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
    lm = "void qg::k_affine<8, 2, true, true, false>(QgAffineArgs)"
    lm_topk = "void qg::k_affine<8, 2, true, true, true>(QgAffineArgs)"  # the top-k projection: not the greedy entry
    fin = "qg::k_lmhead_finalize(QgAffineArgs, int)"
    moe_gu, moe_dn = "qg::k_moe_gateup(QgMoeArgs)", "qg::k_moe_down(QgMoeArgs)"
    fetch = [("void at::native::elementwise_kernel<bitwise_not>", calib_kib / 2)] * 2 + [
        (lm_topk, 99000.0), (lm, 40000.0), (lm, 42000.0), (fin, 20.0), (moe_gu, 7000.0), (moe_dn, 3500.0)]
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
    assert lmh["bytes_per_launch"] == round((41000.0 * 2 + 16) * 1024)  # one kernel: the finish is fused
    assert fin not in lmh["kernels"]
    assert t["kernels"]["moe_expert_qgemv"]["bytes_per_launch"] == round((7000 * 2 + 6 + 3500 * 2 + 2) * 1024)
    assert "mlp_block" not in t["kernels"] and "qgemv_affine4" not in t["kernels"]
    # an M = 1 pass fills its own table and keeps the M = 8 one
    lm1 = "void qg::k_affine<1, 2, true, true, false>(QgAffineArgs)"
    _counter_csv(tmp_path / "f1.csv", "FETCH_SIZE",
                 [("void at::native::elementwise_kernel<bitwise_not>", calib_kib / 2), (lm1, 40500.0)])
    _counter_csv(tmp_path / "w1.csv", "WRITE_SIZE",
                 [("void at::native::elementwise_kernel<bitwise_not>", calib_kib), (lm1, 2.0)])
    bench.traffic_from_counters(str(tmp_path / "f1.csv"), str(tmp_path / "w1.csv"), M=1)
    t = json.loads(out.read_text())
    assert t["kernels_m1"]["lmhead_argmax"]["bytes_per_launch"] == round((40500.0 * 2 + 2) * 1024)
    assert t["kernels"]["lmhead_argmax"]["bytes_per_launch"] == round((41000.0 * 2 + 16) * 1024)


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


def test_kernel_times_from_stats(tmp_path, monkeypatch):
    """rocprofv3 kernel_stats.csv averages (ns) become per-entry-point kernel-only times (us)."""
    out = tmp_path / "kt.json"
    monkeypatch.setattr(bench, "KERNEL_TIMES_FILE", str(out))
    stats = tmp_path / "kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs"])
        w.writeheader()
        w.writerow({"Name": "void qg::k_affine<8, 2, true, true, false>(QgAffineArgs)", "Calls": 10,
                    "TotalDurationNs": 210000, "AverageNs": 21000.0})
        w.writerow({"Name": "void qg::k_affine<8, 0, true, true, false>(QgAffineArgs)", "Calls": 10,
                    "TotalDurationNs": 80000, "AverageNs": 8000.0})
        w.writerow({"Name": "void qg::k_split_reduce<0>(QgAffineArgs)", "Calls": 10,
                    "TotalDurationNs": 33000, "AverageNs": 3300.0})
    bench.kernel_times_from_stats(str(stats))
    t = json.loads(out.read_text())
    assert t["source_hash"] == bench.kernel_source_hash()
    assert t["entries"]["lmhead_argmax"]["kernel_us_m8"] == pytest.approx(21.0)
    assert t["entries"]["qgemv_affine4"]["kernel_us_m8"] == pytest.approx(11.3)
    assert "moe_expert_qgemv" not in t["entries"]


def test_oracle_all_cores_build_gives_the_same_bits():
    """The CPU baseline's all-cores oracle (OpenMP over output rows) returns exactly the
    single-threaded oracle's results."""
    import numpy as np

    import oracle
    from bit_quantized_decode_group_amd import synth
    d = synth.lm_head(M=4, V=3000, K=512, seed=77)
    m = synth.moe_token(E=8, D=256, I=256, top_k=2, seed=78)
    b = synth.mlp_block(M=3, D=512, I=512, seed=79)
    def run():
        return (oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"], draft=d["draft"][:4]),
                oracle.moe(m["x"], m["logits"][0], 2, m["w_gu"], m["w_down"], 8, 256, 256),
                oracle.mlp_block(b["x"], b["gamma"], b["eps"], b["codes_gu"], b["scales_gu"], b["biases_gu"],
                                 b["codes_d"], b["scales_d"], b["biases_d"]))
    try:
        assert oracle.use_threads(1) == 1
        one = run()
        assert oracle.use_threads(4) >= 1
        many = run()
    finally:
        oracle.use_threads(1)
    (l1, i1, g1, a1), (y1, e1, p1), z1 = one
    (l2, i2, g2, a2), (y2, e2, p2), z2 = many
    assert np.array_equal(l1, l2) and np.array_equal(i1, i2) and np.array_equal(g1, g2) and a1 == a2
    assert np.array_equal(y1, y2) and np.array_equal(e1, e2) and np.array_equal(p1, p2)
    assert np.array_equal(z1, z2)

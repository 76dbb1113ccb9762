"""Host logic of the HBM traffic summary: copy calibration and per-kernel scaling."""
import csv
import json
import os

from jagged_attention_recommendation_amd import counters

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def write_run(path, counter, rows):
    path.mkdir()
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, (k, v) in enumerate(rows, 1):
            # two dimension rows per dispatch, summed by the reader
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Grid_Size": 1, "Counter_Name": counter,
                        "Counter_Value": v / 2})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Grid_Size": 1, "Counter_Name": counter,
                        "Counter_Value": v / 2})


def test_summary_scales_by_the_copy(tmp_path):
    kib = (256 << 20) / 1024
    write_run(tmp_path / "f", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1.0)] +
              [("__amd_rocclr_copyBuffer", kib / 2)] * 3 +
              [("void gdpa::bwddl::dq_dl_kernel<0, true, true>(gdpa::BwdArgs)", 1000.0)] * 2)
    write_run(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 0.0)] +
              [("__amd_rocclr_copyBuffer", kib)] * 3 +
              [("void gdpa::bwddl::dq_dl_kernel<0, true, true>(gdpa::BwdArgs)", 300.0)] * 2)
    s = counters.summarize(tmp_path / "f", tmp_path / "w")
    assert s["fetch_scale"] == 2.0 and s["write_scale"] == 1.0
    assert s["kernels"]["dq"] == {"dispatches": 2, "fetch_kib": 1000.0, "write_kib": 300.0,
                                  "bytes": 1000 * 1024 * 2 + 300 * 1024}
    assert s["csrc_sha256"] == counters.csrc_digest()
    p = tmp_path / "summary.txt"
    p.write_text("# header\njson: " + json.dumps(s) + "\n")
    assert counters.load_summary(p) == s


def test_kernel_bytes_count_each_operand_once():
    """Per-kernel algorithmic bytes: the tensors each kernel reads and writes, counted by hand."""
    from jagged_attention_recommendation_amd import inputs, workload
    import numpy as np
    lq, lk = np.array([5, 9]), np.array([3, 7])
    for act in ("softmax", "silu"):
        p = inputs.make_problem("kb", seed=1, H=2, D=32, lq=lq, lk=lk, dtype="bf16", act=act,
                                causal=False, bias_buckets=0)
        tq, tk, row = 14, 10, 2 * 32 * 2  # rows of Q and of K; bytes of one row (H x D bf16)
        sm = act == "softmax"
        assert workload.kernel_bytes(p, "fwd") == workload.fwd_bytes(p)
        # dQ: Q, dO, K, V read, dQ written; softmax adds O (for D), lse, and the D vector written
        dq = (2 * tq + 2 * tk) * row + tq * row + (tq * row + 2 * tq * 2 * 4 if sm else 0)
        # dK/dV: Q, dO, K, V read, dK, dV written; softmax adds lse and D read
        dkdv = (2 * tq + 2 * tk) * row + 2 * tk * row + (2 * tq * 2 * 4 if sm else 0)
        assert workload.kernel_bytes(p, "dq") == dq
        assert workload.kernel_bytes(p, "dkdv") == dkdv


def test_sq_summary_mfma_busy(tmp_path):
    """Shader-sequencer summary: SQ counters summed over instances, GRBM clock maxed, and the
    MFMA busy fraction over all 1024 SIMDs against the clock of one XCD (GRBM_GUI_ACTIVE sums
    the 8 XCDs' clocks)."""
    d = tmp_path / "sq"
    d.mkdir()
    rows = []
    for disp, kern in ((1, "void gdpa::fwdk::fwd_kernel<64, 2, false, false, false>(gdpa::FwdArgs)"),
                       (2, "void gdpa::fwdk::fwd_kernel<64, 2, false, false, false>(gdpa::FwdArgs)")):
        for inst in range(2):
            rows.append({"Dispatch_Id": disp, "Kernel_Name": kern, "Grid_Size": 1,
                         "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 1024 * 50})
            rows.append({"Dispatch_Id": disp, "Kernel_Name": kern, "Grid_Size": 1,
                         "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1000})
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        w.writerows(rows)
    s = counters.summarize_sq(d)
    assert s["fwd"]["dispatches"] == 2
    assert s["fwd"]["GRBM_GUI_ACTIVE"] == 1000 and s["fwd"]["SQ_VALU_MFMA_BUSY_CYCLES"] == 1024 * 100
    assert s["fwd"]["mfma_busy_pct"] == 80.0  # 1024 * 100 / (1000 / 8 * 1024)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU; --gpus N > 1 exits with a message before touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr

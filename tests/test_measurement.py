"""CPU tests of the measurement tooling: the rocprofv3 summaries
(profsummary.py) and the sampled-oracle parity check recorded in every bench
row (bench.parity_sample).  A mistake in either would change reported numbers
without failing any GPU test, so each is run here on inputs whose answer is
known."""
import csv
import json

import numpy as np
import pytest

import profsummary


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_traffic_scales_counters_by_the_copy(tmp_path):
    # counters in KiB per dispatch; the 1 GiB copy reads FETCH_SIZE = 2 GiB and
    # WRITE_SIZE = 1 GiB, so fetch bytes are halved and write bytes kept
    gib_kib = 1 << 20
    copy, gemm, lse = "__amd_rocclr_copyBuffer", "void ckl::gemm_store_kernel<x>(y)", "void ckl::fwd_lse_kernel<x>(y)"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(tmp_path / "fetch.csv", hdr, [
        [1, gemm, "FETCH_SIZE", 4 * gib_kib], [2, gemm, "FETCH_SIZE", 2 * gib_kib],
        [3, lse, "FETCH_SIZE", gib_kib], [4, copy, "FETCH_SIZE", 2 * gib_kib]])
    _write_csv(tmp_path / "write.csv", hdr, [
        [1, gemm, "WRITE_SIZE", gib_kib // 2], [2, gemm, "WRITE_SIZE", gib_kib // 2],
        [3, lse, "WRITE_SIZE", 0], [4, copy, "WRITE_SIZE", gib_kib]])
    out = tmp_path / "traffic.json"
    json.dump({"entries": [{"workload": "w", "path": "fused", "stale": True},
                           {"workload": "w", "path": "recompute", "kept": True}]}, open(out, "w"))
    profsummary.traffic(str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"), str(out), "w", "fused", 2)
    doc = json.load(open(out))
    entries = {e["path"]: e for e in doc["entries"]}
    assert entries["recompute"] == {"workload": "w", "path": "recompute", "kept": True}  # other entries kept
    e = entries["fused"]
    assert "stale" not in e and e["steps_profiled"] == 2
    assert e["copy_scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    g = e["kernels"]["gemm_dhdw"]
    assert g["launches"] == 2
    assert g["hbm_read_bytes_per_launch"] == pytest.approx(1.5 * 2**30)  # mean of 4 and 2 GiB, halved
    assert g["hbm_write_bytes_per_launch"] == pytest.approx(0.5 * 2**30)
    assert g["hbm_bytes_per_launch"] == pytest.approx(2.0 * 2**30)
    assert e["kernels"]["fwd_lse"]["hbm_read_bytes_per_launch"] == pytest.approx(0.5 * 2**30)
    assert "copy" not in e["kernels"]


def test_traffic_refuses_a_run_without_the_copy(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(tmp_path / "f.csv", hdr, [[1, "ckl::gemm_store_kernel", "FETCH_SIZE", 10]])
    _write_csv(tmp_path / "w.csv", hdr, [[1, "ckl::gemm_store_kernel", "WRITE_SIZE", 10]])
    with pytest.raises(SystemExit):
        profsummary.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "t.json"), "w", "p", 1)


def test_trace_groups_kernel_classes(tmp_path):
    _write_csv(tmp_path / "stats.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"], [
        ["void ckl::fwd_lse_kernel<a, true>(b)", 2, 3_000_000, 1_500_000, 1_000_000, 2_000_000],
        ["void ckl::gemm_store_kernel<c>(d)", 1, 1_000_000, 1_000_000, 1_000_000, 1_000_000],
        ["some_other_library_kernel", 5, 9_000_000, 1_800_000, 1, 2]])
    out = tmp_path / "t.md"
    profsummary.trace(str(tmp_path / "stats.csv"), str(out), "cmd")
    text = out.read_text()
    assert "| fwd_lse | 2 | 3.000 | 1.5000 | 75.0% |" in text  # foreign kernels are not in the shares
    assert "| gemm_dhdw | 1 | 1.000 | 1.0000 | 25.0% |" in text
    assert "| foreign |" not in text


def test_counters_clock_busy_and_rate(tmp_path):
    # one 1 ms dispatch at 1.7 GHz (GRBM_GUI_ACTIVE sums the 8 XCDs), MFMA
    # pipes busy half of the 1024 SIMDs' cycles, 1e12 flop of bf16 MFMA work
    cyc = 1.7e9 * 1e-3
    rows = [[7, "void ckl::fwd_lse_kernel<a>(b)", name, val, 0, 1_000_000] for name, val in (
        ("GRBM_GUI_ACTIVE", 8 * cyc), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * 1024),
        ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e12 / 512))]
    _write_csv(tmp_path / "c.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                     "Start_Timestamp", "End_Timestamp"], rows)
    out = tmp_path / "c.md"
    profsummary.counters(str(out), "title", [(str(tmp_path / "c.csv"), "cmd")])
    assert "| fwd_lse | 1 | 1.000 | 1.70 | 50.0% | 1000 | - | - | - |" in out.read_text()


def _oracle_step(x):
    import oracle
    ref = oracle.kl_dense(x.H, x.W, x.idx, x.tlogit, mask=x.mask)
    return dict(loss=ref["loss"], lse=ref["lse"].copy(), row_loss=ref["row_loss"].copy(),
                dH=ref["dH"].copy(), dW=ref["dW"].copy())


def test_bench_parity_check_passes_exact_and_catches_errors():
    import bench
    from synth import make_inputs
    x = make_inputs(0, seed=3)  # tiny fp32 workload: tolerances 1e-5
    got = _oracle_step(x)
    r = bench.parity_sample(x, got)
    assert r["pass"] and r["dH_rel_err"] < 1e-12 and r["dW_rel_err"] < 1e-9
    assert 0 in r["rows"] and x.T - 1 in r["rows"] and 0 in r["vocab_rows"] and x.V - 1 in r["vocab_rows"]
    # an error of 1e-3 of the largest entry in one sampled dW row, one sampled
    # dH row, one sampled LSE, or in the loss, each fails the check
    for key in ("dW", "dH", "lse", "loss"):
        bad = _oracle_step(x)
        if key == "loss":
            bad["loss"] *= 1 + 1e-3
        elif key == "lse":
            bad["lse"][r["rows"][-1]] += 1e-2
        else:
            row = (r["vocab_rows"] if key == "dW" else r["rows"])[-1]
            bad[key][row, 0] += 1e-3 * np.abs(bad[key]).max()
        assert not bench.parity_sample(x, bad)["pass"], key


def test_matrix_records_failed_cases_and_goes_on():
    # each case runs in a child process; here (no GPU) every child fails, and
    # each failure becomes a FAILED row with its error while the sweep goes on
    import argparse
    import torch

    import bench
    if torch.cuda.is_available():
        pytest.skip("needs a machine without a GPU: the children must fail")
    args = argparse.Namespace(steps=1, warmup=0, min_time=0.0, case_timeout=120)
    r = bench.matrix(args, cases=[(1, None), (4, 512)])
    assert r["isolation"] == "one child process per (workload, chunk, path)"
    rows = r["matrix"]
    assert [(x["workload"], x["chunk"], x["path"]) for x in rows] == [
        ("small-bf16", 1024, "fused"), ("small-bf16", 1024, "recompute"),
        ("t256k-v201k-packed-bf16", 512, "fused"), ("t256k-v201k-packed-bf16", 512, "recompute")]
    assert all(x["status"] == "FAILED" and "needs a GPU" in x["error"] for x in rows)

"""Host-side logic of bench.py (no GPU): the one-GPU contract, the
algorithmic byte / FLOP counts behind the roofline figures, and the profile
summarizer on synthetic rocprofv3 CSV files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from linear_recurrent_sequence_shortconv_amd.workloads import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_counts_cover_every_timed_kernel():
    w = workloads()["lm-T2048"]
    c = bench.algorithmic_counts(w)
    timer_names = {n for _, names in bench._FAMILIES for n in names} | {
        "chunk_fwd", "chunk_fwd_bwdmode", "chunk_fwd_fused"}
    assert timer_names <= set(c), timer_names - set(c)
    for name, v in c.items():
        assert v["bytes"] > 0 and v["flops"] >= 0 and v["floor_ms"] > 0, name
        assert v["bound"] in ("hbm", "mfma")
    # per token-head, the refinement forward moves e (d + 2 L d) bytes
    th = w.B * w.T * w.H
    assert c["refine_fwd"]["bytes"] == th * 2 * w.d + w.B * w.T * w.H * 2 * w.L * w.d * 2
    # the decode state kernel reads and writes the fp32 state: 8 d^2 bytes per sequence-head
    dec = bench.decode_counts(w)
    assert dec["step_state"][0] > bench.DECODE_BATCH * w.H * 8 * w.d * w.d


def test_kernel_names_map_to_timer_names():
    assert bench._family("_ZN5prism17refine_bwd_kernelIDF16bLi128ELi4ELi0ELi0EEEv") == ["refine_bwd"]
    assert bench._family("_ZN5prism17state_pass_kernelIDF16bLi128ELi64ELb0ELi64EEEvPKf") == ["state_fwd"]
    assert bench._family("_ZN5prism17state_pass_kernelIDF16bLi128ELi64ELb0ELi0EEEvPKf") == ["state_fwd_recompute"]
    assert bench._family("_ZN5prism17state_pass_kernelIDF16bLi128ELi16ELb1ELi0EEEvPKf") == ["state_bwd_stateless"]
    assert bench._family("_ZN5prism17state_pass_kernelIDF16bLi128ELi64ELb1ELi64EEEvPKf") == ["state_bwd"]
    assert bench._family("void prism::state_pass_kernel<__bf16, 128, 64, false, 64>(float const*)") == ["state_fwd"]
    cf = "_ZN5prism16chunk_fwd_kernelIDF16bLi128ELi64ELb{}ELb{}ELi0ELi1EEEvPKT_S3_"
    assert bench._family(cf.format(1, 0)) == ["chunk_fwd_bwdmode"]
    assert bench._family(cf.format(0, 0)) == ["chunk_fwd"]
    assert bench._family(cf.format(0, 1)) == ["chunk_fwd_fused"]
    assert bench._family("void prism::chunk_fwd_kernel<__bf16, 128, 64, false, true, 0, 0>(...)") == [
        "chunk_fwd_fused"]
    assert bench._family("void prism::chunk_fwd_kernel<__bf16, 128, 64, true, false, 0, 0>(...)") == [
        "chunk_fwd_bwdmode"]
    assert bench._family("_ZN5prism17step_state_kernelIDF16bLi128EEEv") == ["step_state"]
    assert bench._family("some_other_kernel") is None


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_summarize_profiles_scales_counters_by_the_copy(tmp_path, monkeypatch):
    d = str(tmp_path)
    k = "_ZN5prism19wgrad_reduce_kernelEPKfPfS2_iiii"
    # copy: FETCH reads half of 1 GiB (KiB), WRITE all of it
    _write_csv(os.path.join(d, "cfetch", "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Value"], [["copy", (1 << 30) / 1024 / 2]])
    _write_csv(os.path.join(d, "cwrite", "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Value"], [["copy", (1 << 30) / 1024]])
    _write_csv(os.path.join(d, "fetch", "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Value"], [[k, 1000.0], [k, 1000.0]])
    _write_csv(os.path.join(d, "write", "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Value"], [[k, 500.0]])
    _write_csv(os.path.join(d, "trace", "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs"], [[k, 4, 400000]])
    # matrix-core pass: 1e6 MOPS = 512 MFLOP in 100 us; busy 1000 cycles per
    # SIMD out of 4000 active cycles per XCD
    mc = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(os.path.join(d, "mfma", "run_counter_collection.csv"), mc,
               [[k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6], [k, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0],
                [k, "SQ_VALU_MFMA_BUSY_CYCLES", 1000.0 * 1024], [k, "GRBM_GUI_ACTIVE", 8 * 4000.0]])
    out = tmp_path / "repo"
    (out / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(out))
    monkeypatch.setattr(bench, "_sources_sha256", lambda: "sha")
    bench.summarize_profiles(d, "lm-T2048")
    rec = json.load(open(out / "profiles" / "hbm_traffic.json"))
    assert abs(rec["calibration"]["fetch_factor"] - 2.0) < 1e-9
    assert abs(rec["calibration"]["write_factor"] - 1.0) < 1e-9
    t = rec["kernels"]["wgrad_reduce"]
    assert t["fetch_bytes"] == 2 * 1000 * 1024 and t["write_bytes"] == 500 * 1024
    md = open(out / "profiles" / "lm-T2048_kernels.md").read()
    assert "| wgrad_reduce | 4 | 100.0 |" in md
    # 0.512 GFLOP; 5.12 TFLOP/s; 0.512e9 / 2.5e15 / 1e-4 s = 0.002048 of the bf16 pipe
    assert "| wgrad_reduce | 0.5 | 0.00 |" in md and "| 5 | 0.002 | 0.250 |" in md


def test_cpu_baseline_process_pool():
    """The oracle baseline runs whole sequences in a pool of spawned worker
    processes and reports the workers it used and the CPU model."""
    import bench
    from linear_recurrent_sequence_shortconv_amd.workloads import make_workload_inputs, workloads
    w = workloads()["tiny-fp32"]
    x = make_workload_inputs(w, seed=0)
    r = bench.cpu_baseline(w, x, budget_s=0.5, backward=True, max_workers=2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 2 and isinstance(r["cpu_model"], str) and r["cpu_model"]
    assert "1 of 1 (b,h) sequences" in r["sample"]


def test_stage_fractions():
    import bench
    from linear_recurrent_sequence_shortconv_amd.workloads import workloads
    w = workloads()["lm-T2048"]
    counts = bench.algorithmic_counts(w)
    kernels = {n: {"total_ms": 0.5, "launches_per_step": 1} for n in
               bench.SCAN_KERNELS + bench.REFINE_KERNELS}
    st = bench.stage_fractions(kernels, counts, "bf16")
    fl = sum(counts[n]["flops"] for n in bench.SCAN_KERNELS)
    t = 0.5e-3 * len(bench.SCAN_KERNELS)
    assert abs(st["scan"]["mfma_frac"] - fl / t / 2.5e15) < 1e-4
    by = sum(counts[n]["bytes"] for n in bench.REFINE_KERNELS)
    t = 0.5e-3 * len(bench.REFINE_KERNELS)
    assert abs(st["refinement"]["hbm_frac"] - by / t / 8e12) < 1e-4
    assert st["scan"]["target_mfma_frac"] == 0.40 and st["refinement"]["target_hbm_frac"] == 0.60

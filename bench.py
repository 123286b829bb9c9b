"""Benchmark of the PRISM layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload lm-T2048]

One step = one pass of the whole hot path over one batch of synthetic input
with the inputs already resident in HBM: the training forward (ShortConv
anchor, L refinement steps, chunked scan, readout, final state; it keeps the
intermediates the backward needs) followed by the training backward (every
input and weight gradient).  The stateless pair (prism_forward +
prism_backward, which recomputes the forward) is timed as well and reported
beside it.  The default workload is the language-model layer shape: B=8, H=16,
T=2048, d_k=d_v=128, L=3, chunk 64, bf16 storage with fp32 accumulation.

Prints one JSON line.  Besides the throughput it reports, for the kernel with
the largest share of the step, its achieved rate against the MI355X peak
(HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s), using algorithmic bytes / FLOPs
per launch divided by the HIP-event-measured average launch duration; and
the float64 oracle timed on a bounded sample on the host CPU.

--calibrate-copy runs only a plain 1 GiB device copy (for scaling HBM byte
counters of rocprofv3 runs) and exits.
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3


def algorithmic_counts(w):
    """Algorithmic bytes and FLOPs per launch of each kernel for workload w.

    Bytes count each tensor once at its storage size (e = 2 for bf16; fp32
    intermediates at 4): what the kernel must read and write, not what it
    happens to re-read.  FLOPs count the dense matrix products of the
    algorithm (2 m n k each); the extra product of the hi/lo split of the
    anchor is an accuracy device and is not counted.  "bound" is the roof
    the kernel would hit first at MI355X peak rates.
    """
    B, T, H, D, L, C = w.B, w.T, w.H, w.d, w.L, w.chunk
    e = 2 if w.dtype == "bf16" else 4
    NC = -(-T // C)
    Tp = NC * C
    th = B * T * H                 # token-heads
    ntp = B * Tp * H               # padded token-heads (workspace rows)
    nch = B * H * NC               # chunks
    bh = B * H
    c = {}
    c["refine_fwd"] = (th * e * D + ntp * 2 * L * D * e, th * 4 * L * D * D)
    # (the training forward also keeps U^T, W_k^T: + 2 C D e per chunk)
    c["chunk_fwd"] = (th * (3 * D * e + 8) + ntp * 2 * L * D * e
                      + nch * (2 * D * D * e + 2 * C * D * e + 4 + 2 * C * D * e),
                      nch * (2 * C * C * D * (4 * L + 6) + 2 * C * D * D * (L + 2)))
    # refinement formed inside the chunk kernel (inference forward): no pairs
    # in HBM; weights and taps once per head
    c["chunk_fwd_fused"] = (th * (3 * D * e + 8) + H * (L * (2 * D * D + D) + 4 * D) * e
                            + nch * (2 * D * D * e + 2 * C * D * e + 4),
                            nch * (2 * C * C * D * (4 * L + 6) + 2 * C * D * D * (L + 2))
                            + th * 4 * L * D * D)
    # products per chunk: C x C x D ones K K^T, K Q^T, T V, T K, R0 Wk^T and,
    # per step, K_l K^T and F W_l; D x D x C ones H, M, E and, per step, H's W_l part
    c["chunk_fwd_bwdmode"] = (th * (4 * D * e + 8) + ntp * 2 * L * D * e
                              + nch * (4 * D * D * e + 2 * C * D * e + 4),
                              nch * (2 * C * C * D * (2 * L + 5) + 2 * C * D * D * (L + 3)))
    # state pass: read M^T, H^T, write S_c (kept by the training forward), S0 /
    # S_T; the forward pass also forms the readout: read Qt, O_loc, write o
    st = (nch * D * D * 3 * e + bh * D * D * 4, nch * 2 * D ** 3)
    c["state_fwd"] = (st[0] + nch * C * D * 2 * e + th * D * e, st[1] + nch * 2 * C * D * D)
    c["state_fwd_recompute"] = st
    # reverse pass: read M, write dS_c^T, dS_T / dS_0; after a training forward
    # it forms E_c = dO^T Qt itself (read dO, Qt), otherwise it reads E^T
    c["state_bwd_stateless"] = (st[0] + bh * D * D * 4, st[1])
    c["state_bwd"] = (nch * D * D * 2 * e + bh * D * D * 8 + nch * C * D * e + th * D * e,
                      st[1] + nch * 2 * C * D * D)
    c["chunk_bwd_state"] = (th * (2 * D * e + 4) + nch * (2 * C * D * e + 2 * D * D * e + 4 * e * C * D + 4 * C)
                            + ntp * L * D * (3 * e + 4),  # read K_l, W_l; write dK_l, dW_l (fp32) partials
                            # C x D x D products dQt, U dS_n, K dS_n^T, K dM^T, Wk dM and
                            # two per step; the D x D x D one dM
                            nch * (2 * C * D * D * (5 + 2 * L) + 2 * D ** 3))
    c["chunk_bwd_solve"] = (th * (4 * D * e + 12) + ntp * 2 * L * D * e + nch * (7 * e * C * D + 8 * C),
                            nch * (2 * C * C * D * (2 * L + 16) + 4 * C ** 3))
    c["chunk_bwd_pairs"] = (th * (5 * D * e + 8) + ntp * 2 * L * D * e + nch * 3 * e * C * D
                            + ntp * L * D * (2 * e + 8),  # dK_l, dW_l (fp32) read and rewritten
                            nch * 2 * C * C * D * 10 * L)
    # refinement + ShortConv backward: read v, dK_l, dW_l (fp32), the direct
    # v-gradient; write u, dp_l (for the weight GEMM) and dv
    c["refine_bwd"] = (th * (4 * D * e + L * D * (2 * e + 4)), th * 6 * L * D * D)
    ns = max(1, min(1024 // (2 * H * max(L, 1)), -(-B * Tp // 64)))
    c["wgrad_gemm"] = (th * L * D * 2 * e + th * D * e * 2 * L + H * L * 2 * ns * D * D * 4,
                       th * 4 * L * D * D)
    c["wgrad_reduce"] = (H * L * 2 * ns * D * D * 4 + H * L * 2 * D * D * 4, H * L * 2 * ns * D * D)
    ntiles = -(-T // 29)
    c["bias_reduce"] = (bh * ntiles * (L * D + 4 * D) * 4 + H * (L * D + 4 * D) * 4, 0)
    # weights in MFMA fragment order for the refinement backward: read W_k,
    # W_p, write W_p, W_p^T, W_k^T
    c["weight_frags"] = (H * L * 5 * D * D * e, 0)
    c["refine_fwd_recompute"] = c["refine_fwd"]
    c.update(decode_counts(w))
    peak_f = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    out = {}
    for name, (byt, flo) in c.items():
        t_hbm = byt / (HBM_PEAK_GBS * 1e9)
        t_mfma = flo / (peak_f * 1e12)
        out[name] = {"bytes": byt, "flops": flo, "bound": "mfma" if t_mfma > t_hbm else "hbm",
                     "floor_ms": max(t_hbm, t_mfma) * 1e3}
    return out


DECODE_BATCH = 64   # sequences in flight in the decode-step measurement


def decode_counts(w, batch=DECODE_BATCH):
    """Algorithmic (bytes, FLOPs) per launch of the two decode-step kernels:
    one token for each of `batch` sequences at the workload's head shape.
    step_refine reads v, the ShortConv history, each head's weights and taps
    once, and writes the L pairs; step_state reads and writes the fp32 state
    (8 d^2 bytes per sequence and head), the history, and reads q, k, v,
    alpha, beta and the pairs, and writes o."""
    B, H, D, L = batch, w.H, w.d, w.L
    e = 2 if w.dtype == "bf16" else 4
    bh = B * H
    refine = (bh * (D * e + 4 * D * e + 2 * L * D * e) + H * (L * (2 * D * D + D) + 4 * D) * e,
              bh * L * 4 * D * D)
    state = (bh * (8 * D * D + 4 * D * e + 2 * L * D * e + 2 * 4 * D * e + 8), bh * (4 + 2 * L) * D * D)
    return {"step_refine": refine, "step_state": state}


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None for every kernel)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    if rec.get("sources_sha256") != _sources_sha256():
        return {}
    return {k: v["bytes_per_launch"] for k, v in rec.get("kernels", {}).items()}


def measured_mfma():
    """Matrix-core FLOPs and busy fraction per kernel from the committed
    counter summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    if rec.get("sources_sha256") != _sources_sha256():
        return {}
    return rec.get("mfma", {})


# rocprofv3 kernel names -> the timer names used by the library and above
_FAMILIES = [("refine_fwd_kernel", ["refine_fwd", "refine_fwd_recompute"]),
             ("chunk_bwd_state_kernel", ["chunk_bwd_state"]),
             ("chunk_bwd_solve_kernel", ["chunk_bwd_solve"]),
             ("chunk_bwd_pairs_kernel", ["chunk_bwd_pairs"]),
             ("refine_bwd_kernel", ["refine_bwd"]),
             ("wgrad_gemm_kernel", ["wgrad_gemm"]),
             ("wgrad_reduce_kernel", ["wgrad_reduce"]),
             ("bias_reduce_kernel", ["bias_reduce"]),
             ("weight_frags_kernel", ["weight_frags"]),
             ("decode_refine_kernel", ["step_refine"]),
             ("step_state_kernel", ["step_state"])]


def _family(kernel_name):
    if "state_pass_kernel" in kernel_name:
        # template <E, D, RB, REV, C_RO>: reverse pass, forward with the fused
        # readout (C_RO > 0), or the backward's forward recompute
        m = re.search(r"ELb([01])ELi(\d+)E", kernel_name)
        if m is None:
            m = re.search(r"\b(true|false), (\d+)>", kernel_name)
            rev = m is not None and m.group(1) == "true"
        else:
            rev = m.group(1) == "1"
        if m is None:
            return ["state_fwd", "state_fwd_recompute", "state_bwd"]
        if rev:
            return ["state_bwd"] if int(m.group(2)) > 0 else ["state_bwd_stateless"]
        return ["state_fwd"] if int(m.group(2)) > 0 else ["state_fwd_recompute"]
    if "chunk_fwd_kernel" in kernel_name:
        # template flags <E, D, C, BWD, FUSE, ...>: mangled Lb0/Lb1, or demangled false/true
        flags = re.findall(r"Lb([01])E", kernel_name) or [
            "1" if x == "true" else "0" for x in re.findall(r"\b(true|false)\b", kernel_name)]
        flags += ["0", "0"]
        if flags[1] == "1":
            return ["chunk_fwd_fused"]
        return ["chunk_fwd_bwdmode"] if flags[0] == "1" else ["chunk_fwd"]
    for key, names in _FAMILIES:
        if key in kernel_name:
            return names
    return None


def _sources_sha256():
    import hashlib
    csrc = os.path.join(ROOT, "linear_recurrent_sequence_shortconv_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def summarize_trace(d, workload):
    """Kernel times of one rocprofv3 --kernel-trace --stats run (directory
    d/trace) against the algorithmic bytes and FLOPs of workload: written to
    profiles/<workload>_kernels.md (no counters; profiles/hbm_traffic.json is
    left as it is)."""
    import csv
    from linear_recurrent_sequence_shortconv_amd.workloads import workloads
    w = workloads()[workload]
    counts = algorithmic_counts(w)
    times, names_of = {}, {}
    for r in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv"))):
        fam = _family(r["Name"])
        if fam:
            names_of[fam[0]] = fam
            t = times.setdefault(fam[0], [0, 0.0])
            t[0] += int(r["Calls"])
            t[1] += float(r["TotalDurationNs"])
    cmd = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/trace -o run -- "
           f"python -u $R/bench.py --workload {workload} --steps 10 --warmup 3 --no-cpu-baseline "
           "--no-varlen --no-decode")
    lines = [f"# Kernel time, workload {workload}", "",
             f"B={w.B} T={w.T} H={w.H} d_k=d_v={w.d} L={w.L} chunk={w.chunk} {w.dtype}; one forward + "
             "backward step (the training pair) and the forward alone.",
             "Made with (R = repository root, OUT = an output directory):", "", "```", cmd,
             f"python bench.py --summarize-profiles $OUT --workload {workload}", "```", "",
             "`algorithmic` bytes and FLOPs are what each kernel must move and compute "
             "(bench.py, algorithmic_counts).", "",
             "| kernel | launches | avg us (rocprofv3) | algorithmic MB | GB/s | frac of 8 TB/s | "
             "algorithmic GFLOP | TFLOP/s |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    rows = []
    for first, (calls, tot) in times.items():
        c = counts.get(first)
        if not c:
            continue
        avg_us = tot / calls / 1e3
        gbs = c["bytes"] / (avg_us * 1e-6) / 1e9
        tfl = c["flops"] / (avg_us * 1e-6) / 1e12
        rows.append((tot, f"| {' / '.join(names_of[first])} | {calls} | {avg_us:.1f} | "
                          f"{c['bytes'] / 1e6:.1f} | {gbs:.0f} | {gbs / HBM_PEAK_GBS:.3f} | "
                          f"{c['flops'] / 1e9:.1f} | {tfl:.0f} |"))
    lines += [r for _, r in sorted(rows, reverse=True)]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernels.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_profiles(d, workload):
    """Turn the rocprofv3 runs under directory d (trace/, fetch/, write/,
    cfetch/, cwrite/ and, if present, mfma/: the commands are listed in the
    written summary) into profiles/hbm_traffic.json and
    profiles/<workload>_kernels.md."""
    import csv
    import collections
    from linear_recurrent_sequence_shortconv_amd.workloads import workloads
    w = workloads()[workload]

    def counters(sub):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(os.path.join(d, sub, "run_counter_collection.csv"))):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return agg

    def copy_kib(sub):   # the 1 GiB calibration copy: the largest dispatch
        return max(max(v) for v in counters(sub).values())

    f_factor = (1 << 30) / 1024 / copy_kib("cfetch")
    w_factor = (1 << 30) / 1024 / copy_kib("cwrite")
    names_of = {}          # first timer name of a kernel -> all its timer names
    per = collections.defaultdict(lambda: {"fetch": [], "write": []})
    for sub in ("fetch", "write"):
        for name, vals in counters(sub).items():
            fam = _family(name)
            if fam:
                names_of[fam[0]] = fam
                per[fam[0]][sub] += vals
    traffic = {}
    for first, v in per.items():
        if not v["fetch"] or not v["write"]:
            continue
        fb = sum(v["fetch"]) / len(v["fetch"]) * 1024 * f_factor
        wb = sum(v["write"]) / len(v["write"]) * 1024 * w_factor
        for n in names_of[first]:
            traffic[n] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb)}
    times = {}
    for r in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv"))):
        fam = _family(r["Name"])
        if fam:
            names_of[fam[0]] = fam
            t = times.setdefault(fam[0], [0, 0.0])
            t[0] += int(r["Calls"])
            t[1] += float(r["TotalDurationNs"])
    counts = algorithmic_counts(w)
    cmds = [
        "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/trace -o run -- python -u $R/bench.py --steps 10 --warmup 3 --no-cpu-baseline --no-varlen",
        "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/fetch -o run -- python -u $R/bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-varlen",
        "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/write -o run -- python -u $R/bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-varlen",
        "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/cfetch -o run -- python -u $R/bench.py --calibrate-copy",
        "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/cwrite -o run -- python -u $R/bench.py --calibrate-copy",
        f"cd /tmp && rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d $OUT/mfma -o run -- python -u $R/bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-varlen",
        f"cd /tmp && rocprofv3 --pmc {' '.join(ISSUE_COUNTERS)} --output-format csv -d $OUT/issue -o run -- python -u $R/bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-varlen",
        f"cd /tmp && rocprofv3 --pmc {' '.join(LDS_COUNTERS)} --output-format csv -d $OUT/ldsq -o run -- python -u $R/bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-varlen",
        f"python bench.py --summarize-profiles $OUT --workload {workload}",
    ]
    mfma_csv = os.path.join(d, "mfma", "run_counter_collection.csv")
    mfma_lines, mfma_rec = (_mfma_table(mfma_csv, times, names_of, counts)
                            if os.path.exists(mfma_csv) else ([], {}))
    ia = os.path.join(d, "issue", "run_counter_collection.csv")
    ib = os.path.join(d, "ldsq", "run_counter_collection.csv")
    issue_lines, issue_rec = (_issue_table(ia, ib, times, names_of)
                              if os.path.exists(ia) else ([], {}))
    rec = {"workload": workload, "sources_sha256": _sources_sha256(),
           "calibration": {"fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
                           "copy_bytes": 1 << 30},
           "commands": cmds, "kernels": traffic, "mfma": mfma_rec, "issue": issue_rec}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# Kernel time and HBM traffic, workload {workload}",
             "",
             f"B={w.B} T={w.T} H={w.H} d_k=d_v={w.d} L={w.L} chunk={w.chunk} {w.dtype}; one forward + backward step.",
             f"step_refine / step_state: the decode step (prism_step, one token) for B={DECODE_BATCH} sequences "
             "at the same head shape, which bench.py also times.",
             "Made with (R = repository root, OUT = an output directory; each rocprofv3 run on its own):",
             "", "```"] + cmds + ["```", "",
             f"HBM byte counters are scaled by the readings of a plain 1 GiB device copy: FETCH_SIZE x {f_factor:.3f}, "
             f"WRITE_SIZE x {w_factor:.3f}.  `algorithmic` is the byte count each kernel must move "
             "(bench.py, algorithmic_counts); `ratio` = measured / algorithmic.", "",
             "| kernel | launches | avg us (rocprofv3) | algorithmic MB | measured MB | ratio | GB/s (algorithmic) | frac of 8 TB/s |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    rows = []
    for first, (calls, tot) in times.items():
        avg_us = tot / calls / 1e3
        c = counts.get(first)
        if not c:
            continue
        meas = traffic.get(first, {}).get("bytes_per_launch")
        gbs = c["bytes"] / (avg_us * 1e-6) / 1e9
        rows.append((tot, f"| {' / '.join(names_of[first])} | {calls} | {avg_us:.1f} | {c['bytes'] / 1e6:.1f} | "
                          f"{(meas / 1e6) if meas else float('nan'):.1f} | "
                          f"{(meas / c['bytes']) if meas else float('nan'):.2f} | {gbs:.0f} | {gbs / HBM_PEAK_GBS:.3f} |"))
    lines += [r for _, r in sorted(rows, reverse=True)]
    lines += mfma_lines
    lines += issue_lines
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernels.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Issue and LDS counters (gfx950), two rocprofv3 --pmc runs (at most 8 SQ
# counters each).  SQ_WAVE_CYCLES, SQ_WAIT_ANY and SQ_WAIT_INST_ANY are in
# quad-cycles; instruction counts are summed over the shader engines.
ISSUE_COUNTERS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_INSTS_VALU",
                  "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"]
LDS_COUNTERS = ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU",
                "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE"]
CLOCK_GHZ = 2.4


def _issue_table(path_a, path_b, times, names_of):
    """Markdown lines and a per-timer-name record from the issue / LDS counter
    runs: VALU, LDS, SALU, VMEM instructions per wave; the fraction of wave
    time spent waiting for anything (SQ_WAIT_ANY / SQ_WAVE_CYCLES) and for an
    instruction to issue (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES); `VALU issue` =
    SQ_INSTS_VALU x 4 cycles (a wave64 instruction on a 16-lane SIMD) over
    the kernel-trace duration x 1024 SIMDs x 2.4 GHz; `LDS conflict` =
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (LDS busy cycles lost to bank
    conflicts)."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in (path_a, path_b):
        if not os.path.exists(path):
            continue
        for r in csv.DictReader(open(path)):
            fam = _family(r["Kernel_Name"])
            if fam:
                names_of.setdefault(fam[0], fam)
                per[fam[0]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = ["", "Issue and LDS, two rocprofv3 --pmc runs with " + ", ".join(ISSUE_COUNTERS) + " and "
           + ", ".join(LDS_COUNTERS) + ": per-wave instruction counts (SQ_INSTS_* / SQ_WAVES); "
           "`wait` = SQ_WAIT_ANY / SQ_WAVE_CYCLES (wave time waiting on anything: memory, "
           "dependencies, barriers); `issue wait` = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; `VALU issue` "
           "= SQ_INSTS_VALU x 4 cycles / (kernel-trace duration x 1024 SIMDs x 2.4 GHz), the share "
           "of the chip's VALU issue slots used; `LDS conflict` = SQ_LDS_BANK_CONFLICT / "
           "SQ_LDS_IDX_ACTIVE.", "",
           "| kernel | waves | VALU / wave | LDS / wave | SALU / wave | VMEM / wave | wait | issue wait | "
           "VALU issue | LDS conflict |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    rows, rec = [], {}
    for first, v in per.items():
        def avg(c):
            x = v.get(c, [])
            return sum(x) / len(x) if x else 0.0
        waves = avg("SQ_WAVES")
        if waves <= 0 or first not in times:
            continue
        calls, tot = times[first]
        sec = tot / calls * 1e-9
        wc = avg("SQ_WAVE_CYCLES")
        wait = avg("SQ_WAIT_ANY") / wc if wc > 0 else float("nan")
        iwait = avg("SQ_WAIT_INST_ANY") / wc if wc > 0 else float("nan")
        valu_issue = avg("SQ_INSTS_VALU") * 4 / (sec * N_SIMD * CLOCK_GHZ * 1e9)
        lds_act = avg("SQ_LDS_IDX_ACTIVE")
        confl = avg("SQ_LDS_BANK_CONFLICT") / lds_act if lds_act > 0 else float("nan")
        r = {"waves": round(waves), "valu_per_wave": round(avg("SQ_INSTS_VALU") / waves, 1),
             "lds_per_wave": round(avg("SQ_INSTS_LDS") / waves, 1),
             "salu_per_wave": round(avg("SQ_INSTS_SALU") / waves, 1),
             "vmem_per_wave": round(avg("SQ_INSTS_VMEM") / waves, 1),
             "wait": round(wait, 3), "issue_wait": round(iwait, 3), "valu_issue": round(valu_issue, 3),
             "lds_conflict": round(confl, 3)}
        rows.append((tot, f"| {' / '.join(names_of[first])} | {r['waves']} | {r['valu_per_wave']:.0f} | "
                          f"{r['lds_per_wave']:.0f} | {r['salu_per_wave']:.0f} | {r['vmem_per_wave']:.0f} | "
                          f"{wait:.2f} | {iwait:.2f} | {valu_issue:.3f} | {confl:.3f} |"))
        for n in names_of[first]:
            rec[n] = r
    return out + [r for _, r in sorted(rows, reverse=True)], rec


# Matrix-core counters (gfx950): SQ_INSTS_VALU_MFMA_MOPS_* count multiply and
# add operations / 512, summed over the shader engines; SQ_VALU_MFMA_BUSY_CYCLES
# sums the cycles each SIMD's matrix unit is busy; GRBM_GUI_ACTIVE reads once
# per XCD, so the per-dispatch value is the XCDs' sum of the active cycles.
MFMA_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
N_XCD = 8
N_SIMD = 256 * 4


def _mfma_table(path, times, names_of, counts):
    """Markdown lines: matrix-core FLOPs and busy time per kernel, from one
    rocprofv3 --pmc run with MFMA_COUNTERS (one row per dispatch and counter).
    TFLOP/s divide the counted FLOPs by the kernel-trace average duration;
    `pipe frac` is the time the counted FLOPs need at the dense peaks
    (bf16 2.5 PFLOP/s, fp32 157.3 TFLOP/s) over that duration; `busy` is the
    matrix units' busy cycles over the SIMDs' active cycles.  Returns the
    lines and a per-timer-name record {counted flops, pipe frac, busy}."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        fam = _family(r["Kernel_Name"])
        if fam:
            names_of.setdefault(fam[0], fam)
            per[fam[0]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = ["", "Matrix cores (MFMA), one rocprofv3 --pmc run with " + ", ".join(MFMA_COUNTERS) + ": "
           "counted FLOP = 512 x the MOPS counters; TFLOP/s over the kernel-trace average duration; "
           "`pipe frac` = time the counted FLOPs need at the dense peaks (bf16 2.5 PFLOP/s, fp32 "
           "157.3 TFLOP/s) / duration; `busy` = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
           f"{N_XCD} XCDs x {N_SIMD} SIMDs).  `algorithmic GFLOP` is the products the algorithm "
           "needs (bench.py, algorithmic_counts).", "",
           "| kernel | counted GFLOP bf16 | counted GFLOP fp32 | algorithmic GFLOP | TFLOP/s (bf16) | "
           "pipe frac | busy |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    rows = []
    rec = {}
    for first, v in per.items():
        def avg(c):
            x = v.get(c, [])
            return sum(x) / len(x) if x else 0.0
        fb, ff = avg(MFMA_COUNTERS[0]) * 512, avg(MFMA_COUNTERS[1]) * 512
        if fb + ff <= 0 or first not in times:
            continue
        calls, tot = times[first]
        sec = tot / calls * 1e-9
        pipe = (fb / (MFMA_BF16_PEAK_TFLOPS * 1e12) + ff / (MFMA_F32_PEAK_TFLOPS * 1e12)) / sec
        gui = avg(MFMA_COUNTERS[3])
        busy = avg(MFMA_COUNTERS[2]) / (gui / N_XCD * N_SIMD) if gui > 0 else float("nan")
        alg = counts.get(first, {}).get("flops", 0)
        rows.append((tot, f"| {' / '.join(names_of[first])} | {fb / 1e9:.1f} | {ff / 1e9:.2f} | {alg / 1e9:.1f} | "
                          f"{fb / sec / 1e12:.0f} | {pipe:.3f} | {busy:.3f} |"))
        for n in names_of[first]:
            rec[n] = {"flops_bf16": round(fb), "flops_f32": round(ff), "pipe_frac": round(pipe, 4),
                      "busy": round(busy, 4)}
    return out + [r for _, r in sorted(rows, reverse=True)], rec


def roofline_for(name, counts, avg_ms, dtype, traffic=None):
    c = counts.get(name)
    if c is None or avg_ms <= 0:
        return None
    if c["bound"] == "mfma":
        achieved = c["flops"] / (avg_ms * 1e-3) / 1e12
        peak = MFMA_BF16_PEAK_TFLOPS if dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
        unit = "TFLOP/s"
    else:
        achieved = c["bytes"] / (avg_ms * 1e-3) / 1e9
        peak = HBM_PEAK_GBS
        unit = "GB/s"
    return {"kernel": name, "bound": c["bound"], "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": (traffic or {}).get(name),
            "algorithmic_bytes": c["bytes"], "algorithmic_flops": c["flops"],
            "avg_launch_ms": round(avg_ms, 5), "roofline_floor_ms": round(c["floor_ms"], 5)}


def _oracle_sequence(args):
    """One (b, h) sequence through the float64 oracle (a CPU-baseline task):
    forward, and the backward when asked.  Runs in a pool worker."""
    from threadpoolctl import threadpool_limits
    from oracle import prism_oracle as O
    seq, W, backward = args
    with threadpool_limits(limits=1):
        O.forward(seq["q"], seq["k"], seq["v"], seq["alpha"], seq["beta"], *W)
        if backward:
            O.backward(seq["q"], seq["k"], seq["v"], seq["alpha"], seq["beta"], *W, dO=seq["dO"])
    return seq["q"].shape[1]


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, budget_s=20.0, backward=False, max_workers=16):
    """The float64 oracle, as it stands, on the host cores: whole (b, h)
    sequences of the same inputs spread over a process pool (one BLAS thread
    per worker, workers = the cores this process may use, at most
    max_workers), submitted in order until the time budget is spent.  Workers
    are started and warmed before the clock runs.  Returns tokens/s scaled to
    the workload's unit (a token spans all H heads)."""
    import multiprocessing as mp
    from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]

    def task(b, h):
        seq = {n: x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v", "alpha", "beta", "dO")}
        W = [x[n][h:h + 1] for n in ("Wk", "Wp", "wbeta", "conv")] if w.L > 0 else [None] * 4
        return (seq, W, backward)

    # spawned workers: a fresh interpreter each (this process has the GPU open)
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        tiny = {n: x[n][:1, :2, :1] for n in ("q", "k", "v", "alpha", "beta", "dO")}
        Wt = [x[n][:1] for n in ("Wk", "Wp", "wbeta", "conv")] if w.L > 0 else [None] * 4
        list(ex.map(_oracle_sequence, [(tiny, Wt, backward)] * workers))   # warm-up
        t0 = time.perf_counter()
        it = iter(pairs)
        pending, done_tokens, seqs = set(), 0, 0
        for _ in range(workers):
            nxt = next(it, None)
            if nxt is not None:
                pending.add(ex.submit(_oracle_sequence, task(*nxt)))
        while pending:
            finished, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in finished:
                done_tokens += f.result()
                seqs += 1
            if time.perf_counter() - t0 < budget_s:
                for _ in finished:
                    nxt = next(it, None)
                    if nxt is not None:
                        pending.add(ex.submit(_oracle_sequence, task(*nxt)))
        wall = time.perf_counter() - t0
    tokens = done_tokens / w.H
    return {"value": round(tokens / wall, 2), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{seqs} of {w.B * w.H} (b,h) sequences x T={w.T}, "
                      f"{'fwd+bwd' if backward else 'fwd'}, float64, {workers} worker processes "
                      f"with one thread each, {wall:.1f} s wall"}


# The two stages the targets are stated for: the chunked scan (chunk-local
# solve and products, the state passes, and their backward) against the bf16
# MFMA peak, and the refinement / ShortConv stage (its forward, its backward
# with the ShortConv adjoint, and the weight-gradient kernels) against HBM.
SCAN_KERNELS = ("chunk_fwd", "state_fwd", "state_bwd", "chunk_bwd_state", "chunk_bwd_solve",
                "chunk_bwd_pairs")
REFINE_KERNELS = ("refine_fwd", "refine_bwd", "wgrad_gemm", "wgrad_reduce", "bias_reduce",
                  "weight_frags")


def stage_fractions(kernels, counts, dtype):
    """Aggregate rates of the two stages over one training step: scan
    sum(FLOP) / sum(t) against the dense MFMA peak (and its sum(bytes) /
    sum(t) against HBM), refinement sum(bytes) / sum(t) against HBM; with the
    counter-measured MFMA busy fraction of the scan kernels (time-weighted)
    when the committed counter summary matches the current sources."""
    peak_f = MFMA_BF16_PEAK_TFLOPS if dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    mf = measured_mfma()

    def agg(names):
        t = sum(kernels[n]["total_ms"] for n in names if n in kernels) * 1e-3
        by = sum(counts[n]["bytes"] * kernels[n]["launches_per_step"] for n in names if n in kernels)
        fl = sum(counts[n]["flops"] * kernels[n]["launches_per_step"] for n in names if n in kernels)
        return t, by, fl

    t, by, fl = agg(SCAN_KERNELS)
    scan = None
    if t > 0:
        busy = None
        if all(n in mf for n in SCAN_KERNELS if n in kernels):
            busy = round(sum(mf[n]["busy"] * kernels[n]["total_ms"] for n in SCAN_KERNELS if n in kernels)
                         / (t * 1e3), 4)
        scan = {"kernels": [n for n in SCAN_KERNELS if n in kernels], "ms": round(t * 1e3, 4),
                "tflops": round(fl / t / 1e12, 1), "mfma_frac": round(fl / t / 1e12 / peak_f, 4),
                "mfma_busy_counted": busy, "target_mfma_frac": 0.40,
                "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    t, by, fl = agg(REFINE_KERNELS)
    refine = None
    if t > 0:
        refine = {"kernels": [n for n in REFINE_KERNELS if n in kernels], "ms": round(t * 1e3, 4),
                  "gbs": round(by / t / 1e9, 1), "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                  "target_hbm_frac": 0.60}
    return {"scan": scan, "refinement": refine}


def decode_bench(w, steps, batch=DECODE_BATCH):
    """The decode step (prism_step, one token per sequence) at the workload's
    head shape with `batch` sequences: event-timed calls, each kernel's own
    average from the library's event timer, and the HBM roofline of the
    state kernel, which dominates.  Its bytes per call: the fp32 state read
    and written (8 d^2 per sequence and head), q, k, v, o, alpha, beta, the
    L refinement pairs and the ShortConv history read and written."""
    import numpy as np
    import torch
    from linear_recurrent_sequence_shortconv_amd import prism as P
    from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs

    B, H, d, L = batch, w.H, w.d, w.L
    x = make_inputs(B, 1, H, d, L, w.dtype, seed=1, random_S0=True)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda a, t=tdt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
    args = tuple(dev(x[n]) for n in ("q", "k", "v")) + tuple(
        dev(x[n], torch.float32) for n in ("alpha", "beta")) + tuple(
        dev(x.get(n)) for n in ("Wk", "Wp", "wbeta", "conv"))
    S = dev(x["S0"], torch.float32)
    cs = torch.zeros((B, 4, H, d), dtype=tdt, device="cuda")
    for _ in range(3):
        P.step(*args, S=S, conv_state=cs)
    torch.cuda.synchronize()
    n = max(steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        P.step(*args, S=S, conv_state=cs)
    e1.record()
    torch.cuda.synchronize()
    us_call = e0.elapsed_time(e1) * 1e3 / n
    with P.KernelTimer() as kt:
        for _ in range(n):
            P.step(*args, S=S, conv_state=cs)
        torch.cuda.synchronize()
    us = {n: tot * 1e3 / cnt for n, (tot, cnt) in kt.result.items()}
    nbytes = decode_counts(w, B)["step_state"][0]
    gbps = nbytes / (us["step_state"] * 1e-6) / 1e9
    return {"workload": f"decode step B={B} H={H} d={d} L={L} {w.dtype}",
            "us_per_call": round(us_call, 2),
            "kernels_us": {n: round(x, 2) for n, x in us.items()},
            "tokens_per_s": round(B / (us_call * 1e-6), 1),
            "roofline": {"kernel": "step_state", "bound": "hbm", "achieved": round(gbps, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": nbytes,
                         "traffic": measured_traffic().get("step_state")}}


def varlen_bench(steps, B=64, H=4, d=64, L=2, chunk=64, tmax=200, seed=3):
    """Packed batch of ragged histories at the sequential-recommendation head
    shape (forward, as that configuration is quoted): lengths uniform in
    [tmax / 10, tmax], seeded.  Real tokens per second of the packed call and
    of the same sequences padded to tmax in a dense call."""
    import numpy as np
    import torch
    from linear_recurrent_sequence_shortconv_amd import prism as P
    from linear_recurrent_sequence_shortconv_amd.workloads import make_inputs

    rng = np.random.default_rng(seed)
    lengths = rng.integers(tmax // 10, tmax + 1, size=B)
    N = int(lengths.sum())
    x = make_inputs(1, N, H, d, L, "bf16", seed=seed)
    bf, f32 = torch.bfloat16, torch.float32
    dev = lambda a, t=bf: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
    packed = (dev(x["q"][0]), dev(x["k"][0]), dev(x["v"][0]), dev(x["alpha"][0], f32),
              dev(x["beta"][0], f32)) + tuple(dev(x[n]) for n in ("Wk", "Wp", "wbeta", "conv"))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).to("cuda")
    # the same sequences, right-padded to tmax (alpha = 1, beta = 0 past the end)
    cpu = np.concatenate([[0], np.cumsum(lengths)])
    def pad(a, fill):
        out = np.full((B, tmax) + a.shape[2:], fill, dtype=np.float64)
        for b in range(B):
            out[b, :lengths[b]] = a[0, cpu[b]:cpu[b + 1]]
        return out
    dense = (dev(pad(x["q"], 0.0)), dev(pad(x["k"], 0.0)), dev(pad(x["v"], 0.0)),
             dev(pad(x["alpha"], 1.0), f32), dev(pad(x["beta"], 0.0), f32)) + packed[5:]

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_p = timed(lambda: P.forward(*packed, chunk=chunk, cu_seqlens=cu, max_seqlen=tmax))
    ms_d = timed(lambda: P.forward(*dense, chunk=chunk))
    return {"workload": f"packed histories B={B} H={H} d={d} L={L} bf16, lengths U[{tmax // 10},{tmax}] "
                        f"(mean {lengths.mean():.0f}), forward",
            "tokens": N, "ms_packed": round(ms_p, 4), "ms_padded_dense": round(ms_d, 4),
            "tokens_per_s_packed": round(N / (ms_p * 1e-3), 1),
            "tokens_per_s_padded": round(N / (ms_d * 1e-3), 1)}


SWEEP = ("long-T2048", "long-T4096", "long-T8192", "long-T16384",
         "depth-L0", "depth-L1", "depth-L2", "depth-L4", "depth-L8")


def sweep(steps, names=SWEEP):
    """Training-pair step (forward keeping the intermediates + backward) and
    forward alone for the long-context sweep (T = 2K..16K at 16384 tokens per
    batch) and the refinement-depth sweep (L = 0..8, B=4, T=4096); inputs are
    resident in HBM before timing.  One JSON line."""
    import numpy as np
    import torch
    from linear_recurrent_sequence_shortconv_amd import prism as P
    from linear_recurrent_sequence_shortconv_amd.workloads import make_workload_inputs, workloads

    rows = []
    for name in names:
        w = workloads()[name]
        x = make_workload_inputs(w, seed=0)
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dev = lambda a, t=tdt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
        f32 = torch.float32
        a = (dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["alpha"], f32), dev(x["beta"], f32)) + (
            tuple(dev(x[n]) for n in ("Wk", "Wp", "wbeta", "conv")) if w.L > 0 else (None,) * 4)
        dO = dev(x["dO"])
        del x
        desc = P.make_desc(w.B, w.T, w.H, w.d, w.d, w.L, w.chunk, P.PRISM_BF16)
        ws_f = P._workspace(P.forward_workspace_bytes(desc), a[0].device)[1]
        ws_ft = P._workspace(P.forward_train_workspace_bytes(desc), a[0].device)[1]
        ws_bt = P._workspace(P.backward_train_workspace_bytes(desc), a[0].device)[1]
        saved = P._workspace(P.saved_bytes(desc), a[0].device)[1]

        def train():
            P.forward(*a, chunk=w.chunk, workspace=ws_ft, saved=saved)
            P.backward(*a, dO=dO, chunk=w.chunk, workspace=ws_bt, saved=saved)

        def fwd():
            P.forward(*a, chunk=w.chunk, workspace=ws_f)

        res = {"workload": name, "B": w.B, "T": w.T, "L": w.L}
        for key, fn in (("fwd_bwd", train), ("fwd", fwd)):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            res[f"ms_{key}"] = round(ms, 4)
            res[f"tokens_per_s_{key}"] = round(w.B * w.T / (ms * 1e-3), 1)
        rows.append(res)
        print(json.dumps(res), file=sys.stderr, flush=True)
        del a, dO, ws_f, ws_ft, ws_bt, saved
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": rows, "dtype": "bf16", "data": "synthetic", "steps": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="lm-T2048")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forward-only", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed-batch measurement")
    ap.add_argument("--sweep", action="store_true",
                    help="time the long-context and refinement-depth sweeps instead (one JSON line)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from the rocprofv3 runs under DIR and exit")
    args = ap.parse_args()

    if args.summarize_profiles:
        if os.path.isdir(os.path.join(args.summarize_profiles, "cfetch")):
            summarize_profiles(args.summarize_profiles, args.workload)
        else:   # a kernel trace only
            summarize_trace(args.summarize_profiles, args.workload)
        return

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(sequences and heads are independent, so several GPUs would each run this same "
              "per-GPU workload).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.sweep:
        sweep(args.steps)
        return

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))
        return

    from linear_recurrent_sequence_shortconv_amd import prism as P
    from linear_recurrent_sequence_shortconv_amd.workloads import make_workload_inputs, workloads

    w = workloads()[args.workload]
    x = make_workload_inputs(w, seed=0)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda a, t=tdt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
    f32 = torch.float32
    q, k, v, dO = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dO"])
    alpha, beta = dev(x["alpha"], f32), dev(x["beta"], f32)
    if w.L > 0:
        Wk, Wp, wbeta, conv = dev(x["Wk"]), dev(x["Wp"]), dev(x["wbeta"]), dev(x["conv"])
    else:
        Wk = Wp = wbeta = conv = None

    desc = P.make_desc(w.B, w.T, w.H, w.d, w.d, w.L, w.chunk, P.PRISM_BF16 if w.dtype == "bf16" else P.PRISM_F32)
    backward = not args.forward_only
    try:
        P.backward_workspace_bytes(desc)
    except RuntimeError:
        backward = False
    ws_f = P._workspace(P.forward_workspace_bytes(desc), q.device)[1]
    ws_b = P._workspace(P.backward_workspace_bytes(desc), q.device)[1] if backward else None
    ws_ft = P._workspace(P.forward_train_workspace_bytes(desc), q.device)[1] if backward else None
    ws_bt = P._workspace(P.backward_train_workspace_bytes(desc), q.device)[1] if backward else None
    saved = P._workspace(P.saved_bytes(desc), q.device)[1] if backward else None

    def step():
        # a training step: the forward keeps what the backward needs
        if backward:
            P.forward(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, chunk=w.chunk, workspace=ws_ft,
                      saved=saved)
            P.backward(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, dO=dO, chunk=w.chunk,
                       workspace=ws_bt, saved=saved)
        else:
            P.forward(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, chunk=w.chunk, workspace=ws_f)

    def stateless_step():
        P.forward(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, chunk=w.chunk, workspace=ws_f)
        P.backward(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, dO=dO, chunk=w.chunk,
                   workspace=ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing (events on the current stream, which the library uses)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps

    # the stateless pair (prism_forward + prism_backward, which recomputes)
    ms_stateless = None
    if backward:
        for _ in range(2):
            stateless_step()
        torch.cuda.synchronize()
        s_start, s_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_start.record()
        for _ in range(args.steps):
            stateless_step()
        s_end.record()
        torch.cuda.synchronize()
        ms_stateless = s_start.elapsed_time(s_end) / args.steps

    # forward pass alone (same inputs, same workspace)
    def fwd_step():
        P.forward(q, k, v, alpha, beta, Wk, Wp, wbeta, conv, chunk=w.chunk, workspace=ws_f)

    for _ in range(2):
        fwd_step()
    torch.cuda.synchronize()
    f_start, f_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f_start.record()
    for _ in range(args.steps):
        fwd_step()
    f_end.record()
    torch.cuda.synchronize()
    ms_fwd = f_start.elapsed_time(f_end) / args.steps

    # per-kernel timing of the forward alone, then of the training step, each
    # over its own timed region (HIP events around each launch)
    with P.KernelTimer() as kf:
        for _ in range(args.steps):
            fwd_step()
        torch.cuda.synchronize()
    fwd_kernels = {n: round(tot / c, 5) for n, (tot, c) in kf.result.items()}
    with P.KernelTimer() as kt:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    kernels = {n: {"total_ms": round(tot / args.steps, 5), "launches_per_step": c // args.steps,
                   "avg_launch_ms": round(tot / c, 5)} for n, (tot, c) in kt.result.items()}
    counts = algorithmic_counts(w)
    traffic = measured_traffic()
    dominant = max(kernels, key=lambda n: kernels[n]["total_ms"]) if kernels else None
    roof = (roofline_for(dominant, counts, kernels[dominant]["avg_launch_ms"], w.dtype, traffic)
            if dominant else None)
    for n in kernels:
        r = roofline_for(n, counts, kernels[n]["avg_launch_ms"], w.dtype, traffic)
        if r:
            kernels[n].update(bound=r["bound"], achieved=r["achieved"], unit=r["unit"],
                              frac=r["frac"], floor_ms=r["roofline_floor_ms"])

    decode = None if args.no_decode else decode_bench(w, args.steps)
    varlen = None if args.no_varlen else varlen_bench(args.steps)

    tokens = w.B * w.T
    value = tokens / (ms * 1e-3)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x, backward=backward)

    line = {
        "metric": "PRISM layer tokens/s fwd and fwd+bwd at T=2K\u201316K; % of MFMA/HBM peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d_k": w.d, "d_v": w.d,
                   "L": w.L, "chunk": w.chunk, "global_batch": w.B, "seq_len": w.T,
                   "passes": "fwd+bwd" if backward else "fwd", "parallelism": "single GPU"},
        "forward": {"ms_per_step": round(ms_fwd, 4), "tokens_per_s": round(tokens / (ms_fwd * 1e-3), 1),
                    "kernels_avg_ms": fwd_kernels},
        "stateless_pair": (None if ms_stateless is None else
                           {"ms_per_step": round(ms_stateless, 4),
                            "tokens_per_s": round(tokens / (ms_stateless * 1e-3), 1)}),
        "roofline": roof,
        "stages": stage_fractions(kernels, counts, w.dtype) if backward else None,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "decode": decode,
        "varlen": varlen,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""Turn rocprofv3 CSV output of bench.py runs into short text summaries.

Usage (from the repository root, after the profiler runs below have written
their CSVs under OUT_DIR):

    python -m w8a8_integer_linear_amd.profiling OUT_DIR

Reads  OUT_DIR/kt/*kernel_stats.csv      (rocprofv3 --kernel-trace --stats)
       OUT_DIR/fetch/*counter_collection.csv (rocprofv3 --pmc FETCH_SIZE)
       OUT_DIR/write/*counter_collection.csv (rocprofv3 --pmc WRITE_SIZE)
       OUT_DIR/busy/*counter_collection.csv (rocprofv3 --pmc SQ_BUSY_CYCLES
                                    SQ_VALU_MFMA_BUSY_CYCLES), if present
       OUT_DIR/valu/*counter_collection.csv (rocprofv3 --pmc SQ_INSTS_VALU
                                    SQ_BUSY_CYCLES SQ_WAVES), if present
       OUT_DIR/power.txt (amd-smi metric -p -c samples taken while bench.py
                          ran its step loop), if present
       OUT_DIR/power_ceiling.txt (the same while bench.py ran the matrix-core
                          ceiling kernel), if present
Writes profiles/kernels_headline_step.txt (per-kernel durations),
       profiles/pmc_traffic.json + profiles/pmc_traffic.txt (HBM bytes per
       launch, scaled by the reading of the calibration copy of 512 MiB) and
       profiles/mfma_busy_clock.txt (per kernel: the shader clock it ran at,
       SQ busy cycles per shader engine over the dispatch's duration, and the
       fraction of those cycles the SIMDs' matrix pipes were busy) and
       profiles/lds_bank_conflicts.txt (from OUT_DIR/lds, if present),
       profiles/valu_issue.txt (per kernel: the time its vector instructions
       alone take to issue, against its duration),
       profiles/power_headline_step.txt and profiles/power_mfma_ceiling.txt.
"""
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 << 20


def _one(pattern):
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _short(name):
    name = name.replace("qlin::(anonymous namespace)::", "").replace("qlin::", "")
    return name.split("(")[0] if "gemm_kernel" not in name else name.split(")")[0] + ")"


def kernel_stats(out_dir):
    path = _one(os.path.join(out_dir, "kt", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    res = []
    for r in rows:
        res.append({"kernel": _short(r["Name"]), "calls": int(r["Calls"]),
                    "total_ns": float(r["TotalDurationNs"]),
                    "avg_ns": float(r["AverageNs"]), "pct": float(r["Percentage"])})
    return res


def dispatches(out_dir, sub, name):
    """{dispatch id: (short kernel name, counter value in KiB)}."""
    path = _one(os.path.join(out_dir, sub, "*counter_collection.csv"))
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == name:
            out[int(r["Dispatch_Id"])] = (_short(r["Kernel_Name"]), float(r["Counter_Value"]))
    return out


def busy_clock(out_dir):
    """Per kernel: median effective shader clock (GHz) and MFMA-busy fraction."""
    path = _one(os.path.join(out_dir, "busy", "*counter_collection.csv"))
    info = list(csv.DictReader(open(_one(os.path.join(out_dir, "busy", "*agent_info.csv")))))
    gpu = [r for r in info if r["Agent_Type"] == "GPU"][0]
    n_se, n_simd = int(gpu["Array_Count"]), int(gpu["Simd_Count"])
    per = {}
    for r in csv.DictReader(open(path)):
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": _short(r["Kernel_Name"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    by = {}
    for d in per.values():
        if d["dur_s"] <= 0 or "SQ_BUSY_CYCLES" not in d:
            continue
        cycles = d["SQ_BUSY_CYCLES"] / n_se
        by.setdefault(d["name"], []).append(
            (cycles / d["dur_s"] / 1e9, d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n_simd / cycles,
             d["dur_s"] * 1e6))
    return {k: tuple(statistics.median(v[i] for v in vals) for i in range(3)) + (len(vals),)
            for k, vals in by.items()}, n_se, n_simd


def bench_line(out_dir):
    """The JSON line bench.py printed in the traced run (None if absent)."""
    path = os.path.join(out_dir, "kt.log")
    if not os.path.exists(path):
        return None
    lines = [ln for ln in open(path) if ln.startswith("{")]
    return json.loads(lines[-1]) if lines else None


def main(out_dir, digest=None):
    os.makedirs(PROFILES, exist_ok=True)
    stats = kernel_stats(out_dir)
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(PROFILES, "kernels_headline_step.txt"), "w") as f:
        f.write("# rocprofv3 --kernel-trace --stats of the headline training step\n")
        f.write("# (12000 tokens, 5376 -> 7168, Hadamard block 128).  Command:\n")
        f.write("#   rocprofv3 --kernel-trace --stats -d OUT/kt -o kt --output-format csv -- "
                "python bench.py --cpu-tokens 0 --step-kernels-only\n")
        f.write(f"# {'kernel':<70} {'calls':>5} {'avg_us':>9} {'pct':>6}\n")
        for s in sorted(stats, key=lambda r: -r["total_ns"]):
            f.write(f"  {s['kernel'][:70]:<70} {s['calls']:>5} {s['avg_ns'] / 1e3:>9.2f} "
                    f"{s['pct']:>6.2f}\n")
        line = bench_line(out_dir)
        if line:
            f.write("# The same run's bench line: per-call time from HIP events over the timed\n"
                    "# steps, against the profiler's average over every call (warmup included).\n")
            f.write(f"# {'call':<14} {'bench_us':>9} {'rocprof_us':>11}\n")
            for call, ent in line.get("breakdown", {}).items():
                keys = bench.KERNEL_OF.get(call, [])
                prof = sum(st["avg_ns"] for k in keys for st in stats if k in st["kernel"]) / 1e3
                f.write(f"  {call:<14} {ent['ms'] * 1e3:>9.1f} {prof:>11.1f}\n")
    fetch = dispatches(out_dir, "fetch", "FETCH_SIZE")
    write = dispatches(out_dir, "write", "WRITE_SIZE")
    # The calibration copies are the 'copy' dispatches that wrote COPY_BYTES
    # (both runs execute the same dispatch sequence, so ids line up).
    target = COPY_BYTES / 1024
    cal = [d for d, (n, v) in write.items()
           if "copy" in n.lower() and abs(v - target) < 0.01 * target and d in fetch]
    if not cal:
        raise RuntimeError("calibration copy not found in the counter output")
    f_fac = COPY_BYTES / (statistics.median(fetch[d][1] for d in cal) * 1024)
    w_fac = COPY_BYTES / (statistics.median(write[d][1] for d in cal) * 1024)
    per = {}
    for d, (n, fv) in fetch.items():
        if d in cal or d not in write or write[d][0] != n:
            continue
        per.setdefault(n, []).append((fv * 1024 * f_fac, write[d][1] * 1024 * w_fac))
    kernels = {}
    for n, vals in per.items():
        fb = statistics.median(v[0] for v in vals)
        wb = statistics.median(v[1] for v in vals)
        kernels[n] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                      "bytes_per_launch": round(fb + wb), "launches": len(vals)}
    if digest is None:
        digest = bench.source_digest()
    rec = {"source_digest": digest, "calibration_dispatches": cal, "fetch_scale": f_fac,
           "write_scale": w_fac, "kernels": kernels,
           "commands": ["rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o fetch --output-format csv -- "
                        "python bench.py --steps 2 --warmup 1 --cpu-tokens 0 --step-kernels-only --copy-calibration",
                        "rocprofv3 --pmc WRITE_SIZE -d OUT/write -o write --output-format csv -- "
                        "python bench.py --steps 2 --warmup 1 --cpu-tokens 0 --step-kernels-only --copy-calibration"]}
    with open(os.path.join(PROFILES, "pmc_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    with open(os.path.join(PROFILES, "pmc_traffic.txt"), "w") as f:
        f.write("# HBM bytes per launch from FETCH_SIZE / WRITE_SIZE, scaled so that a plain copy\n")
        f.write(f"# of {COPY_BYTES >> 20} MiB reads and writes exactly that much "
                f"(fetch x{f_fac:.3f}, write x{w_fac:.3f}).\n")
        for c in rec["commands"]:
            f.write(f"#   {c}\n")
        f.write(f"# {'kernel':<70} {'fetch_MB':>9} {'write_MB':>9} {'total_MB':>9}\n")
        for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["bytes_per_launch"]):
            f.write(f"  {k[:70]:<70} {v['fetch_bytes'] / 1e6:>9.1f} {v['write_bytes'] / 1e6:>9.1f} "
                    f"{v['bytes_per_launch'] / 1e6:>9.1f}\n")
    print(open(os.path.join(PROFILES, "kernels_headline_step.txt")).read())
    print(open(os.path.join(PROFILES, "pmc_traffic.txt")).read())
    if glob.glob(os.path.join(out_dir, "busy", "*counter_collection.csv")):
        res, n_se, n_simd = busy_clock(out_dir)
        with open(os.path.join(PROFILES, "mfma_busy_clock.txt"), "w") as f:
            f.write("# Shader clock and matrix-pipe occupancy per kernel of the headline step.\n")
            f.write("#   rocprofv3 --pmc SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES -d OUT/busy -o busy "
                    "--output-format csv -- python bench.py --steps 2 --warmup 1 --cpu-tokens 0 --step-kernels-only\n")
            f.write(f"# clock = SQ_BUSY_CYCLES / {n_se} shader engines / dispatch duration; "
                    f"mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / {n_simd} SIMDs / busy cycles.\n")
            f.write("# Fraction of the 2.4 GHz dense INT8 peak = mfma_busy x clock / 2.4.\n")
            f.write(f"# {'kernel':<70} {'clock_GHz':>9} {'mfma_busy':>9} {'of_peak':>8} "
                    f"{'dur_us':>8} {'n':>3}\n")
            for k, (clk, busy, dur, n) in sorted(res.items(), key=lambda kv: -kv[1][2]):
                f.write(f"  {k[:70]:<70} {clk:>9.3f} {busy:>9.3f} {busy * clk / 2.4:>8.3f} "
                        f"{dur:>8.1f} {n:>3}\n")
        print(open(os.path.join(PROFILES, "mfma_busy_clock.txt")).read())
    if glob.glob(os.path.join(out_dir, "lds", "*counter_collection.csv")):
        lds_summary(out_dir)
    if glob.glob(os.path.join(out_dir, "valu", "*counter_collection.csv")):
        valu_summary(out_dir)
    if os.path.exists(os.path.join(out_dir, "power.txt")):
        power_summary(out_dir)
    if os.path.exists(os.path.join(out_dir, "power_ceiling.txt")):
        power_summary(out_dir, "power_ceiling.txt", "power_mfma_ceiling.txt",
                      "# Socket power and graphics clocks while the matrix-core ceiling kernel "
                      "runs back to back\n# (the products' MFMA sequence on random fragments, "
                      "no memory traffic).\n"
                      "#   python bench.py --mfma-ceiling-seconds 6 &  sleep 4;\n"
                      "#   10 x (amd-smi metric -p -c; sleep 0.2)\n")


def valu_summary(out_dir):
    """profiles/valu_issue.txt: per kernel, the vector instructions issued per
    dispatch and the time they take to issue at the kernel's own clock (a
    wave64 VALU instruction occupies its SIMD for 4 cycles), against the
    dispatch duration: where the two are close, the kernel is bound by its
    vector instructions as much as by memory."""
    path = _one(os.path.join(out_dir, "valu", "*counter_collection.csv"))
    info = list(csv.DictReader(open(_one(os.path.join(out_dir, "valu", "*agent_info.csv")))))
    gpu = [r for r in info if r["Agent_Type"] == "GPU"][0]
    n_se, n_simd = int(gpu["Array_Count"]), int(gpu["Simd_Count"])
    per = {}
    for r in csv.DictReader(open(path)):
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": _short(r["Kernel_Name"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    by = {}
    for d in per.values():
        if d["dur_s"] <= 0 or not d.get("SQ_BUSY_CYCLES") or "SQ_INSTS_VALU" not in d:
            continue
        clock = d["SQ_BUSY_CYCLES"] / n_se / d["dur_s"]
        issue_s = d["SQ_INSTS_VALU"] * 4 / n_simd / clock
        by.setdefault(d["name"], []).append((d["dur_s"] * 1e6, clock / 1e9, d["SQ_INSTS_VALU"],
                                             issue_s * 1e6))
    with open(os.path.join(PROFILES, "valu_issue.txt"), "w") as f:
        f.write("# Vector-instruction issue time per dispatch of the headline step's kernels.\n")
        f.write("#   rocprofv3 --pmc SQ_INSTS_VALU SQ_BUSY_CYCLES SQ_WAVES -d OUT/valu -o valu "
                "--output-format csv -- python bench.py --steps 2 --warmup 1 --cpu-tokens 0 "
                "--step-kernels-only\n")
        f.write(f"# valu_us = SQ_INSTS_VALU x 4 cycles / {n_simd} SIMDs / clock, clock = "
                f"SQ_BUSY_CYCLES / {n_se} shader engines / duration.\n")
        f.write(f"# {'kernel':<62} {'dur_us':>8} {'clock_GHz':>9} {'valu_insts':>11} "
                f"{'valu_us':>8} {'ratio':>6}\n")
        for k, vals in sorted(by.items(), key=lambda kv: -statistics.median(v[0] for v in kv[1])):
            dur, clk, ins, iss = (statistics.median(v[i] for v in vals) for i in range(4))
            f.write(f"  {k[:62]:<62} {dur:>8.1f} {clk:>9.3f} {ins:>11.0f} {iss:>8.1f} "
                    f"{iss / dur:>6.2f}\n")
    print(open(os.path.join(PROFILES, "valu_issue.txt")).read())


STEP_POWER_HEADER = ("# Socket power and graphics clocks while the headline step runs back to back.\n"
                     "#   python bench.py --steps 3000 --cpu-tokens 0 --step-kernels-only &  "
                     "sleep 4;\n"
                     "#   10 x (amd-smi metric -p -c; sleep 0.2)\n")


def power_summary(out_dir, src="power.txt", dst="power_headline_step.txt",
                  header=STEP_POWER_HEADER):
    """profiles/<dst> from the amd-smi samples in OUT/<src> (by default those
    taken while bench.py ran its timed steps)."""
    import re
    text = open(os.path.join(out_dir, src)).read()
    rows = []
    for block in text.split("--- sample")[1:]:
        p = re.search(r"SOCKET_POWER:\s*(\d+)", block)
        clocks = [int(c) for c in re.findall(r"GFX_\d+:\s+CLK:\s*(\d+)", block)]
        if p and clocks:
            rows.append((int(p.group(1)), min(clocks), max(clocks)))
    with open(os.path.join(PROFILES, dst), "w") as f:
        f.write(header)
        f.write("# The MI355X board power limit is 1400 W.\n")
        f.write(f"# {'sample':>6} {'socket_W':>9} {'gfx_clk_min_MHz':>16} {'gfx_clk_max_MHz':>16}\n")
        for i, (pw, lo, hi) in enumerate(rows):
            f.write(f"  {i + 1:>6} {pw:>9} {lo:>16} {hi:>16}\n")
    print(open(os.path.join(PROFILES, dst)).read())


def lds_summary(out_dir):
    """profiles/lds_bank_conflicts.txt: per kernel, LDS instructions and
    bank-conflict cycles per dispatch (OUT/lds from the command below)."""
    path = _one(os.path.join(out_dir, "lds", "*counter_collection.csv"))
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = _short(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    with open(os.path.join(PROFILES, "lds_bank_conflicts.txt"), "w") as f:
        f.write("# LDS activity per dispatch of the headline step's kernels.\n")
        f.write("#   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAVES "
                "-d OUT/lds -o lds --output-format csv -- python bench.py --steps 2 --warmup 1 "
                "--cpu-tokens 0 --step-kernels-only\n")
        f.write(f"# {'kernel':<70} {'lds_insts':>12} {'conflict_cyc':>12} {'waves':>7}\n")
        for k, d in sorted(vals.items(), key=lambda kv: -statistics.mean(
                kv[1].get("SQ_INSTS_LDS", [0]))):
            m = {c: statistics.mean(v) for c, v in d.items()}
            if m.get("SQ_INSTS_LDS", 0) == 0:
                continue
            f.write(f"  {k[:70]:<70} {m['SQ_INSTS_LDS']:>12.0f} "
                    f"{m['SQ_LDS_BANK_CONFLICT']:>12.0f} {m['SQ_WAVES']:>7.0f}\n")
    print(open(os.path.join(PROFILES, "lds_bank_conflicts.txt")).read())


if __name__ == "__main__":
    main(sys.argv[1])

"""Summaries of rocprofv3 CSV output for the GEMV, written under profiles/.

    python -m block_wise_int4_matmulnbits_amd.profiling trace DIR OUT.md CMD [TIMED]
        kernel stats and dispatch facts of a --kernel-trace --stats run;
        TIMED: dispatches of the bench's timed region (the last ones)
    python -m block_wise_int4_matmulnbits_amd.profiling traffic \\
        GEMV_FETCH GEMV_WRITE COPY_FETCH COPY_WRITE COPY_BYTES WORKLOAD M \\
        OUT.json OUT.md CMD...
        HBM bytes per GEMV launch from FETCH_SIZE and WRITE_SIZE passes
        (KiB per dispatch), each scaled by what the same counter reads for a
        device copy of COPY_BYTES, next to the algorithmic bytes.
    python -m block_wise_int4_matmulnbits_amd.profiling decode PROFROOT OUT.json OUT.md
        every decode configuration profiled under PROFROOT/<config>/{trace,
        fetch,write} (a --kernel-trace --stats run and FETCH_SIZE and
        WRITE_SIZE passes of bench.py on that configuration; each directory
        holds cmd.txt, the command that made it) and the device-copy
        calibration under PROFROOT/copy_{fetch,write}: kernel time, HBM bytes
        per launch and their fractions of 8 TB/s, per configuration.
    python -m block_wise_int4_matmulnbits_amd.profiling counters TAG TRACE_DIR \
        OUT.md FLOPS CMD_TRACE CMD_PMC PMC_DIR...
        duration statistics of the kernels whose name contains TAG in a
        --kernel-trace --stats run, and the per-dispatch mean of every counter
        of the --pmc runs in PMC_DIR... (FETCH_SIZE scaled by the device-copy
        factor of profiles/hbm_traffic.json), with the shader clock (GRBM_GUI_ACTIVE
        over the 8 XCDs) and the MFMA-busy share where counted.

Reads CSV only; runs nothing on the GPU.
"""
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMV_TAG = "mnb_gemv_kernel"
DECODE_TAG = "::mnb_ge"          # every GEMV/GEMM kernel of the library
PEAK_HBM_BYTES_PER_S = 8e12


def source_files():
    """Every source the kernels and the launch planner are built from."""
    root = os.path.dirname(HERE)
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*")))
    files.append(os.path.join(root, "include", "mnb.h"))
    return [f for f in files if os.path.isfile(f)]


def kernel_source_hash():
    """sha256[:16] over the kernel, device-helper, planner and header sources:
    a counter figure taken on other sources is stale."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def trace_summary(trace_dir, out_md, cmd, timed=0, tag=GEMV_TAG):
    """timed: the number of dispatches of the bench's timed region (the last
    ones traced; the warm-up dispatches come first).  tag: a substring of the
    kernel's name."""
    stats = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    trace = _one(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    with open(stats) as f:
        stats_text = f.read().strip()
    rows = [r for r in _rows(trace) if tag in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    r = rows[-1]
    facts = ("grid %s work-items, workgroup %s, arch VGPRs %s (as traced), SGPRs %s, "
             "LDS %s B, scratch %s B" % (r["Grid_Size_X"], r["Workgroup_Size_X"], r["VGPR_Count"],
                                         r["SGPR_Count"], r["LDS_Block_Size"], r["Scratch_Size"]))
    med = statistics.median(durs)
    with open(out_md, "w") as f:
        f.write("# %s\n\nCommand (repository root, one MI355X, libraries built in-tree):\n\n"
                "    %s\n\n`kernel_stats.csv`:\n\n```\n%s\n```\n\n" % (
                    r["Kernel_Name"], cmd, stats_text))
        f.write("GEMV dispatches traced: %d; median duration %.3f us "
                "(min %.3f, max %.3f).\n\n" % (len(durs), med, min(durs), max(durs)))
        if 0 < timed <= len(durs):
            t = durs[-timed:]
            f.write("Timed region (the last %d dispatches, after the bench's warm-up): "
                    "mean %.3f us, median %.3f us.\n\n" % (timed, statistics.mean(t),
                                                          statistics.median(t)))
        f.write("Dispatch: %s.\n" % facts)
    return med


def _per_dispatch(d, counter, tag=None):
    rows = _rows(_one(os.path.join(d, "**", "*counter_collection.csv")))
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and (tag is None or tag in r["Kernel_Name"])]
    return vals


def counters_summary(tag, trace_dir, out_md, flops, cmd_trace, cmd_pmc, pmc_dirs):
    trace = _one(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    rows = [r for r in _rows(trace) if tag in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    name = rows[-1]["Kernel_Name"]
    r = rows[-1]
    mean = statistics.mean(durs)
    vals = {}
    pmc_durs = []
    for d in pmc_dirs:
        crows = [x for x in _rows(_one(os.path.join(d, "**", "*counter_collection.csv")))
                 if tag in x["Kernel_Name"]]
        disp = {}
        for x in crows:
            disp.setdefault(x["Dispatch_Id"], {}).setdefault(x["Counter_Name"], 0.0)
            disp[x["Dispatch_Id"]][x["Counter_Name"]] += float(x["Counter_Value"])
            pmc_durs.append((int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) / 1e3)
        for c in {c for v in disp.values() for c in v}:
            if c == "GRBM_GUI_ACTIVE" and c in vals:
                continue
            vals[c] = statistics.mean(v[c] for v in disp.values() if c in v)
    with open(os.path.join(os.path.dirname(HERE), "profiles", "hbm_traffic.json")) as f:
        fetch_scale = json.load(f)["fetch_scale"]
    pmc_mean = statistics.mean(pmc_durs) if pmc_durs else float("nan")
    with open(out_md, "w") as f:
        f.write("# %s\n\n" % name)
        f.write("Commands (repository root, one MI355X, libraries built in-tree):\n\n")
        f.write("    %s\n" % cmd_trace)
        f.write("    %s   (one run per counter set below)\n\n" % cmd_pmc)
        f.write("Kernel trace: %d dispatches, mean %.2f us, median %.2f us (min %.2f, max %.2f); "
                "%.1f TFLOP/s at the mean (%.4g FLOP per call).\n\n"
                % (len(durs), mean, statistics.median(durs), min(durs), max(durs),
                   flops / (mean * 1e-6) / 1e12, flops))
        f.write("Dispatch: grid %s work-items, workgroup %s, arch VGPRs %s, accumulation VGPRs %s, "
                "LDS %s B, scratch %s B.\n\n"
                % (r["Grid_Size_X"], r["Workgroup_Size_X"], r["VGPR_Count"],
                   r.get("Accum_VGPR_Count", "?"), r["LDS_Block_Size"], r["Scratch_Size"]))
        f.write("Counters, mean per dispatch over the counter runs (kernel mean %.2f us under "
                "counting):\n\n| counter | value |\n|---|---|\n" % pmc_mean)
        for c in sorted(vals):
            f.write("| %s | %.6g |\n" % (c, vals[c]))
        f.write("\nDerived:\n\n")
        if "GRBM_GUI_ACTIVE" in vals:
            ghz = vals["GRBM_GUI_ACTIVE"] / 8 / (pmc_mean * 1e3)
            if ghz <= 2.45:
                f.write("- shader clock: %.2f GHz (GRBM_GUI_ACTIVE / 8 XCDs / kernel time)\n" % ghz)
            else:   # the counter spans more than a short kernel: no clock
                f.write("- GRBM_GUI_ACTIVE / 8 XCDs / kernel time: %.2f GHz, above the part's 2.4 GHz: on a "
                        "launch this short the counter spans more than the kernel, so it gives no clock "
                        "(and no MFMA-busy fraction)\n" % ghz)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals and \
                vals["GRBM_GUI_ACTIVE"] / 8 / (pmc_mean * 1e3) <= 2.45:
            f.write("- MFMA busy: %.1f%% of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs)\n"
                    % (100 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (vals["GRBM_GUI_ACTIVE"] / 8 * 1024)))
        if "SQ_INSTS_VALU" in vals and vals.get("SQ_INSTS_MFMA", 0) > 0:
            f.write("- other VALU instructions per MFMA: %.2f\n"
                    % ((vals["SQ_INSTS_VALU"] - vals["SQ_INSTS_MFMA"]) / vals["SQ_INSTS_MFMA"]))
        if vals.get("SQ_WAVES", 0) > 0:
            f.write("- waves: %d, %.2f per SIMD of the 1024 over the dispatch\n"
                    % (vals["SQ_WAVES"], vals["SQ_WAVES"] / 1024))
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM"):
                if c in vals:
                    f.write("- %s per wave: %.0f\n" % (c, vals[c] / vals["SQ_WAVES"]))
        if vals.get("SQ_WAVE_CYCLES", 0) > 0 and "SQ_WAIT_ANY" in vals:
            f.write("- waiting: SQ_WAIT_ANY / SQ_WAVE_CYCLES = %.0f%% of wave cycles\n"
                    % (100 * vals["SQ_WAIT_ANY"] / vals["SQ_WAVE_CYCLES"]))
        if "FETCH_SIZE" in vals:
            f.write("- HBM fetch: %.1f MB per call (FETCH_SIZE KiB x 1024 x %.4f, the device-copy "
                    "factor of profiles/hbm_traffic.json)\n"
                    % (vals["FETCH_SIZE"] * 1024 * fetch_scale / 1e6, fetch_scale))
        if "WRITE_SIZE" in vals:
            f.write("- HBM write: %.1f MB per call\n" % (vals["WRITE_SIZE"] * 1024 / 1e6))
    return mean


def _cmd(d):
    try:
        with open(os.path.join(d, "cmd.txt")) as f:
            return f.read().strip()
    except OSError:
        return "(command not recorded)"


def _durations(trace_dir, tag):
    rows = [r for r in _rows(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))
            if tag in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows, [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]


def kernel_short_name(full):
    """'mnb_gemv_kernel<1, 2, 2, 1>' from a demangled rocprofv3 kernel name."""
    import re
    m = re.search(r"(mnb_\w+)(<[^>]*>)?\(", full)
    return (m.group(1) + (m.group(2) or "")) if m else full


def decode_summary(root, out_json, out_md, timed=500):
    """Per decode configuration (a subdirectory of root named
    workload:m:out_dtype): the mean kernel time of the last `timed`
    dispatches of the trace run, FETCH_SIZE and WRITE_SIZE per dispatch
    (median) scaled by the device-copy factors, and the fractions of
    8 TB/s they make."""
    sys.path.insert(0, os.path.dirname(HERE))
    from block_wise_int4_matmulnbits_amd import workloads as W
    kib = 1024.0
    copy = {}
    for kind, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        d = os.path.join(root, "copy_" + kind)
        with open(os.path.join(d, "bytes.txt")) as f:
            nbytes = int(f.read())
        copy[kind] = {"scale": nbytes / (max(_per_dispatch(d, counter)) * kib),
                      "bytes": nbytes, "cmd": _cmd(d)}
    out = {"kernel_src_sha256_16": kernel_source_hash(),
           "fetch_scale": copy["fetch"]["scale"], "write_scale": copy["write"]["scale"],
           "copy_bytes": copy["fetch"]["bytes"], "configs": {}}
    lines = []
    for key in sorted(os.listdir(root)):
        d = os.path.join(root, key)
        if key.startswith("copy_") or not os.path.isdir(d):
            continue
        name, m, odt = key.split(":")
        m = int(m)
        w = W.WORKLOADS[name]
        alg = w.bytes_per_call(m)
        rows, durs = _durations(os.path.join(d, "trace"), DECODE_TAG)
        t = durs[-timed:] if len(durs) >= timed else durs
        mean_us = statistics.mean(t)
        fetch = statistics.median(_per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE", DECODE_TAG)) \
            * kib * copy["fetch"]["scale"]
        write = statistics.median(_per_dispatch(os.path.join(d, "write"), "WRITE_SIZE", DECODE_TAG)) \
            * kib * copy["write"]["scale"]
        r = rows[-1]
        e = {"workload": name, "m": m, "out_dtype": odt, "K": w.K, "N": w.N,
             "kernel": kernel_short_name(r["Kernel_Name"]),
             "dispatches_traced": len(durs), "timed_dispatches": len(t),
             "kernel_mean_us": round(mean_us, 3), "kernel_median_us": round(statistics.median(t), 3),
             "algorithmic_bytes": alg, "fetch_bytes": round(fetch), "write_bytes": round(write),
             "alg_frac_of_8TBs": round(alg / (mean_us * 1e-6) / PEAK_HBM_BYTES_PER_S, 4),
             "fetch_frac_of_8TBs": round(fetch / (mean_us * 1e-6) / PEAK_HBM_BYTES_PER_S, 4),
             "fetch_over_alg": round(fetch / alg, 4),
             # rocprofv3 decodes the descriptor's VGPR blocks with a granule of
             # 4 where gfx950 allocates wave64 VGPRs in 8s: twice the traced
             # figure is the allocation (75 registers -> 80 -> 40 traced).
             "vgprs_traced": int(r["VGPR_Count"]), "vgprs_allocated": 2 * int(r["VGPR_Count"]),
             "accum_vgprs_traced": int(r.get("Accum_VGPR_Count") or 0),
             "grid": int(r["Grid_Size_X"]), "workgroup": int(r["Workgroup_Size_X"]),
             "lds_bytes": int(r["LDS_Block_Size"]),
             "cmd_trace": _cmd(os.path.join(d, "trace")), "cmd_fetch": _cmd(os.path.join(d, "fetch")),
             "cmd_write": _cmd(os.path.join(d, "write"))}
        out["configs"][key] = e
        lines.append("| %s | %d | %s | `%s` | %.2f | %.2f | %d | %.4f | %.1f%% | %.1f%% | %d (%d) | %d x %d |" % (
            name, m, odt, e["kernel"], e["kernel_mean_us"], e["kernel_median_us"], alg,
            e["fetch_over_alg"], 100 * e["alg_frac_of_8TBs"], 100 * e["fetch_frac_of_8TBs"],
            e["vgprs_traced"], e["vgprs_allocated"], e["grid"] // e["workgroup"], e["workgroup"]))
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(out_md, "w") as f:
        f.write("# Decode configurations: rocprofv3 kernel time and HBM traffic\n\n")
        f.write("One MI355X; kernel sources sha256[:16] %s.  Per configuration, a `--kernel-trace "
                "--stats` run of bench.py on it (mean of the last %d dispatches, the timed region), then "
                "a `--pmc FETCH_SIZE` and a `--pmc WRITE_SIZE` run (median KiB per dispatch), each "
                "scaled by what the same counter reads for a device copy of %d bytes (fetch factor "
                "%.4f, write factor %.4f).  Fractions are of 8 TB/s.  VGPRs: as traced (rocprofv3 "
                "decodes the descriptor with a granule of 4; gfx950 allocates wave64 VGPRs in 8s, so the "
                "allocation, in brackets, is twice the traced figure).\n\n"
                % (out["kernel_src_sha256_16"], timed, out["copy_bytes"], out["fetch_scale"],
                   out["write_scale"]))
        f.write("| workload | m | out | kernel | mean us | median us | algorithmic B | fetch / alg "
                "| alg GB/s frac | FETCH frac | VGPRs traced (allocated) | grid x wg |\n"
                "|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        f.write("\n".join(lines) + "\n\nCommands (repository root; `$REPO` is its path):\n\n")
        for key, e in out["configs"].items():
            f.write("- %s:\n    - `%s`\n    - `%s`\n    - `%s`\n" % (key, e["cmd_trace"], e["cmd_fetch"],
                                                               e["cmd_write"]))
        f.write("- copy calibration:\n    - `%s`\n    - `%s`\n" % (copy["fetch"]["cmd"], copy["write"]["cmd"]))
    return out


def main(argv):
    if argv[0] == "trace":
        print(trace_summary(argv[1], argv[2], argv[3], int(argv[4]) if len(argv) > 4 else 0,
                            argv[5] if len(argv) > 5 else GEMV_TAG))
    elif argv[0] == "counters":
        tag, tdir, out_md, flops, cmd_t, cmd_p = argv[1:7]
        print(counters_summary(tag, tdir, out_md, float(flops), cmd_t, cmd_p, argv[7:]))
    elif argv[0] == "decode":
        print(json.dumps(decode_summary(argv[1], argv[2], argv[3]), indent=1))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])

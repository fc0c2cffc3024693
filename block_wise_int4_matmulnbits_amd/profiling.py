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
    python -m block_wise_int4_matmulnbits_amd.profiling counters TAG TRACE_DIR \
        OUT.md FLOPS CMD_TRACE CMD_PMC PMC_DIR...
        duration statistics of the kernels whose name contains TAG in a
        --kernel-trace --stats run, and the per-dispatch mean of every counter
        of the --pmc runs in PMC_DIR... (FETCH_SIZE scaled by the factor of
        profiles/lm_head_traffic.json), with the shader clock (GRBM_GUI_ACTIVE
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
KERNEL_SRC = os.path.join(HERE, "csrc", "mnb_gemv.hip")
GEMV_TAG = "mnb_gemv_kernel"


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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


def traffic_summary(gemv_fetch, gemv_write, copy_fetch, copy_write, copy_bytes, workload, m,
                    out_json, out_md, cmd):
    sys.path.insert(0, os.path.dirname(HERE))
    from block_wise_int4_matmulnbits_amd import workloads as W
    w = W.WORKLOADS[workload]
    alg = w.bytes_per_call(m)
    kib = 1024.0
    gf = statistics.median(_per_dispatch(gemv_fetch, "FETCH_SIZE", GEMV_TAG)) * kib
    gw = statistics.median(_per_dispatch(gemv_write, "WRITE_SIZE", GEMV_TAG)) * kib
    # the copy: largest dispatch of the run is the copy of copy_bytes
    cf = max(_per_dispatch(copy_fetch, "FETCH_SIZE")) * kib
    cw = max(_per_dispatch(copy_write, "WRITE_SIZE")) * kib
    f_scale = copy_bytes / cf
    w_scale = copy_bytes / cw
    fetch = gf * f_scale
    write = gw * w_scale
    out = {"workload": workload, "m": m, "kernel_src_sha256_16": kernel_source_hash(),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "hbm_bytes_per_launch": round(fetch + write), "algorithmic_bytes_per_launch": alg,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "raw_fetch_kib": gf / kib, "raw_write_kib": gw / kib,
           "copy_bytes": copy_bytes, "copy_fetch_kib": cf / kib, "copy_write_kib": cw / kib}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(out_md, "w") as f:
        f.write("# HBM traffic of one GEMV launch, %s (m=%d, K=%d, N=%d)\n\n" % (
            workload, m, w.K, w.N))
        f.write("Commands (repository root, one MI355X):\n\n%s\n\n" % "\n".join(
            "    " + c for c in cmd))
        f.write("| | raw counter (KiB/dispatch) | scale (copy of %d B) | bytes |\n|---|---|---|---|\n"
                % copy_bytes)
        f.write("| FETCH_SIZE | %.1f | %.4f | %d |\n" % (gf / kib, f_scale, fetch))
        f.write("| WRITE_SIZE | %.1f | %.4f | %d |\n" % (gw / kib, w_scale, write))
        f.write("\nAlgorithmic bytes per launch: %d.  Measured / algorithmic: fetch %.4f, "
                "total %.4f.  Kernel source sha256[:16] %s.\n" % (
                    alg, fetch / alg, (fetch + write) / alg, out["kernel_src_sha256_16"]))
    return out


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
    with open(os.path.join(os.path.dirname(HERE), "profiles", "lm_head_traffic.json")) as f:
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
            f.write("- shader clock: %.2f GHz (GRBM_GUI_ACTIVE / 8 XCDs / kernel time)\n"
                    % (vals["GRBM_GUI_ACTIVE"] / 8 / (pmc_mean * 1e3)))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
            f.write("- MFMA busy: %.1f%% of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs)\n"
                    % (100 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (vals["GRBM_GUI_ACTIVE"] / 8 * 1024)))
        if "SQ_INSTS_VALU" in vals and "SQ_INSTS_MFMA" in vals:
            f.write("- other VALU instructions per MFMA: %.2f\n"
                    % ((vals["SQ_INSTS_VALU"] - vals["SQ_INSTS_MFMA"]) / vals["SQ_INSTS_MFMA"]))
        if "FETCH_SIZE" in vals:
            f.write("- HBM fetch: %.1f MB per call (FETCH_SIZE KiB x 1024 x %.4f, the device-copy "
                    "factor of profiles/lm_head_traffic.json)\n"
                    % (vals["FETCH_SIZE"] * 1024 * fetch_scale / 1e6, fetch_scale))
        if "WRITE_SIZE" in vals:
            f.write("- HBM write: %.1f MB per call\n" % (vals["WRITE_SIZE"] * 1024 / 1e6))
    return mean


def main(argv):
    if argv[0] == "trace":
        print(trace_summary(argv[1], argv[2], argv[3], int(argv[4]) if len(argv) > 4 else 0,
                            argv[5] if len(argv) > 5 else GEMV_TAG))
    elif argv[0] == "counters":
        tag, tdir, out_md, flops, cmd_t, cmd_p = argv[1:7]
        print(counters_summary(tag, tdir, out_md, float(flops), cmd_t, cmd_p, argv[7:]))
    elif argv[0] == "traffic":
        (gf, gw, cf, cw, cb, wl, m, oj, om) = argv[1:10]
        print(json.dumps(traffic_summary(gf, gw, cf, cw, int(cb), wl, int(m), oj, om, argv[10:])))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])

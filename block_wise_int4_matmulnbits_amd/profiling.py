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


def trace_summary(trace_dir, out_md, cmd, timed=0):
    """timed: the number of dispatches of the bench's timed region (the last
    ones traced; the warm-up dispatches come first)."""
    stats = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    trace = _one(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    with open(stats) as f:
        stats_text = f.read().strip()
    rows = [r for r in _rows(trace) if GEMV_TAG in r["Kernel_Name"]]
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


def main(argv):
    if argv[0] == "trace":
        print(trace_summary(argv[1], argv[2], argv[3], int(argv[4]) if len(argv) > 4 else 0))
    elif argv[0] == "traffic":
        (gf, gw, cf, cw, cb, wl, m, oj, om) = argv[1:10]
        print(json.dumps(traffic_summary(gf, gw, cf, cw, int(cb), wl, int(m), oj, om, argv[10:])))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])

#!/usr/bin/env python3
"""Benchmark of the block-wise INT4 MatMulNBits decode GEMV on one MI355X.

One step = one matmul_nbits launch (the whole path: activation staging,
weight streaming, unpack and zero-point subtract, dot and scale, split-K
reduction, fp16 rounding and direct bf16 narrowing store) on the lm_head
shape, m=1, K=4096, N=151936, fp16 activations, asymmetric zero points,
bf16 output.  Weights, scales and zero points are rotated over enough copies
(>= 512 MB) that the 256 MB last-level cache cannot serve them; every input
is resident in HBM before the timed region starts.

Prints one JSON line.  value = algorithmic bytes per call / time per call
(GB/s); roofline.traffic comes from the committed rocprofv3 counter summary
for the current kernel source (null if the kernel changed since).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "m=1 INT4 GEMV achieved HBM GB/s (% of MI355X peak) and µs/call"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(workload_name, m):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source, workload and row count."""
    from block_wise_int4_matmulnbits_amd import profiling
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_src_sha256_16") != profiling.kernel_source_hash()
            or t.get("workload") != workload_name or t.get("m") != m):
        return None
    return t.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="lm_head")
    ap.add_argument("--m", type=int, default=None, help="rows (default: the workload's)")
    ap.add_argument("--out-dtype", default="bf16", choices=["f16", "bf16"])
    ap.add_argument("--rotate-mb", type=int, default=512,
                    help="minimum bytes of rotated weight copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run torch's device copy of this many MiB "
                         "(reference kernel for scaling HBM counters)")
    return ap.parse_args()


def calib_copy(mib, reps=5):
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "reps": reps}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the decode GEMV shards by output "
              "columns with no exchange between GPUs, and multi-GPU runs are not "
              "part of this build (asked for --gpus %d, WORLD_SIZE=%d)"
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)
        return

    import numpy as np
    import torch

    import block_wise_int4_matmulnbits_amd as mnb
    from block_wise_int4_matmulnbits_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = W.WORKLOADS[args.workload]
    m = w.m if args.m is None else args.m
    out_dtype = W.BF16 if args.out_dtype == "bf16" else W.F16
    t0 = time.time()
    d = W.generate_workload(w, m)
    log("[bench] generated %s inputs in %.1f s" % (w.name, time.time() - t0))

    dev = torch.device("cuda:0")
    bytes_per_call = w.bytes_per_call(m)
    weight_bytes = d["B"].nbytes + d["scales"].nbytes + (d["zp"].nbytes if d["zp"] is not None else 0)
    R = max(1, math.ceil(args.rotate_mb * 1e6 / weight_bytes))
    adt = torch.bfloat16 if w.a_dtype == W.BF16 else torch.float16
    A = torch.from_numpy(np.ascontiguousarray(d["A"][:m]).view(np.int16)).to(dev).view(adt)
    B0 = torch.from_numpy(d["B"]).to(dev)
    S0 = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    Z0 = None if d["zp"] is None else torch.from_numpy(d["zp"]).to(dev)
    copies = [(B0, S0, Z0)] + [(B0.clone(), S0.clone(), None if Z0 is None else Z0.clone())
                               for _ in range(R - 1)]
    out = torch.empty((m, w.N), dtype=torch.bfloat16 if out_dtype == W.BF16 else torch.float16,
                      device=dev)
    stream = torch.cuda.current_stream(dev)
    L = mnb.lib()
    a_dt = W.BF16 if w.a_dtype == W.BF16 else W.F16
    raw = [(A.data_ptr(), a_dt, m, w.K, w.N, b.data_ptr(), s.data_ptr(),
            z.data_ptr() if z is not None else None, 32, out.data_ptr(), out_dtype,
            stream.cuda_stream) for (b, s, z) in copies]
    call = L.matmul_nbits

    def step(i):
        st = call(*raw[i % R])
        if st != 0:
            raise mnb.MnbError(st, L)

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    plan = mnb.plan_for_device(m, w.K, w.N, cus)
    info = mnb.mnb_get_kernel_info(m, w.K, plan)
    log("[bench] plan %s kernel %s rotated copies %d" % (plan.as_dict(), info, R))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    c0 = mnb.mnb_counters_get()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    c1 = mnb.mnb_counters_get()
    assert c1["launches"] - c0["launches"] == args.steps
    if out_dtype == W.BF16:
        assert c1["elements_bf16_direct"] - c0["elements_bf16_direct"] == args.steps * m * w.N
    ms = ev0.elapsed_time(ev1) / args.steps
    us = ms * 1e3
    gbs = bytes_per_call / (ms * 1e-3) / 1e9
    log("[bench] %d steps: %.3f us/call (events), wall %.3f us/call, %.1f GB/s = %.1f%% of %.0f"
        % (args.steps, us, wall / args.steps * 1e6, gbs, 100 * gbs / PEAK_HBM_GBS, PEAK_HBM_GBS))

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_call": round(us, 3),
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xf16->f32",
        "data": "synthetic (seeded; no model weights)",
        "config": {
            "workload": w.name, "m": m, "K": w.K, "N": w.N, "block": 32,
            "a_dtype": "bf16" if w.a_dtype == W.BF16 else "f16",
            "out_dtype": args.out_dtype, "zero_points": w.asym,
            "bytes_per_call": bytes_per_call, "rotated_copies": R,
            "plan": plan.as_dict(), "vgprs": info["vgprs"],
            "wgs_per_cu": info["wgs_per_cu"],
            "waves_per_cu": info["wgs_per_cu"] * plan.threads_per_wg // 64,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(w.name, m),
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], parity = cpu_baseline(args, w, d, m, A, copies[0], out_dtype,
                                                      bytes_per_call)
        result["parity_vs_oracle"] = parity
    print(json.dumps(result), flush=True)


def cpu_baseline(args, w, d, m, A, copy0, out_dtype, bytes_per_call):
    """The oracle, as it stands, timed on the host cores over whole calls of
    the same workload for about --cpu-seconds; also checks copy 0 of the GPU
    output against it."""
    import numpy as np
    import torch

    import block_wise_int4_matmulnbits_amd as mnb
    import oracle
    from block_wise_int4_matmulnbits_amd import workloads as W

    threads = oracle.max_threads()
    n, t0 = 0, time.perf_counter()
    while True:
        ref = oracle.matmul_nbits(d["A"][:m], w.a_dtype == W.BF16, d["B"], d["scales"],
                                  d["zp"], m, w.K, w.N, threads=threads)
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    cpu_gbs = n * bytes_per_call / el / 1e9
    log("[bench] oracle: %d calls in %.1f s on %d threads = %.3f GB/s" % (n, el, threads, cpu_gbs))
    # parity of the timed configuration's output (copy 0)
    B, S, Z = copy0
    y16 = torch.empty((m, w.N), dtype=torch.float16, device=A.device)
    ybf = torch.empty((m, w.N), dtype=torch.bfloat16, device=A.device)
    mnb.matmul_nbits(A, B, S, Z, y16)
    mnb.matmul_nbits(A, B, S, Z, ybf)
    torch.cuda.synchronize()
    g16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    gbf = ybf.view(torch.int16).cpu().numpy().view(np.uint16)
    g = g16.view(np.float16).astype(np.float64)
    o = ref["f16"].view(np.float16).astype(np.float64)
    ulp = oracle.f16_ulp(ref["f16"])
    ok1 = bool(np.all(np.abs(g - o) <= 1e-3 * ref["abs"] + ulp))
    ok2 = bool(np.array_equal(gbf, oracle.f16_to_bf16(g16.ravel()).reshape(g16.shape)))
    parity = {"check1": ok1, "check2_bf16_bit_exact": ok2,
              "max_err_fp16_ulp": float(np.max(np.abs(g - o) / ulp)),
              "bit_equal_frac": float(np.mean(g16 == ref["f16"]))}
    log("[bench] parity vs oracle: %s" % parity)
    base = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d whole %s calls (m=%d, K=%d, N=%d) in %.1f s, fp64 C oracle, "
                      "OpenMP over columns" % (n, w.name, m, w.K, w.N, el),
            "ms_per_call": round(el / n * 1e3, 2)}
    return base, parity


if __name__ == "__main__":
    main()

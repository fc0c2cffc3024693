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
(profiles/hbm_traffic.json) for the current kernel sources (null if any of
them changed since).

Besides the headline figure the line carries (skipped with --no-extras):
  attainable   a read-only streaming kernel over the same bytes (the in-repo
               probe): what one launch of this size can pull from HBM;
  launch_floor_us  the read probe over one 16-byte piece, launched back to
               back (one workgroup, and one per CU): the cost of a launch
               before it moves a byte;
  configs      every synthetic configuration in its own output type(s):
               microseconds per call (median and range of 5 timed passes),
               algorithmic GB/s and fraction of 8 TB/s, the read probe over
               the same weight copies and the fraction of it reached, the
               plan, VGPRs and occupancy, and the rocprofv3 kernel time and
               FETCH_SIZE fraction of the committed profile;
  staged_route the fp16 GEMV followed by a separate fp16 -> bf16 cast launch,
               against the direct bf16 store (bits compared);
  decode_step  a decode step of GEMVs (4 layers of q/k/v/o, gate_up and down,
               then the lm_head), launched eagerly and as one captured HIP
               graph (outputs compared);
  offline_layout  the natural layout against the offline odd/even nibble
               layout (converted once by mnb_repack_weights);
  prefill      m = 512 and 2048 rows on the gate_up and down shapes (the
               matrix-core tile kernel), TFLOP/s against the fp16 peak.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "m=1 INT4 GEMV achieved HBM GB/s (% of MI355X peak) and µs/call"
PEAK_HBM_GBS = 8000.0
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_FP16_MFMA_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# The synthetic configurations: workload, rows, output types.
CONFIGS = [("tiny_1k", 1, ("f16",)), ("asym_4k", 1, ("f16",)), ("gate_up_bf16", 1, ("bf16",)),
           ("down_rows_bf16", 2, ("bf16",)), ("down_rows_bf16", 4, ("bf16",)),
           ("down_rows_bf16", 8, ("bf16",)), ("lm_head", 1, ("f16", "bf16"))]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_profile(workload_name, m, out_dtype):
    """The committed rocprofv3 record of one configuration (kernel time,
    FETCH_SIZE and WRITE_SIZE bytes per launch), if it was taken on the
    current kernel sources; else None."""
    from block_wise_int4_matmulnbits_amd import profiling
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha256_16") != profiling.kernel_source_hash():
        return None
    return t.get("configs", {}).get("%s:%d:%s" % (workload_name, m, out_dtype))


def measured_traffic(workload_name, m, out_dtype="bf16"):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of a
    configuration from the committed profile, or None."""
    e = measured_profile(workload_name, m, out_dtype)
    return None if e is None else e["fetch_bytes"] + e["write_bytes"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="lm_head")
    ap.add_argument("--m", type=int, default=None, help="rows (default: the workload's)")
    ap.add_argument("--out-dtype", default="bf16", choices=["f16", "bf16"])
    ap.add_argument("--rotate-mb", type=int, default=512,
                    help="minimum bytes of rotated weight copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline GEMV only (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="seconds of whole oracle calls on every usable core")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run torch's device copy of this many MiB "
                         "(reference kernel for scaling HBM counters)")
    ap.add_argument("--prefill-only", default=None, metavar="SHAPE:M",
                    help="only run one prefill shape (gate_up or down, M rows) "
                         "--warmup + --steps times under its default plan "
                         "(profiling runs)")
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


class Resident:
    """One workload's inputs in device memory, with rotated weight copies."""

    def __init__(self, w, m, out_dtype, rotate_mb, d=None):
        import numpy as np
        import torch
        from block_wise_int4_matmulnbits_amd import workloads as W
        self.w, self.m = w, m
        d = W.generate_workload(w, m) if d is None else d
        self.d = d
        dev = torch.device("cuda:0")
        weight_bytes = d["B"].nbytes + d["scales"].nbytes + (
            d["zp"].nbytes if d["zp"] is not None else 0)
        self.R = max(1, math.ceil(rotate_mb * 1e6 / weight_bytes))
        adt = torch.bfloat16 if w.a_dtype == W.BF16 else torch.float16
        self.A = torch.from_numpy(np.ascontiguousarray(d["A"][:m]).view(np.int16)).to(dev).view(adt)
        B0 = torch.from_numpy(d["B"]).to(dev)
        S0 = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
        Z0 = None if d["zp"] is None else torch.from_numpy(d["zp"]).to(dev)
        self.copies = [(B0, S0, Z0)] + [
            (B0.clone(), S0.clone(), None if Z0 is None else Z0.clone()) for _ in range(self.R - 1)]
        self.out_dtype = out_dtype
        self.out = torch.empty((m, w.N), dtype=torch.bfloat16 if out_dtype == W.BF16 else torch.float16,
                               device=dev)
        self.a_dt = W.BF16 if w.a_dtype == W.BF16 else W.F16
        self.bytes_per_call = w.bytes_per_call(m)

    def raw(self, stream, out=None, out_dtype=None):
        out = self.out if out is None else out
        out_dtype = self.out_dtype if out_dtype is None else out_dtype
        return [(self.A.data_ptr(), self.a_dt, self.m, self.w.K, self.w.N, b.data_ptr(),
                 s.data_ptr(), z.data_ptr() if z is not None else None, 32, out.data_ptr(),
                 out_dtype, stream) for (b, s, z) in self.copies]


def plan_fields(plan):
    """The fields of a decode plan that its engine reads."""
    keys = {0: ("lanes_per_col", "blocks_per_lane", "cols_per_tile", "workgroups"),
            3: ("waves_per_wg", "blocks_per_lane", "cols_per_tile", "workgroups", "a_via_lds")}
    d = plan.as_dict()
    return dict({"engine": d["engine"]}, **{k: d[k] for k in keys.get(d["engine"], ())})


def event_time_us(stream, fn, n):
    """Mean microseconds per fn() over n calls, HIP events on `stream`."""
    import torch
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(n):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n * 1e3


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
    if args.prefill_only:
        prefill_only(args)
        return

    import torch

    import block_wise_int4_matmulnbits_amd as mnb
    from block_wise_int4_matmulnbits_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = W.WORKLOADS[args.workload]
    m = w.m if args.m is None else args.m
    out_dtype = W.BF16 if args.out_dtype == "bf16" else W.F16
    t0 = time.time()
    res = Resident(w, m, out_dtype, args.rotate_mb)
    log("[bench] generated %s inputs in %.1f s" % (w.name, time.time() - t0))

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    L = mnb.lib()
    raw = res.raw(stream.cuda_stream)
    R = res.R
    call = L.matmul_nbits

    def step(i):
        st = call(*raw[i % R])
        if st != 0:
            raise mnb.MnbError(st, L)

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    plan = mnb.plan_for_device(m, w.K, w.N, cus)
    info = mnb.mnb_get_kernel_info(m, w.K, plan)
    log("[bench] plan %s kernel %s rotated copies %d" % (plan.as_dict(), info, R))

    # Untimed warm-up: the first few hundred launches of a sustained run see
    # the clocks settle; the timed region measures the steady state.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    c0 = mnb.mnb_counters_get()
    wall0 = time.perf_counter()
    us = event_time_us(stream, step, args.steps)
    wall = time.perf_counter() - wall0
    c1 = mnb.mnb_counters_get()
    assert c1["launches"] - c0["launches"] == args.steps
    if out_dtype == W.BF16:
        assert c1["elements_bf16_direct"] - c0["elements_bf16_direct"] == args.steps * m * w.N
    ms = us * 1e-3
    bytes_per_call = res.bytes_per_call
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
            "traffic": measured_traffic(w.name, m, args.out_dtype),
        },
        "cpu_baseline": None,
    }

    if not args.no_extras:
        att = attainable(res, stream, cus)
        if att:
            result["roofline"]["attainable"] = att
            result["roofline"]["frac_of_attainable"] = round(gbs / att["gbs"], 4)
        result["launch_floor_us"] = launch_floor(stream, cus)
        result["configs"] = decode_configs(args, stream, cus)
        if w.name == "lm_head" and m == 1:
            result["staged_route"] = staged_route(res, stream, L)
        result["decode_step"] = decode_step(args, stream, L)
        result["prefill"] = prefill(stream, L, cus, args.rotate_mb)
        result["offline_layout"] = offline_layout(args, stream, L, cus)

    if not args.no_cpu_baseline:
        result["cpu_baseline"], parity = cpu_baseline(args, w, res.d, m, res.A, res.copies[0],
                                                      out_dtype, bytes_per_call)
        result["parity_vs_oracle"] = parity
    print(json.dumps(result), flush=True)


def attainable(res, stream, cus):
    """The in-repo read-only streaming kernel over the packed weights of the
    rotated copies (the bulk of the GEMV's bytes), best of a few launch
    shapes: the bandwidth one launch of this size can draw."""
    path = os.path.join(ROOT, "block_wise_int4_matmulnbits_amd", "libmnb_probe.so")
    if not os.path.exists(path):
        return None
    import torch
    P = ctypes.CDLL(path)
    P.mnb_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    bufs = [b for (b, _, _) in res.copies]
    n = bufs[0].numel() // 16 * 16
    best = None
    for unroll, per_cu in ((-1, 8), (-4, 2), (-2, 4)):
        wg = cus * per_cu
        sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")

        def go(i):
            P.mnb_probe_read(bufs[i % len(bufs)].data_ptr(), n, sink.data_ptr(), wg, unroll,
                             stream.cuda_stream)
        for i in range(20):
            go(i)
        us = event_time_us(stream, go, 200)
        if best is None or us < best[0]:
            best = (us, unroll, per_cu)
    gbs = n / (best[0] * 1e-6) / 1e9
    log("[bench] attainable read: %d B in %.2f us = %.1f GB/s" % (n, best[0], gbs))
    return {"gbs": round(gbs, 1), "bytes": n, "us": round(best[0], 3),
            "kernel": "read probe, unroll %d, %d workgroups/CU" % (best[1], best[2])}


def launch_floor(stream, cus):
    """Microseconds per launch of the read probe over one 16-byte piece,
    launched back to back on one stream: with one workgroup, and with one
    per CU (each of its threads past the piece loads nothing).  What any
    launch on this stream costs before it moves a byte."""
    path = os.path.join(ROOT, "block_wise_int4_matmulnbits_amd", "libmnb_probe.so")
    if not os.path.exists(path):
        return None
    import torch
    P = ctypes.CDLL(path)
    P.mnb_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    buf = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = {}
    for key, wg in (("one_workgroup", 1), ("one_per_cu", cus)):
        sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")

        def go(i):
            P.mnb_probe_read(buf.data_ptr(), 16, sink.data_ptr(), wg, 1, stream.cuda_stream)
        for i in range(100):
            go(i)
        out[key] = round(sorted(event_time_us(stream, go, 2000) for _ in range(3))[1], 3)
    log("[bench] launch floor: %s us" % out)
    return out


def decode_configs(args, stream, cus, passes=5):
    """Every synthetic configuration in its own output type(s), default
    plan, rotated weight copies (the 1024 x 1024 one stays cache-resident):
    microseconds per call as the median and range of `passes` timed passes,
    algorithmic GB/s, the read probe over the same weight copies (and the
    fraction of it reached), the plan, VGPRs and occupancy, and the committed
    rocprofv3 kernel time and FETCH_SIZE fraction when they were taken on
    the current sources."""
    import block_wise_int4_matmulnbits_amd as mnb
    from block_wise_int4_matmulnbits_amd import workloads as W
    out = {}
    L = mnb.lib()
    shared = {}
    for name, m, odts in CONFIGS:
        w = W.WORKLOADS[name]
        if name not in shared:
            shared.clear()
            shared[name] = W.generate_workload(w, max(w.m_max, 8) if name == "down_rows_bf16" else w.m)
        for odt in odts:
            res = Resident(w, m, W.BF16 if odt == "bf16" else W.F16,
                           0 if name == "tiny_1k" else args.rotate_mb, d=shared[name])
            raw = res.raw(stream.cuda_stream)

            def go(i):
                st = L.matmul_nbits(*raw[i % len(raw)])
                if st != 0:
                    raise mnb.MnbError(st, L)
            for i in range(200):
                go(i)
            n = max(200, int(0.05 / (res.bytes_per_call / 5e12)))
            samples = sorted(event_time_us(stream, go, n) for _ in range(passes))
            us = samples[len(samples) // 2]
            plan = mnb.plan_for_device(m, w.K, w.N, cus)
            info = mnb.mnb_get_kernel_info(m, w.K, plan)
            gbs = res.bytes_per_call / (us * 1e-6) / 1e9
            e = {"m": m, "K": w.K, "N": w.N, "out_dtype": odt, "bytes_per_call": res.bytes_per_call,
                 "us_per_call": round(us, 3), "us_min": round(samples[0], 3), "us_max": round(samples[-1], 3),
                 "passes": passes, "calls_per_pass": n,
                 "GB/s": round(gbs, 1), "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4),
                 "rotated_copies": res.R, "plan": plan_fields(plan),
                 "vgprs": info["vgprs"], "wgs_per_cu": info["wgs_per_cu"],
                 "waves_per_cu": info["wgs_per_cu"] * plan.threads_per_wg // 64,
                 "lds_bytes": info["lds_bytes"]}
            if m > 1:
                flops = 2.0 * m * w.N * w.K
                e["fp32_valu_floor_us"] = round(flops / (PEAK_FP32_VALU_TFLOPS * 1e12) * 1e6, 3)
            att = attainable(res, stream, cus)
            e["attainable"] = att
            e["frac_of_attainable"] = round(gbs / att["gbs"], 4) if att else None
            prof = measured_profile(name, m, odt)
            if prof is not None:
                e["rocprof"] = {k: prof[k] for k in ("kernel_mean_us", "fetch_bytes", "write_bytes",
                                                     "fetch_over_alg", "alg_frac_of_8TBs",
                                                     "fetch_frac_of_8TBs")}
            else:
                e["rocprof"] = None
            out["%s:m%d:%s" % (name, m, odt)] = e
            log("[bench] %s m=%d %s: %.3f us/call (%.3f-%.3f), %.1f GB/s = %.1f%% of 8 TB/s, %s, %d VGPRs, "
                "%d waves/CU" % (name, m, odt, us, samples[0], samples[-1], gbs, 100 * gbs / PEAK_HBM_GBS,
                                 plan_fields(plan), info["vgprs"], e["waves_per_cu"]))
            del res
    return out


def staged_route(res, stream, L):
    """The staged route (fp16 GEMV into a staging buffer, then a separate
    fp16 -> bf16 cast launch) against the direct bf16 store, on the same
    rotated inputs; both must give the same bf16 bits."""
    import torch
    from block_wise_int4_matmulnbits_amd import workloads as W
    stage = torch.empty(res.out.shape, dtype=torch.float16, device="cuda")
    direct = torch.empty(res.out.shape, dtype=torch.bfloat16, device="cuda")
    staged = torch.empty_like(direct)
    raw_d = res.raw(stream.cuda_stream, direct, W.BF16)
    raw_s = res.raw(stream.cuda_stream, stage, W.F16)

    def go_direct(i):
        L.matmul_nbits(*raw_d[i % len(raw_d)])

    def go_staged(i):
        L.matmul_nbits(*raw_s[i % len(raw_s)])
        staged.copy_(stage)

    for i in range(50):
        go_direct(i)
        go_staged(i)
    n = 1000
    us_d = event_time_us(stream, go_direct, n)
    us_s = event_time_us(stream, go_staged, n)
    go_direct(0)
    go_staged(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(direct.view(torch.int16), staged.view(torch.int16)))
    log("[bench] staged route %.3f us/call (2 launches) vs direct %.3f us (1 launch); bits equal %s"
        % (us_s, us_d, same))
    return {"direct_us": round(us_d, 3), "staged_us": round(us_s, 3),
            "saving_us": round(us_s - us_d, 3), "launches_direct": 1, "launches_staged": 2,
            "staging_bytes": stage.numel() * 2, "bf16_bits_equal": same}


def decode_step(args, stream, L, layers=4):
    """One decode step of m=1 GEMVs: per layer q, k, v, o (4096 x 4096),
    gate_up (28672 x 4096) and down (4096 x 14336), distinct weights per
    layer, then the lm_head; eager launches against one captured HIP graph
    replayed on the same stream.  Outputs of the graph equal the eager ones."""
    import numpy as np
    import torch
    from block_wise_int4_matmulnbits_amd import workloads as W
    shapes = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
              ("gate_up", 4096, 28672), ("down", 14336, 4096)]
    dev = torch.device("cuda:0")
    base = {}
    for name, K, N in shapes + [("lm_head", 4096, 151936)]:
        if (K, N) not in base:
            d = W.generate(1, K, N, W.F16, True, 0.001, 0.01, 1.0, 50 + len(base))
            base[(K, N)] = (torch.from_numpy(d["B"]).to(dev),
                            torch.from_numpy(d["scales"].view(np.int16)).to(dev),
                            torch.from_numpy(d["zp"]).to(dev),
                            torch.from_numpy(np.ascontiguousarray(d["A"][:1]).view(np.int16)).to(dev))
    calls = []
    outs = []
    for layer in range(layers):
        for name, K, N in shapes:
            B, S, Z, A = base[(K, N)]
            if layer:
                B, S, Z = B.clone(), S.clone(), Z.clone()
            o = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
            calls.append((A, B, S, Z, o, K, N))
            outs.append(o)
    B, S, Z, A = base[(4096, 151936)]
    o = torch.empty((1, 151936), dtype=torch.bfloat16, device=dev)
    calls.append((A, B, S, Z, o, 4096, 151936))
    outs.append(o)
    nbytes = sum(W.Workload("x", 1, K, N, W.F16, (W.BF16,), True, 0, 0, 0, 0).bytes_per_call()
                 for (_, _, _, _, _, K, N) in calls)

    def launch_all(s):
        for (A, B, S, Z, o, K, N) in calls:
            st = L.matmul_nbits(A.data_ptr(), W.F16, 1, K, N, B.data_ptr(), S.data_ptr(),
                                Z.data_ptr(), 32, o.data_ptr(), W.BF16, s)
            assert st == 0, st

    for _ in range(10):
        launch_all(stream.cuda_stream)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o in outs:
        o.fill_(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch_all(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    same = True
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        same &= all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(eager, outs))
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
    n = 50
    us_eager = event_time_us(stream, lambda i: launch_all(stream.cuda_stream), n)
    us_graph = event_time_us(stream, lambda i: g.replay(), n)
    log("[bench] decode step (%d GEMVs, %.0f MB): eager %.1f us, graph %.1f us; graph == eager %s"
        % (len(calls), nbytes / 1e6, us_eager, us_graph, same))

    # Launch cost at the small end: a chain of 64 GEMVs of the 1024 x 1024
    # shape (cache-resident weights), eager against one replayed graph.
    d = W.generate(1, 1024, 1024, W.F16, False, 0.002, 0.02, 1.0, 70)
    sB = torch.from_numpy(d["B"]).to(dev)
    sS = torch.from_numpy(d["scales"].view(np.int16)).to(dev)
    sA = torch.from_numpy(np.ascontiguousarray(d["A"][:1]).view(np.int16)).to(dev)
    souts = [torch.empty((1, 1024), dtype=torch.float16, device=dev) for _ in range(64)]

    def chain(s):
        for o in souts:
            st = L.matmul_nbits(sA.data_ptr(), W.F16, 1, 1024, 1024, sB.data_ptr(), sS.data_ptr(),
                                None, 32, o.data_ptr(), W.F16, s)
            assert st == 0, st
    for _ in range(10):
        chain(stream.cuda_stream)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        chain(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    us_ce = event_time_us(stream, lambda i: chain(stream.cuda_stream), 20) / len(souts)
    us_cg = event_time_us(stream, lambda i: g2.replay(), 20) / len(souts)
    log("[bench] 64 small GEMVs (1024 x 1024): eager %.2f us each, graph %.2f us each" % (us_ce, us_cg))
    return {"gemvs": len(calls), "layers": layers, "bytes": nbytes,
            "eager_us": round(us_eager, 2), "graph_us": round(us_graph, 2),
            "graph_GB/s": round(nbytes / (us_graph * 1e-6) / 1e9, 1),
            "graph_outputs_equal_eager": bool(same),
            "small_chain": {"gemvs": len(souts), "K": 1024, "N": 1024,
                            "eager_us_per_gemv": round(us_ce, 3), "graph_us_per_gemv": round(us_cg, 3)}}


def offline_layout(args, stream, L, cus):
    """The second page's offline odd/even nibble interleave
    (MNB_LAYOUT_EVEN_ODD, converted once by mnb_repack_weights) against the
    natural layout, same plan otherwise, interleaved A/B on rotated copies.
    With the interleave the dequant yields (k, k+1) pairs and the
    activations skip their reorder."""
    import ctypes
    import torch
    import block_wise_int4_matmulnbits_amd as mnb
    from block_wise_int4_matmulnbits_amd import workloads as W
    out = {}
    for name, m in (("lm_head", 1), ("gate_up_bf16", 1), ("down_rows_bf16", 8)):
        w = W.WORKLOADS[name]
        res = Resident(w, m, W.BF16, args.rotate_mb)
        raw_n = res.raw(stream.cuda_stream)
        eo = [torch.empty_like(b) for (b, _, _) in res.copies]
        for (b, _, _), e in zip(res.copies, eo):
            mnb.mnb_repack_weights(b, mnb.MNB_LAYOUT_NATURAL, e, mnb.MNB_LAYOUT_EVEN_ODD, stream=stream)
        raw_e = [(r[0], r[1], r[2], r[3], r[4], e.data_ptr()) + tuple(r[6:]) for r, e in zip(raw_n, eo)]
        pn = mnb.plan_for_device(m, w.K, w.N, cus)
        pe = mnb.mnb_plan(**dict(pn.as_dict(), b_layout=mnb.MNB_LAYOUT_EVEN_ODD))
        assert mnb.mnb_plan_check(m, w.K, w.N, pe) == 0
        n = max(200, int(0.05 / (res.bytes_per_call / 5e12)))
        best = {"natural": 1e30, "even_odd": 1e30}
        for rep in range(3):
            for key, raw, plan in (("natural", raw_n, pn), ("even_odd", raw_e, pe)):
                pp = ctypes.byref(plan)

                def go(i, raw=raw, pp=pp):
                    L.matmul_nbits_planned(*raw[i % len(raw)], pp)
                for i in range(100):
                    go(i)
                best[key] = min(best[key], event_time_us(stream, go, n))
        b0 = res.copies[0][0]
        scratch = torch.empty_like(b0)

        def conv(i):
            mnb.mnb_repack_weights(b0, mnb.MNB_LAYOUT_NATURAL, scratch, mnb.MNB_LAYOUT_EVEN_ODD,
                                   stream=stream)
        conv(0)
        us_conv = event_time_us(stream, conv, 20)
        out["%s:m%d" % (name, m)] = {
            "natural_us": round(best["natural"], 3), "even_odd_us": round(best["even_odd"], 3),
            "gain_pct": round(100 * (best["natural"] - best["even_odd"]) / best["natural"], 2),
            "repack_us_once": round(us_conv, 2), "weight_bytes": b0.numel()}
        log("[bench] offline layout %s m=%d: natural %.3f us, even/odd %.3f us (repack once %.1f us)"
            % (name, m, best["natural"], best["even_odd"], us_conv))
        del res, eo, scratch
    return out


PREFILL_SHAPES = {"gate_up": (4096, 28672), "down": (14336, 4096)}


def prefill_only(args):
    """One prefill shape, default plan, bf16 in and out: --warmup untimed and
    --steps timed launches (for kernel traces and counter passes)."""
    import numpy as np
    import torch
    import block_wise_int4_matmulnbits_amd as mnb
    from block_wise_int4_matmulnbits_amd import workloads as W
    name, m = args.prefill_only.split(":")
    m = int(m)
    K, N = PREFILL_SHAPES[name]
    d = W.generate(1, K, N, W.BF16, True, 0.001, 0.01, 0.5, 90)
    dev = torch.device("cuda:0")
    B = torch.from_numpy(d["B"]).to(dev)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev)
    Z = torch.from_numpy(d["zp"]).to(dev)
    A = (torch.randn((m, K), device=dev) * 0.5).to(torch.bfloat16)
    o = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    L = mnb.lib()

    def go(i):
        st = L.matmul_nbits(A.data_ptr(), W.BF16, m, K, N, B.data_ptr(), S.data_ptr(), Z.data_ptr(),
                            32, o.data_ptr(), W.BF16, stream.cuda_stream)
        assert st == 0, st
    for i in range(args.warmup):
        go(i)
    us = event_time_us(stream, go, args.steps)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = mnb.plan_for_device(m, K, N, cus)
    print(json.dumps({"prefill": name, "m": m, "K": K, "N": N, "steps": args.steps,
                      "warmup": args.warmup, "us_per_call": round(us, 2),
                      "TFLOP/s": round(2.0 * m * N * K / (us * 1e-6) / 1e12, 1),
                      "plan": plan.as_dict()}), flush=True)


PREFILL_HEIGHTS = {"gate_up": (512, 2048), "down": (16, 64, 512, 2048)}


def prefill(stream, L, cus, rotate_mb):
    """Prefill heights (m > 8) on the gate_up and down-projection shapes:
    microseconds per call and TFLOP/s against the dense fp16 matrix-core
    peak.  The large heights reuse one weight copy (they are bound by the
    matrix core); the small ones, bound by the weight read, rotate over
    enough copies that none is still cached."""
    import numpy as np
    import torch
    import block_wise_int4_matmulnbits_amd as mnb
    from block_wise_int4_matmulnbits_amd import workloads as W
    out = {}
    dev = torch.device("cuda:0")
    for name, (K, N) in PREFILL_SHAPES.items():
        d = W.generate(1, K, N, W.BF16, True, 0.001, 0.01, 0.5, 90)
        B = torch.from_numpy(d["B"]).to(dev)
        S = torch.from_numpy(d["scales"].view(np.int16)).to(dev)
        Z = torch.from_numpy(d["zp"]).to(dev)
        wbytes = B.numel() + 2 * S.numel() + Z.numel()
        for m in PREFILL_HEIGHTS[name]:
            A = (torch.randn((m, K), device=dev) * 0.5).to(torch.bfloat16)
            o = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            copies = [(B, S, Z)]
            if m <= 64:
                copies += [(B.clone(), S.clone(), Z.clone()) for _ in range(math.ceil(rotate_mb * 1e6 / wbytes) - 1)]

            def go(i):
                b, sc, z = copies[i % len(copies)]
                st = L.matmul_nbits(A.data_ptr(), W.BF16, m, K, N, b.data_ptr(), sc.data_ptr(),
                                    z.data_ptr(), 32, o.data_ptr(), W.BF16, stream.cuda_stream)
                assert st == 0, st
            for i in range(5):
                go(i)
            us = event_time_us(stream, go, max(20, 2 * len(copies)))
            tflops = 2.0 * m * N * K / (us * 1e-6) / 1e12
            plan = mnb.plan_for_device(m, K, N, cus)
            out["%s:m%d" % (name, m)] = {
                "m": m, "K": K, "N": N, "us_per_call": round(us, 2), "TFLOP/s": round(tflops, 1),
                "pct_of_fp16_mfma_peak": round(100 * tflops / PEAK_FP16_MFMA_TFLOPS, 2),
                "weight_GB/s": round(wbytes / (us * 1e3), 1), "rotated_copies": len(copies),
                "plan": {k: v for k, v in plan.as_dict().items()
                         if k in ("engine", "row_tiles", "cols_per_tile", "waves_per_wg", "workgroups", "k_splits")}}
            log("[bench] prefill %s m=%d: %.1f us, %.1f TFLOP/s" % (name, m, us, tflops))
            del A, o, copies
    return out


def oracle_threads():
    """Host cores the oracle may use: the process's CPU affinity, capped by
    OMP_NUM_THREADS where the environment sets it (the GPU machine gives each
    GPU a 16-core share and sets it so)."""
    cores = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return (min(cores, int(cap)) if cap.isdigit() and int(cap) > 0 else cores), cores


def cpu_baseline(args, w, d, m, A, copy0, out_dtype, bytes_per_call):
    """The oracle, as it stands, timed on the host over whole calls of the
    same workload: on every usable core for about --cpu-seconds, and on one
    thread for three calls; the median call time of each.  Also checks
    copy 0 of the GPU output against it."""
    import numpy as np
    import torch

    import block_wise_int4_matmulnbits_amd as mnb
    import oracle
    from block_wise_int4_matmulnbits_amd import workloads as W

    threads, affinity = oracle_threads()

    def timed_calls(nthreads, seconds, min_calls):
        times, ref = [], None
        t_start = time.perf_counter()
        while len(times) < min_calls or time.perf_counter() - t_start < seconds:
            t0 = time.perf_counter()
            ref = oracle.matmul_nbits(d["A"][:m], w.a_dtype == W.BF16, d["B"], d["scales"],
                                      d["zp"], m, w.K, w.N, threads=nthreads)
            times.append(time.perf_counter() - t0)
        return sorted(times), ref

    t_all, ref = timed_calls(threads, args.cpu_seconds, 3)
    t_one, _ = timed_calls(1, 0.0, 3)
    med_all, med_one = t_all[len(t_all) // 2], t_one[len(t_one) // 2]
    gbs_all, gbs_one = bytes_per_call / med_all / 1e9, bytes_per_call / med_one / 1e9
    log("[bench] oracle: %d calls on %d threads, median %.1f ms = %.3f GB/s; 1 thread: median %.1f ms "
        "= %.4f GB/s (%d cores in the affinity mask)"
        % (len(t_all), threads, med_all * 1e3, gbs_all, med_one * 1e3, gbs_one, affinity))
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
    err = np.abs(g - o)
    ok1 = bool(np.all(err <= 1e-3 * ref["abs"] + ulp))
    ok2 = bool(np.array_equal(gbf, oracle.f16_to_bf16(g16.ravel()).reshape(g16.shape)))
    ulps = err / ulp
    worst = np.unravel_index(int(np.argmax(ulps)), ulps.shape)
    # Outputs off by more than one fp16 ulp are sums with heavy cancellation:
    # |y| is a small fraction of sum |a w|, so the fp32 accumulation error
    # (relative to sum |a w|) is many ulps of y, still far inside check 1.
    off = ulps > 1
    parity = {"check1": ok1, "check2_bf16_bit_exact": ok2,
              "max_err_fp16_ulp": float(ulps.max()),
              "bit_equal_frac": float(np.mean(g16 == ref["f16"])),
              "outputs_over_1_ulp": int(off.sum()),
              "worst": {"row": int(worst[0]), "col": int(worst[1]), "y": float(o[worst]),
                        "sum_abs_aw": float(ref["abs"][worst]),
                        "y_over_sum_abs": float(abs(o[worst]) / ref["abs"][worst]),
                        "err_over_check1_bound": float(err[worst] / (1e-3 * ref["abs"][worst] + ulp[worst]))},
              "median_y_over_sum_abs_where_over_1_ulp":
                  float(np.median(np.abs(o[off]) / ref["abs"][off])) if off.any() else None,
              "median_y_over_sum_abs_all": float(np.median(np.abs(o) / ref["abs"]))}
    log("[bench] parity vs oracle: %s" % parity)
    base = {"value": round(gbs_all, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "whole %s calls (m=%d, K=%d, N=%d), fp64 C oracle with OpenMP over columns: "
                      "%d calls on %d threads (median), and 3 calls on 1 thread; %d cores in the "
                      "affinity mask" % (w.name, m, w.K, w.N, len(t_all), threads, affinity),
            "ms_per_call": round(med_all * 1e3, 2),
            "ms_per_call_range": [round(t_all[0] * 1e3, 2), round(t_all[-1] * 1e3, 2)],
            "single_thread": {"value": round(gbs_one, 5), "unit": "GB/s", "cores": 1,
                              "ms_per_call": round(med_one * 1e3, 1),
                              "ms_per_call_range": [round(t_one[0] * 1e3, 1), round(t_one[-1] * 1e3, 1)]},
            "affinity_cores": affinity}
    return base, parity


if __name__ == "__main__":
    main()

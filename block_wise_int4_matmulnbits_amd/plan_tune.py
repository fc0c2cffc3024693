"""Tune the prefill planner's cost model (m > 8).

The planner (``mnb_plan_default`` in csrc/mnb_api.cpp) prices every prefill
tiling, and the 8-row decode plan run once per 8 rows, with a fitted cost
and takes the cheapest.  This script produces both halves of that:

  python -m block_wise_int4_matmulnbits_amd.plan_tune sweep OUT.json
      (GPU) times every tiling that mnb_plan_check accepts, each with one
      resident generation of workgroups, and the decode plan for m <= 16,
      on a fixed list of shapes (bf16 in and out, random weights).  One
      weight copy per shape: at the few-row heights it stays in the 256 MB
      last-level cache, so those times run below a call on cold weights;
      the model uses their ranking.
  python -m block_wise_int4_matmulnbits_amd.plan_tune fit IN.json
      (CPU) fits the cost of each tiling by non-negative least squares on
      relative error and prints the table the planner holds, and the
      regret of the fitted choice on every measured shape.
  python -m block_wise_int4_matmulnbits_amd.plan_tune sweep-grid OUT.json
      (GPU) times the 4x4x4 MFMA decode kernel (2 <= m <= 8) under its
      default lane split with whole workgroups per CU, from half a CU's
      worth to one resident generation (always timed), and the planner's
      own grid, on a list of decode shapes (bf16, weights rotated over
      enough copies that none stays in cache).

Cost of a tiling (µs), with R = ceil(tiles / CUs) rounds of tiles over the
compute units (a tiling that splits K over S workgroups has S times the
tiles), k the thousands of K per workgroup (K / S), W the weight bytes per
CU in MB (0.578 bytes per weight with the scales and zero points) and U the
MB per CU of fp32 partial sums a split writes (S * m * N * 4 / CUs):
    t0 + a*k*(R-1) + g*(R-1) + d*k + h*W + u*U
Cost of the decode plan: per launch of r rows, a part that grows with K (the
activation staging and the per-wave work of each workgroup) and a part
linear in the weight MB with a rate per row,
    max(exp(c0) * (K/4096)^c1 + MB * (c2 + c3 * r/8), 3 us),
summed over the ceil(m/8) launches.  (A power law in N, as first fitted,
ran 15-20% below the launches on 151936 columns, where the time is linear
in the weights.)
"""
from __future__ import annotations

import json
import math
import os
import sys

# (row tiles, columns, waves, K splits over workgroups)
TILINGS = ([(1, 16, 4, 1), (1, 16, 8, 1), (1, 32, 4, 1), (1, 64, 2, 1), (1, 128, 4, 1), (2, 128, 4, 1),
            (4, 128, 4, 1), (1, 256, 8, 1), (2, 256, 8, 1), (4, 256, 8, 1), (8, 256, 8, 1)] +
           [(rt, cols, waves, s) for rt, cols, waves in ((1, 128, 4), (2, 128, 4), (4, 128, 4), (1, 256, 8), (2, 256, 8))
            for s in (2, 4, 8, 16)])
MAX_SPLIT_WORKSPACE = 32 << 20   # bytes of partial sums a default plan may take (MNB_MAX_SPLIT_WORKSPACE)
BYTES_PER_WEIGHT = 0.578   # 4 bits + a 2-byte scale and a 4-bit zero point per 32

SHAPES = [(64, 4096, 28672), (128, 4096, 28672), (256, 4096, 28672), (16, 4096, 28672), (64, 14336, 4096),
          (128, 14336, 4096), (24, 14336, 4096), (32, 4096, 6144), (128, 4096, 6144), (192, 14336, 4096),
          (24, 4096, 151936), (64, 4096, 151936), (12, 4096, 6144), (9, 2048, 8192), (16, 14336, 8192),
          (32, 4096, 65536), (384, 14336, 4096), (192, 4096, 6144), (256, 4096, 6144), (1152, 4096, 4096),
          (768, 4096, 6144), (320, 14336, 14336), (384, 4096, 6144), (2176, 14336, 4096), (2048, 14336, 4096),
          (1536, 4096, 6144), (640, 4096, 14336), (384, 4096, 151936), (640, 4096, 151936), (1152, 4096, 14336),
          (1024, 4096, 28672), (128, 4096, 151936), (256, 14336, 4096), (1024, 14336, 4096),
          (16, 14336, 4096), (9, 4096, 151936), (16, 4096, 151936), (12, 4096, 4096), (9, 8192, 2048),
          (16, 14336, 2048), (12, 8192, 28672), (512, 4096, 28672), (2048, 4096, 28672), (512, 14336, 4096),
          (48, 14336, 4096), (96, 14336, 4096), (32, 14336, 4096), (4096, 4096, 28672), (16, 4096, 4096),
          (64, 4096, 4096), (32, 8192, 8192), (512, 4096, 4096), (96, 4096, 151936), (160, 14336, 4096),
          (9, 14336, 4096), (12, 14336, 4096), (24, 4096, 4096), (48, 4096, 4096), (96, 4096, 6144),
          (64, 8192, 2048), (32, 14336, 2048), (256, 4096, 4096), (48, 4096, 28672), (80, 14336, 4096)]


def key_of(t):
    """"rt,cols,waves" for a tiling without a K split, "rt,cols,waves,sS" with one
    (and "m,K,N" for a shape)."""
    if len(t) == 4:
        return "%d,%d,%d" % t[:3] if t[3] == 1 else "%d,%d,%d,s%d" % t
    return "%d,%d,%d" % t


def tiles_of(t, m, N):
    rt, cols, _, splits = t
    rows = 256 if rt == 8 else 32 * rt
    return -(-m // rows) * -(-N // cols) * splits


def workspace_bytes(t, m, N):
    return t[3] * m * N * 4 if t[3] > 1 else 0


def admitted(t, m, N, cus):
    """A tiling the planner considers: one that splits K over workgroups only
    while its tiles fit in less than four rounds over the compute units (the
    split is there to fill the device, not to add rounds)."""
    return t[3] == 1 or tiles_of(t, m, N) < 4 * cus


def tiling_features(t, m, K, N, cus):
    R = -(-tiles_of(t, m, N) // cus)
    k = K / t[3] / 1e3
    return [1.0, k * (R - 1), float(R - 1), k, N * K * BYTES_PER_WEIGHT / cus / 1e6,
            workspace_bytes(t, m, N) / cus / 1e6]


DECODE_LAUNCH_US = 3.0        # the time one decode launch takes however small


def decode_cost(p, m, K, N):
    mb = N * K * BYTES_PER_WEIGHT / 1e6

    def one(r):
        return max(math.exp(p[0]) * (K / 4096) ** p[1] + mb * (p[2] + p[3] * r / 8), DECODE_LAUNCH_US)
    full, rem = divmod(m, 8)
    return full * one(8) + (one(rem) if rem else 0.0)


def sweep(out_path):
    import ctypes
    import torch
    import block_wise_int4_matmulnbits_amd as mnb
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    L = mnb.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    props = torch.cuda.get_device_properties(0)
    res = {"cus": cus, "device": props.name, "arch": getattr(props, "gcnArchName", ""), "shapes": {}}

    def timed(raw, plan):
        pp = ctypes.byref(plan)

        def go():
            st = L.matmul_nbits_planned(*raw, pp)
            assert st == 0, mnb.mnb_status_string(st)
        go()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        go()
        e1.record(stream)
        torch.cuda.synchronize()
        n = int(min(200, max(3, 20000 / max(e0.elapsed_time(e1) * 1e3, 1.0))))
        best = float("inf")
        for _ in range(3):
            e0.record(stream)
            for _ in range(n):
                go()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / n)
        return best

    for m, K, N in SHAPES:
        A = (torch.randn(m, K, device=dev) * 0.5).to(torch.bfloat16)
        B = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev)
        S = (torch.rand(N, K // 32, device=dev) * 0.01 + 0.001).to(torch.float16)
        Z = torch.randint(0, 256, (N, (K // 32 + 1) // 2), dtype=torch.uint8, device=dev)
        O = torch.empty(m, N, dtype=torch.bfloat16, device=dev)
        raw = (A.data_ptr(), mnb.MNB_BF16, m, K, N, B.data_ptr(), S.data_ptr(), Z.data_ptr(), 32,
               O.data_ptr(), mnb.MNB_BF16, stream.cuda_stream)
        row = {}
        for t in TILINGS:
            rt, cols, waves, splits = t
            p = mnb.mnb_plan(engine=2, row_tiles=rt, cols_per_tile=cols, waves_per_wg=waves, workgroups=1,
                             k_splits=splits)
            if mnb.mnb_plan_check(m, K, N, p) != 0 or workspace_bytes(t, m, N) > MAX_SPLIT_WORKSPACE:
                continue
            occ = mnb.mnb_get_kernel_info(m, K, p)["wgs_per_cu"]
            tiles = tiles_of(t, m, N)
            p = mnb.mnb_plan(engine=2, row_tiles=rt, cols_per_tile=cols, waves_per_wg=waves,
                             workgroups=max(1, min(tiles, occ * cus)), k_splits=splits)
            row[key_of(t)] = {"us": round(timed(raw, p), 3), "occ": occ, "tiles": tiles}
        if m <= 16:
            row["decode"] = {"us": round(timed(raw, mnb.plan_for_device(8, K, N, cus)), 3)}
        res["shapes"][key_of((m, K, N))] = row
        print(key_of((m, K, N)), " ".join("%s=%.1f" % (k, v["us"]) for k, v in row.items()), flush=True)
        del A, B, S, Z, O
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)


GRID_SHAPES = [(4096, 28672), (4096, 151936), (4096, 6144), (4096, 4096), (14336, 4096), (4096, 14336),
               (8192, 8192), (2048, 8192), (2048, 28672), (2048, 151936), (5120, 14336), (6144, 14336)]


def sweep_grid(out_path):
    import ctypes
    import torch
    import block_wise_int4_matmulnbits_amd as mnb
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    L = mnb.lib()
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    res = {"cus": cus, "device": props.name, "arch": getattr(props, "gcnArchName", ""), "shapes": {}}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for K, N in GRID_SHAPES:
        for m in (2, 3, 4, 6, 8):
            base = mnb.plan_for_device(m, K, N, cus)
            if base.engine != 3:
                continue
            A = (torch.randn(m, K, device=dev) * 0.5).to(torch.bfloat16)
            wbytes = N * K // 2 + N * K // 16 + N * K // 64
            ncopy = max(1, min(8, int(512e6 // wbytes)))
            copies = [(torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev),
                       (torch.rand(N, K // 32, device=dev) * 0.01 + 0.001).to(torch.float16),
                       torch.randint(0, 256, (N, (K // 32 + 1) // 2), dtype=torch.uint8, device=dev))
                      for _ in range(ncopy)]
            O = torch.empty(m, N, dtype=torch.bfloat16, device=dev)
            occ = mnb.mnb_get_kernel_info(m, K, base)["wgs_per_cu"]
            tiles = -(-N // base.cols_per_tile)
            row = {}
            grids = {max(1, min(-(-tiles // 2), int(f * cus))) for f in (0.5, 1, 1.5, 2, 3, 4, 5, 6, 8) if f <= occ}
            grids.add(base.workgroups)   # the planner's own pick is always timed,
            grids.add(max(1, min(-(-tiles // 2), occ * cus)))   # and one resident generation
            for wg in sorted(grids):
                p = mnb.mnb_plan(**dict(base.as_dict(), workgroups=wg))
                assert mnb.mnb_plan_check(m, K, N, p) == 0

                def go(i):
                    B, S, Z = copies[i % ncopy]
                    st = L.matmul_nbits_planned(A.data_ptr(), mnb.MNB_BF16, m, K, N, B.data_ptr(), S.data_ptr(),
                                                Z.data_ptr(), 32, O.data_ptr(), mnb.MNB_BF16, stream.cuda_stream,
                                                ctypes.byref(p))
                    assert st == 0, mnb.mnb_status_string(st)
                for i in range(30):
                    go(i)
                n = max(100, min(2000, int(0.05 / (wbytes / 5e12))))
                best = float("inf")
                for _ in range(3):
                    e0.record(stream)
                    for i in range(n):
                        go(i)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    best = min(best, e0.elapsed_time(e1) * 1e3 / n)
                row[str(wg)] = round(best, 3)
            res["shapes"][key_of((m, K, N))] = {"occ": occ, "tiles": tiles, "us": row}
            print(key_of((m, K, N)), "occ", occ, " ".join("%s:%.2f" % kv for kv in row.items()), flush=True)
            del A, copies, O
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)


def fit_model(data):
    """(table, decode): the cost coefficients of every tiling, fitted by
    non-negative least squares on relative error, and the decode plan's."""
    import numpy as np
    from scipy.optimize import least_squares, nnls
    cus = data["cus"]
    shapes = [(tuple(map(int, k.split(","))), row) for k, row in data["shapes"].items()]
    table = {}
    for t in TILINGS:
        X, y = [], []
        for (m, K, N), row in shapes:
            if key_of(t) in row and admitted(t, m, N, cus):
                X.append(tiling_features(t, m, K, N, cus))
                y.append(row[key_of(t)]["us"])
        X, y = np.array(X), np.array(y)
        table[t], _ = nnls(X / y[:, None], np.ones_like(y))
    pts = [((m, K, N), row["decode"]["us"]) for (m, K, N), row in shapes if "decode" in row]
    dec = least_squares(lambda p: [decode_cost(p, *s) / us - 1 for s, us in pts], [1.5, 0.5, 0.1, 0.1]).x
    return table, dec


def model_pick(table, dec, m, K, N, cus, candidates):
    """The cheapest of `candidates` (tiling keys and "decode") by the model."""
    cost = {}
    for t in TILINGS:
        if key_of(t) in candidates and admitted(t, m, N, cus):
            cost[key_of(t)] = sum(f * c for f, c in zip(tiling_features(t, m, K, N, cus), table[t]))
    if "decode" in candidates:
        cost["decode"] = decode_cost(dec, m, K, N)
    return min(cost, key=cost.get)


def fit(path):
    data = json.load(open(path))
    table, dec = fit_model(data)
    print("// rt, cols, waves, splits, t0, a, g, d, h, u")
    for t in TILINGS:
        print("    {%d, %d, %d, %d, %s}," % (*t, ", ".join("%.4f" % v for v in table[t])))
    print("// decode: %s" % ", ".join("%.4f" % v for v in dec))
    regrets, vs_unsplit = [], []
    for key, row in sorted(data["shapes"].items()):
        m, K, N = map(int, key.split(","))
        pick = model_pick(table, dec, m, K, N, data["cus"], row)
        best = min(v["us"] for v in row.values())
        unsplit = min(v["us"] for k, v in row.items() if ",s" not in k)
        regrets.append(row[pick]["us"] / best - 1)
        vs_unsplit.append(row[pick]["us"] / unsplit - 1)
        print("%-18s pick %-12s %8.2f us  best %8.2f  regret %4.1f%%  vs best unsplit %+5.1f%%" % (
            key, pick, row[pick]["us"], best, 100 * regrets[-1], 100 * vs_unsplit[-1]))
    print("mean regret %.2f%%, max %.1f%%; against the best plan without a K split: mean %+.2f%%, worst %+.1f%%" % (
        100 * sum(regrets) / len(regrets), 100 * max(regrets), 100 * sum(vs_unsplit) / len(vs_unsplit),
        100 * max(vs_unsplit)))


if __name__ == "__main__":
    cmds = {"sweep": sweep, "fit": fit, "sweep-grid": sweep_grid}
    if len(sys.argv) != 3 or sys.argv[1] not in cmds:
        sys.exit("usage: python -m block_wise_int4_matmulnbits_amd.plan_tune sweep|fit|sweep-grid FILE.json")
    cmds[sys.argv[1]](os.path.abspath(sys.argv[2]))

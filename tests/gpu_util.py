"""Helpers shared by the GPU tests: upload seeded inputs, run the C ABI,
download bits, and the two acceptance checks.

Check 1: |y_gpu - y_oracle| <= 1e-3 * sum_k |a_k w_k| + 1 fp16 ulp of y
(compared as numbers; equal infinities pass).
Check 2: the bf16 output is bit-identical to the oracle's fp16 -> bf16
narrowing of the GPU's own fp16 output.
"""
import sys

import numpy as np
import torch


def require_gpu():
    """GPU tests fail (never skip) without a gfx950 device, so that a run on
    the wrong machine cannot pass vacuously."""
    assert torch.cuda.is_available(), "no GPU visible: GPU tests must run on MI355X"
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), "expected gfx950, found %s" % arch


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(d, m=None):
    m = d["m"] if m is None else m
    dev = "cuda"
    adt = torch.bfloat16 if d.get("a_is_bf16", d.get("a_dtype") == 1) else torch.float16
    A = torch.from_numpy(np.ascontiguousarray(d["A"][:m]).view(np.int16)).to(dev).view(adt)
    B = torch.from_numpy(np.ascontiguousarray(d["B"])).to(dev)
    S = torch.from_numpy(np.ascontiguousarray(d["scales"]).view(np.int16)).to(dev).view(torch.float16)
    Z = None if d["zp"] is None else torch.from_numpy(np.ascontiguousarray(d["zp"])).to(dev)
    return A, B, S, Z


def new_out(m, N, out_dtype, sentinel=True):
    dt = torch.bfloat16 if out_dtype == 1 else torch.float16
    if sentinel:   # 0xFFFF: a NaN no finite input can produce
        return torch.full((m, N), -1, dtype=torch.int16, device="cuda").view(dt)
    return torch.empty((m, N), dtype=dt, device="cuda")


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f16_values(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def check1(y_gpu_f16, ref, oracle_mod):
    """Returns (ok_mask, max_err_in_ulps)."""
    g = f16_values(y_gpu_f16)
    o = f16_values(ref["f16"])
    ulp = oracle_mod.f16_ulp(ref["f16"])
    same_inf = np.isinf(g) & np.isinf(o) & (np.sign(g) == np.sign(o))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(g - o))
    tol = 1e-3 * ref["abs"] + ulp
    ok = err <= tol
    ok &= ~np.isnan(g)
    finite = np.isfinite(ulp) & np.isfinite(err)
    max_ulps = float(np.max(err[finite] / ulp[finite])) if finite.any() else 0.0
    return ok, max_ulps


def check2(y_gpu_bf16, y_gpu_f16, oracle_mod):
    want = oracle_mod.f16_to_bf16(np.asarray(y_gpu_f16).ravel()).reshape(y_gpu_f16.shape)
    return np.asarray(y_gpu_bf16) == want

"""Loader for tests/golden/hand_cases.json: turns each case's compact
description into packed arrays (no arithmetic of the method here: only
placing given nibbles and bytes into the stored layout)."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_cases.json")


def _int(v):
    return int(v, 16) if isinstance(v, str) else int(v)


def _fill_set(spec, length, conv):
    arr = [conv(spec["fill"])] * length
    for k, v in spec.get("set", {}).items():
        arr[int(k)] = conv(v)
    return arr


def load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def build_case(c):
    m, K, N = c["m"], c["K"], c["N"]
    nb = K // 32
    a_is_bf16 = c["a_dtype"] == "bf16"
    if "a_bits" in c:
        A = np.array([_fill_set(r, K, _int) for r in c["a_bits"]], np.uint16)
    else:
        vals = np.array([_fill_set(r, K, float) for r in c["a"]], np.float64)
        assert not a_is_bf16
        h = vals.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), vals), "a not exact in fp16"
        A = h.view(np.uint16)
    if "bytes" in c:
        B = np.array([[_int(col["fill"])] * (K // 2) for col in c["bytes"]],
                     np.uint8)
    else:
        q = np.array([_fill_set(col, K, int) for col in c["q"]], np.uint8)
        assert q.max() <= 15
        B = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    zb = (nb + 1) // 2
    if "zp_bytes" in c:
        zp = np.array([[_int(v) for v in col] for col in c["zp_bytes"]], np.uint8)
        assert zp.shape == (N, zb)
    elif c.get("zp") is not None:
        z = np.array(c["zp"], np.uint8)
        zp = np.zeros((N, zb), np.uint8)
        for b in range(nb):
            zp[:, b // 2] |= (z[:, b] << (4 * (b % 2))).astype(np.uint8)
    else:
        zp = None
    s = np.array(c["scales"], np.float64)
    sh = s.astype(np.float16)
    assert np.array_equal(sh.astype(np.float64), s), "scale not exact in fp16"
    scales = sh.view(np.uint16).reshape(N, nb)
    exp16 = np.array([[_int(v) for v in row] for row in c["expected_f16"]], np.uint16)
    expbf = np.array([[_int(v) for v in row] for row in c["expected_bf16"]], np.uint16)
    absum = np.array(c["abs"], np.float64) if "abs" in c else None
    return dict(m=m, K=K, N=N, A=A, a_is_bf16=a_is_bf16, B=B, scales=scales,
                zp=zp, value=np.array(c["value"], np.float64), f16=exp16,
                bf16=expbf, abs=absum)

"""fp64 CPU oracle for the block-wise INT4 MatMulNBits decode GEMV.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never imports, links or calls
it, and this package never imports the product.

The arithmetic lives in ``mnb_oracle.c`` (plain C, fp64, one loop nest that
follows the definition on the onnx-genai pages "perf(cuda): let the split-K
decode GEMV store bf16 directly" and "PORT-1 (offline bias+interleave)").
This module only builds that file with gcc and marshals numpy arrays.

Every output is pinned by ``tests/test_oracle_pins.py`` against something
other than the oracle itself:
  * ``f16``/``bf16``/``f64``: hand-derived closed forms
    (``tests/golden/hand_cases.json``), exhaustive checks of the rounding
    routines against numpy/torch, an exact-integer recomputation of the sums,
    brute force with a closed form, and invariants;
  * ``abs`` (the sum of |a*w|, which scales the first acceptance check):
    hand-derived values, the exact-integer sum of |a|*|q-z|*|s|, and the
    brute-force closed form;
  * ``f16_ulp`` (the other term of that check): every one of the 65,536 fp16
    patterns against the gap to the next pattern of larger magnitude and
    against numpy's spacing, plus a hand table.
``tests/test_oracle_mutations.py`` plants 21 plausible mistakes in a copy of
this package, one at a time, and checks that each fails a pin.  No function
is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mnb_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmnb_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP). Returns the library path."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.mnb_oracle_matmul_nbits.restype = ctypes.c_int
        lib.mnb_oracle_matmul_nbits.argtypes = [
            u16p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            u8p, u16p, u8p, i64p, ctypes.c_int64, u16p, u16p, f64p, f64p,
            ctypes.c_int, ctypes.c_int]
        lib.mnb_oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.mnb_oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.mnb_oracle_f16_to_f64.restype = ctypes.c_double
        lib.mnb_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.mnb_oracle_bf16_to_f64.restype = ctypes.c_double
        lib.mnb_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.mnb_oracle_f16_to_bf16.restype = ctypes.c_uint16
        lib.mnb_oracle_f16_to_bf16.argtypes = [ctypes.c_uint16]
        lib.mnb_oracle_bf16_to_f16.restype = ctypes.c_uint16
        lib.mnb_oracle_bf16_to_f16.argtypes = [ctypes.c_uint16]
        lib.mnb_oracle_f64_to_f16_array.argtypes = [f64p, u16p, ctypes.c_int64]
        lib.mnb_oracle_f16_to_bf16_array.argtypes = [u16p, u16p, ctypes.c_int64]
        lib.mnb_oracle_bf16_to_f16_array.argtypes = [u16p, u16p, ctypes.c_int64]
        lib.mnb_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return int(_load().mnb_oracle_max_threads())


def matmul_nbits(A_bits, a_is_bf16, B, scales, zero_points, m, K, N,
                 cols=None, threads=0, weights_f16=False):
    """Run the oracle.

    A_bits: uint16 [m, K] (fp16 or bf16 bit patterns, per ``a_is_bf16``)
    B: uint8 [N, K/2]; scales: uint16 [N, K/32] fp16 bits;
    zero_points: uint8 [N, ceil(K/64)] or None (every zero point 8).
    cols: optional int64 column indices (a sample of the N columns).
    weights_f16: round every dequantised weight (q - z) * s to fp16 (RNE)
    before the dot product -- the packed-half dequant of the second page's
    GEMV ("Why the premise fails here", item 3), which the prefill kernel
    follows.  ``abs`` is then the sum of |a * w| over the rounded weights.
    Returns dict with ``f16`` and ``bf16`` (uint16 [m, ncols]), ``f64`` and
    ``abs`` (float64 [m, ncols]).
    """
    lib = _load()
    A_bits = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if zero_points is not None:
        zero_points = np.ascontiguousarray(zero_points, dtype=np.uint8)
    assert A_bits.size == m * K and B.size == N * (K // 2)
    assert scales.size == N * (K // 32)
    if zero_points is not None:
        assert zero_points.size == N * ((K // 32 + 1) // 2)
    if cols is not None:
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        assert cols.size == 0 or (cols.min() >= 0 and cols.max() < N)
        ncols = cols.size
    else:
        ncols = N
    y16 = np.zeros((m, ncols), np.uint16)
    ybf = np.zeros((m, ncols), np.uint16)
    y64 = np.zeros((m, ncols), np.float64)
    ab = np.zeros((m, ncols), np.float64)
    rc = lib.mnb_oracle_matmul_nbits(
        _ptr(A_bits, ctypes.c_uint16), int(bool(a_is_bf16)), m, K, N,
        _ptr(B, ctypes.c_uint8), _ptr(scales, ctypes.c_uint16),
        _ptr(zero_points, ctypes.c_uint8), _ptr(cols, ctypes.c_int64), ncols,
        _ptr(y16, ctypes.c_uint16), _ptr(ybf, ctypes.c_uint16),
        _ptr(y64, ctypes.c_double), _ptr(ab, ctypes.c_double), int(threads),
        int(bool(weights_f16)))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"f16": y16, "bf16": ybf, "f64": y64, "abs": ab}


def f64_to_f16(x):
    """fp64 -> fp16 bits, round to nearest even (array or scalar)."""
    lib = _load()
    x = np.ascontiguousarray(np.atleast_1d(x), dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib.mnb_oracle_f64_to_f16_array(_ptr(x, ctypes.c_double),
                                    _ptr(out, ctypes.c_uint16), x.size)
    return out


def f16_to_bf16(h):
    """Narrow fp16 bit patterns to bf16 bit patterns (exact widen, then RNE)."""
    lib = _load()
    h = np.ascontiguousarray(np.atleast_1d(h), dtype=np.uint16)
    out = np.empty(h.shape, np.uint16)
    lib.mnb_oracle_f16_to_bf16_array(_ptr(h, ctypes.c_uint16),
                                     _ptr(out, ctypes.c_uint16), h.size)
    return out


def bf16_to_f16(b):
    """Convert bf16 bit patterns to fp16 bit patterns (RNE)."""
    lib = _load()
    b = np.ascontiguousarray(np.atleast_1d(b), dtype=np.uint16)
    out = np.empty(b.shape, np.uint16)
    lib.mnb_oracle_bf16_to_f16_array(_ptr(b, ctypes.c_uint16),
                                     _ptr(out, ctypes.c_uint16), b.size)
    return out


def f16_value(h) -> float:
    return float(_load().mnb_oracle_f16_to_f64(int(h)))


def bf16_value(b) -> float:
    return float(_load().mnb_oracle_bf16_to_f64(int(b)))


def f16_ulp(h_bits):
    """One fp16 ulp at each fp16 value: 2^(max(floor(log2|y|), -14) - 10).

    For y = 0 (and subnormals) this is 2^-24; infinities give inf."""
    h = np.asarray(h_bits, dtype=np.uint16)
    expo = ((h >> 10) & 0x1F).astype(np.int32)
    e = np.maximum(expo - 15, -14)
    ulp = np.ldexp(1.0, e - 10)
    return np.where(expo == 31, np.inf, ulp)

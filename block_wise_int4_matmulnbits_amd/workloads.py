"""Seeded synthetic inputs for the INT4 MatMulNBits decode GEMV.

This module only draws random bytes and values; it holds none of the
method's arithmetic (no dequantisation, no dot product, no output
rounding).  The same arrays feed the HIP path and the CPU oracle.

The named workloads mirror the shapes the onnx-genai pages talk about (a
fused gate_up projection, a down projection run as a small-batch row loop,
an lm_head-sized GEMV; "PORT-1 (offline bias+interleave)", Result table,
and "perf(cuda): let the split-K decode GEMV store bf16 directly", the
small-batch row-loop paragraph).  The models behind those pages are not
available, so seeded random data of the same shape and value ranges stands
in for them.

Recipe (numpy ``Generator(PCG64(seed))``, drawn in this order):
  1. A: ``normal(0, sigma, (m_max, K))`` in float64, rounded to fp16 (numpy,
     RNE) or to bf16 (torch float32 -> bfloat16, RNE);
  2. B: ``integers(0, 256, (N, K/2), uint8)`` -- two independent uniform
     nibbles per byte;
  3. scales: ``uniform(lo, hi, (N, K/32))`` rounded to fp16;
  4. zero points: ``integers(0, 256, (N, ceil(K/64)), uint8)`` (two uniform
     4-bit zero points per byte), or None for the symmetric case.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F16 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    m: int
    K: int
    N: int
    a_dtype: int            # F16 or BF16
    out_dtypes: tuple       # output dtypes the workload runs
    asym: bool              # zero points present
    scale_lo: float
    scale_hi: float
    sigma: float
    seed: int
    m_max: int = 0          # rows drawn (>= m); rows are shared across m

    @property
    def nblocks(self) -> int:
        return self.K // 32

    def bytes_per_call(self, m=None) -> int:
        """Algorithmic HBM bytes of one call: packed weights, scales, zero
        points, activations once and output once."""
        m = self.m if m is None else m
        nb = self.K // 32
        b = self.N * self.K // 2 + self.N * nb * 2
        if self.asym:
            b += self.N * ((nb + 1) // 2)
        return b + m * self.K * 2 + m * self.N * 2


WORKLOADS = {
    "tiny_1k": Workload("tiny_1k", 1, 1024, 1024, F16, (F16,), False,
                        0.002, 0.02, 1.0, 0),
    "asym_4k": Workload("asym_4k", 1, 4096, 4096, F16, (F16,), True,
                        0.002, 0.02, 1.0, 1),
    "gate_up_bf16": Workload("gate_up_bf16", 1, 4096, 28672, BF16, (BF16,),
                             True, 0.001, 0.01, 1.0, 2),
    "down_rows_bf16": Workload("down_rows_bf16", 8, 14336, 4096, BF16,
                               (BF16,), True, 0.001, 0.01, 0.5, 3, m_max=8),
    "lm_head": Workload("lm_head", 1, 4096, 151936, F16, (F16, BF16), True,
                        0.001, 0.01, 1.0, 4),
}


def _round_activations(x64: np.ndarray, a_dtype: int) -> np.ndarray:
    if a_dtype == F16:
        return x64.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def generate(m, K, N, a_dtype=F16, asym=True, scale_lo=0.002, scale_hi=0.02,
             sigma=1.0, seed=0, m_max=None):
    """Draw one input set.  Returns a dict of numpy arrays:

    ``A`` uint16 [m_max, K] (bit patterns of ``a_dtype``), ``B`` uint8
    [N, K/2], ``scales`` uint16 [N, K/32] (fp16 bits), ``zp`` uint8
    [N, ceil(K/64)] or None.
    """
    assert K % 32 == 0
    m_max = max(m, m_max or 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = K // 32
    a64 = rng.normal(0.0, sigma, (m_max, K))
    A = _round_activations(a64, a_dtype)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.uniform(scale_lo, scale_hi, (N, nb)).astype(np.float16)
    scales = scales.view(np.uint16)
    zp = rng.integers(0, 256, (N, (nb + 1) // 2), dtype=np.uint8) if asym else None
    return {"A": A, "B": B, "scales": scales, "zp": zp, "a_dtype": a_dtype,
            "m": m, "K": K, "N": N}


def generate_workload(w: Workload, m=None):
    m = w.m if m is None else m
    return generate(m, w.K, w.N, w.a_dtype, w.asym, w.scale_lo, w.scale_hi,
                    w.sigma, w.seed, m_max=max(w.m_max, m))

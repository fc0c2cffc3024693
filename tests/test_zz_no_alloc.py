"""matmul_nbits_noalloc against matmul_nbits, through the C ABI.

The no-allocation entry point runs the default plan with the library's fixed
per-device workspace instead of the per-stream one, so its output must be
bit-identical to matmul_nbits on the same inputs: here on two calls in a row
whose plans split K over workgroups, the second smaller than the first (its
partial sums reuse the start of the buffer the first call filled), then a
decode call that needs no workspace.  Both output types.
"""
import numpy as np
import pytest
import torch

import block_wise_int4_matmulnbits_amd as mnb
from block_wise_int4_matmulnbits_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _call(fn, d, m, out_dtype):
    A, B, S, Z = G.to_dev(d, m)
    out = G.new_out(m, d["N"], out_dtype)
    c0 = mnb.mnb_counters_get()
    fn(A, B, S, Z, out)
    torch.cuda.synchronize()
    c1 = mnb.mnb_counters_get()
    return G.bits(out), c1["launches"] - c0["launches"]


def test_noalloc_matches_matmul_nbits():
    G.require_gpu()
    mnb.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # The down projection at 64 rows (8 slices of 64 x 128 tiles at 256 CUs:
    # 8 MB of partial sums), then 16 rows over 2048 columns (2 MB), then one
    # row of the gate_up shape (a decode plan).
    for m, K, N, seed in ((64, 14336, 4096, 1201), (16, 14336, 2048, 1202), (1, 4096, 28672, 1203)):
        d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, seed)
        plan = mnb.plan_for_device(m, K, N, cus)
        split = plan.engine == 2 and plan.k_splits > 1
        if cus == 256 and m > 1:
            assert split, plan.as_dict()
        G.log("[noalloc] m=%d K=%d N=%d plan %s" % (m, K, N, plan.as_dict()))
        for out_dtype in (W.F16, W.BF16):
            ref, n_ref = _call(mnb.matmul_nbits, d, m, out_dtype)
            got, n_got = _call(mnb.matmul_nbits_noalloc, d, m, out_dtype)
            assert not np.any(got == 0xFFFF)
            assert np.array_equal(got, ref), "m=%d: %d outputs differ" % (m, int(np.sum(got != ref)))
            assert n_got == n_ref == (2 if split else 1)

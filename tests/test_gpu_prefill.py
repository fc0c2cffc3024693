"""GPU parity of the prefill path (m > 8 rows, the matrix-core tile kernel)
against the fp64 oracle, through the C ABI.

Same acceptance as the decode path: check 1 on the fp16 output, check 2
(bf16 output bit-identical to the narrowing of the fp16 output), counters,
no stale element.  The summation order of an output depends only on K, so
rows computed in launches of different heights are bit-identical.
"""
import numpy as np
import pytest
import torch

import block_wise_int4_matmulnbits_amd as mnb
from block_wise_int4_matmulnbits_amd import workloads as W
from tests import gpu_util as G
from tests.test_gpu_parity import assert_parity, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    mnb.lib()


@pytest.mark.parametrize("m,K,N,a_dtype,asym", [
    (9, 4096, 1000, W.F16, True),       # smallest prefill height, one 16-row tile
    (16, 4096, 64, W.BF16, True),       # exactly one tile
    (17, 1024, 130, W.F16, False),      # ragged rows and columns, zero point 8
    (100, 32 * 37, 77, W.BF16, True),   # K not a whole number of 128-wide steps
    (130, 14336, 300, W.BF16, True),    # down-projection K, row tail of 2
    (256, 4096, 1024, W.F16, True),     # several row and column blocks
])
def test_prefill_default_plan(oracle_mod, m, K, N, a_dtype, asym):
    d = W.generate(m, K, N, a_dtype, asym, 0.001, 0.01, 0.5, 700 + m)
    plan = mnb.plan_for_device(m, K, N, torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan.engine == 2
    assert_parity(oracle_mod, d, m, "prefill", None)


@pytest.mark.parametrize("rt", [1, 2, 4, 8])
def test_prefill_every_row_tiling_and_small_grids(oracle_mod, rt):
    """Every row-tile count, with fewer workgroups than tiles (each walks
    several (row block, column block) tiles) and ragged K."""
    m, K, N = 16 * rt + 5, 32 * 61, 200
    d = W.generate(m, K, N, W.F16 if rt % 2 else W.BF16, rt != 2, 0.002, 0.02, 1.0, 720 + rt)
    for wg in (1, 3):
        plan = dict(engine=2, row_tiles=rt, cols_per_tile=64, waves_per_wg=4, workgroups=wg)
        assert_parity(oracle_mod, d, m, "prefill rt=%d wg=%d" % (rt, wg), plan)


def test_prefill_engine_for_decode_heights(oracle_mod):
    """The prefill engine also serves m <= 8 when asked for explicitly."""
    d = W.generate(3, 4096, 129, W.BF16, True, 0.001, 0.01, 0.5, 730)
    plan = dict(engine=2, row_tiles=1, cols_per_tile=64, waves_per_wg=4, workgroups=2)
    assert_parity(oracle_mod, d, 3, "prefill m=3", plan)


def test_prefill_rows_do_not_depend_on_launch_height():
    """Rows 0..16 of a 40-row launch equal a 17-row launch of the same rows,
    under different row tilings."""
    d = W.generate(40, 14336, 96, W.BF16, True, 0.001, 0.01, 0.5, 740)
    y40, _ = run(d, 40, W.BF16)
    p17 = dict(engine=2, row_tiles=2, cols_per_tile=64, waves_per_wg=4, workgroups=5)
    y17, _ = run(dict(d, A=d["A"][:17]), 17, W.BF16, p17)
    assert np.array_equal(y40[:17], y17)

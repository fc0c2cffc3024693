"""GPU tests of the offline even/odd nibble layout (the second page's PORT-1
interleave, pull request "PORT-1 (offline bias+interleave)", "Method"):
the layout conversion entry point against a numpy statement of the layout,
and the GEMV reading that layout against the fp64 oracle (which takes the
natural layout) through the C ABI.
"""
import numpy as np
import pytest
import torch

import block_wise_int4_matmulnbits_amd as mnb
from block_wise_int4_matmulnbits_amd import workloads as W
from tests import gpu_util as G
from tests.hand_cases import build_case, load_cases
from tests.test_gpu_parity import _workload_inputs, assert_parity, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    mnb.lib()


def even_odd(B):
    """The layout as the header states it: in every little-endian 32-bit word
    of a row, nibble p holds weight 2(p mod 4) + p/4 of the word's eight."""
    w = np.ascontiguousarray(B).view("<u4").astype(np.uint64)
    out = np.zeros_like(w)
    for p in range(8):
        k = 2 * (p % 4) + p // 4
        out |= ((w >> np.uint64(4 * k)) & np.uint64(0xF)) << np.uint64(4 * p)
    return out.astype("<u4").view(np.uint8).reshape(B.shape)


def test_even_odd_statement():
    """The numpy statement against a hand-built word: weights 0..7 in
    natural order give 0x75316420 in the even/odd layout."""
    nat = np.array([[0x10, 0x32, 0x54, 0x76]], np.uint8)
    assert even_odd(nat).view("<u4")[0, 0] == 0x75316420


@pytest.mark.parametrize("N,K", [(1, 32), (7, 96), (300, 4096), (4096, 14336)])
def test_repack_matches_statement_and_round_trips(N, K):
    rng = np.random.default_rng(N + K)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    src = torch.from_numpy(B).cuda()
    eo = torch.empty_like(src)
    mnb.mnb_repack_weights(src, mnb.MNB_LAYOUT_NATURAL, eo, mnb.MNB_LAYOUT_EVEN_ODD)
    back = torch.empty_like(src)
    mnb.mnb_repack_weights(eo, mnb.MNB_LAYOUT_EVEN_ODD, back, mnb.MNB_LAYOUT_NATURAL)
    same = torch.empty_like(src)
    mnb.mnb_repack_weights(src, mnb.MNB_LAYOUT_NATURAL, same, mnb.MNB_LAYOUT_NATURAL)
    inplace = src.clone()
    mnb.mnb_repack_weights(inplace, mnb.MNB_LAYOUT_NATURAL, inplace, mnb.MNB_LAYOUT_EVEN_ODD)
    torch.cuda.synchronize()
    want = even_odd(B)
    assert np.array_equal(eo.cpu().numpy(), want)
    assert np.array_equal(inplace.cpu().numpy(), want)
    assert np.array_equal(back.cpu().numpy(), B)
    assert np.array_equal(same.cpu().numpy(), B)


def _eo_plan(d, m):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = mnb.plan_for_device(m, d["K"], d["N"], cus).as_dict()
    p["b_layout"] = mnb.MNB_LAYOUT_EVEN_ODD
    return p


@pytest.mark.parametrize("name,m", [
    ("tiny_1k", 1), ("asym_4k", 1), ("gate_up_bf16", 1), ("down_rows_bf16", 2),
    ("down_rows_bf16", 8), ("lm_head", 1),
])
def test_even_odd_layout_parity(oracle_mod, name, m):
    """The same call on even/odd weights, every output against the oracle
    on the natural weights (checks 1 and 2)."""
    d = _workload_inputs(name)
    de = dict(d, B=even_odd(d["B"]))
    assert_parity(oracle_mod, de, m, name + " even/odd", _eo_plan(d, m),
                  ref=oracle_mod.matmul_nbits(d["A"][:m], d["a_dtype"] == W.BF16, d["B"],
                                              d["scales"], d["zp"], m, d["K"], d["N"]))


@pytest.mark.parametrize("lpc,bpl,nc", [(16, 2, 2), (32, 1, 4), (64, 2, 2), (128, 1, 1), (448, 1, 2)])
def test_even_odd_layout_every_mode(oracle_mod, lpc, bpl, nc):
    """Lane groups of 16 and 32 lanes, one wave and several waves, ragged K."""
    m, K, N = 2, 32 * 61, 77
    d = W.generate(m, K, N, W.BF16, True, 0.002, 0.02, 1.0, 760 + lpc)
    de = dict(d, B=even_odd(d["B"]))
    plan = dict(lanes_per_col=lpc, blocks_per_lane=bpl, cols_per_tile=nc, workgroups=5,
                interleave=1, b_layout=mnb.MNB_LAYOUT_EVEN_ODD)
    assert_parity(oracle_mod, de, m, "even/odd lpc=%d" % lpc, plan,
                  ref=oracle_mod.matmul_nbits(d["A"][:m], True, d["B"], d["scales"], d["zp"],
                                              m, K, N))


def test_even_odd_layout_mfma4_engine(oracle_mod):
    """The 4x4x4 MFMA kernel on even/odd weights: ragged K and N, one and
    two row quads, one and two column quads per tile."""
    for i, (m, K, N, w, bpl, cols) in enumerate(((2, 32 * 61, 77, 4, 1, 4), (7, 32 * 61, 45, 2, 2, 4),
                                                  (4, 4096, 130, 4, 2, 8), (8, 14336, 33, 7, 4, 4))):
        d = W.generate(m, K, N, W.BF16 if i % 2 else W.F16, i != 2, 0.002, 0.02, 1.0, 780 + i)
        de = dict(d, B=even_odd(d["B"]))
        plan = dict(engine=3, waves_per_wg=w, blocks_per_lane=bpl, cols_per_tile=cols, workgroups=3,
                    b_layout=mnb.MNB_LAYOUT_EVEN_ODD)
        assert_parity(oracle_mod, de, m, "even/odd mfma4", plan,
                      ref=oracle_mod.matmul_nbits(d["A"][:m], d["a_dtype"] == W.BF16, d["B"], d["scales"],
                                                  d["zp"], m, K, N))


CASES = load_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_case_even_odd(case):
    """The golden bits hold for the even/odd layout too (every hand case's
    sums are exact in fp32, so the pairing of the products cannot move them)."""
    c = build_case(case)
    d = dict(A=c["A"], B=even_odd(c["B"]), scales=c["scales"], zp=c["zp"], m=c["m"],
             K=c["K"], N=c["N"], a_dtype=W.BF16 if c["a_is_bf16"] else W.F16)
    plan = _eo_plan(d, c["m"])
    y16, _ = run(d, c["m"], W.F16, plan)
    ybf, _ = run(d, c["m"], W.BF16, plan)
    assert np.array_equal(y16, c["f16"]), [hex(v) for v in y16.ravel()]
    assert np.array_equal(ybf, c["bf16"]), [hex(v) for v in ybf.ravel()]

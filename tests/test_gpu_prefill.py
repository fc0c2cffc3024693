"""GPU parity of the prefill path (m > 8 rows, the matrix-core tile kernel)
against the fp64 oracle, through the C ABI.

Same acceptance as the decode path: check 1 on the fp16 output against the
exact weights, check 2 (bf16 output bit-identical to the narrowing of the
fp16 output), counters, no stale element.  The prefill kernel multiplies
weights rounded to fp16, so it is also held to a much tighter bound against
the oracle run with the same rounded weights: the only difference left is
fp32 accumulation, at most (K/32 + 32 + S) roundings of 2^-24 relative to
sum |a w| (one chained MFMA per block, 32 products each, and S - 1 sums of
K slices), plus one fp16 ulp for the output rounding (the tiles that split
K over their waves or over workgroups add the slices' fp32 sums at the end:
fewer roundings in a chain, not more).  The summation order of an output
depends only on K and on how the plan splits K, so rows computed in
launches of different heights under tilings that do not split K are
bit-identical.
"""
import numpy as np
import pytest
import torch

import block_wise_int4_matmulnbits_amd as mnb
from block_wise_int4_matmulnbits_amd import workloads as W
from tests import gpu_util as G
from tests.hand_cases import build_case, load_cases
from tests.test_gpu_parity import assert_parity, effective_plan, run


def fp16_weight_tol(oracle_mod, ref, K, splits=1):
    """Bound of the prefill kernel against the oracle run with the kernel's
    fp16 weights: the fp32 roundings of one output's chain, plus one ulp."""
    return (K // 32 + 32 + max(splits, 1)) * 2.0 ** -24 * ref["abs"] + oracle_mod.f16_ulp(ref["f16"])


def assert_prefill(oracle_mod, d, m, label, plan=None):
    """Checks 1 and 2; when the call runs the prefill kernel, also the bound
    of its fp16-weight reading."""
    y16, _, _ = assert_parity(oracle_mod, d, m, label, plan)
    eff = effective_plan(m, d["K"], d["N"], plan)
    if eff.get("engine") != 2:
        return y16
    K = d["K"]
    ref = oracle_mod.matmul_nbits(d["A"][:m], d["a_dtype"] == W.BF16, d["B"], d["scales"],
                                  d["zp"], m, K, d["N"], weights_f16=True)
    g = G.f16_values(y16)
    err = np.abs(g - ref["f64"])
    tol = fp16_weight_tol(oracle_mod, ref, K, eff.get("k_splits", 1))
    bad = ~(err <= tol)
    assert not bad.any(), "fp16-weight bound failed at %d of %d outputs" % (bad.sum(), bad.size)
    G.log("[parity] %s: within %.3g of the fp16-weight bound" % (label, float(np.max(err / tol))))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()
    mnb.lib()


# The planner's cost model picks these plans at 256 CUs (row tiles, columns,
# waves, K splits over workgroups), or "decode" for the 8-row decode plan
# run per 8 rows (explicit decode plans above 8 rows are tested below).
@pytest.mark.parametrize("m,K,N,a_dtype,asym,want", [
    (9, 4096, 1000, W.F16, True, (1, 128, 4, 16)),     # few columns: K over 16 workgroups (9.3 us, two decode launches 10.2)
    (16, 4096, 64, W.BF16, True, (1, 128, 4, 16)),     # one column tile, K over 16 workgroups (8.3 us, decode 11.5)
    (17, 1024, 130, W.F16, False, (1, 16, 4, 1)),      # ragged rows and columns, zero point 8, 16-column tiles
    (12, 4096, 6144, W.BF16, True, (1, 128, 4, 4)),    # K over four workgroups at 12 rows
    (9, 2048, 8200, W.F16, False, (1, 256, 8, 4)),     # K over four workgroups, ragged columns
    (100, 32 * 37, 77, W.BF16, True, (1, 16, 4, 1)),   # K not a whole number of 128-wide steps
    (130, 14336, 300, W.BF16, True, (1, 128, 4, 16)),  # down-projection K over 16 workgroups, row tail of 2
    (256, 4096, 1024, W.F16, True, (1, 32, 4, 1)),     # several row and column blocks, K over four waves
    (192, 4096, 6144, W.BF16, True, (2, 128, 4, 1)),   # two 32-row tiles of 128 columns
    (40, 4096, 65536, W.F16, True, (2, 256, 8, 1)),    # two row tiles of 256 columns, several rounds
    (1152, 1024, 4096, W.BF16, True, (4, 256, 8, 1)),  # 128 x 256 tiles
    (640, 512, 14336, W.F16, True, (8, 256, 8, 1)),    # 256 x 256 tiles, weights through LDS
    (1152, 512, 14336, W.BF16, True, (4, 256, 8, 1)),  # 128 x 256 tiles where 256 x 256 would take more rounds
])
def test_prefill_default_plan(oracle_mod, m, K, N, a_dtype, asym, want):
    d = W.generate(m, K, N, a_dtype, asym, 0.001, 0.01, 0.5, 700 + m)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = mnb.plan_for_device(m, K, N, cus)
    if cus == 256:
        if want == "decode":
            assert plan.engine != 2 and plan.as_dict() == mnb.plan_for_device(8, K, N, cus).as_dict()
        else:
            got = (plan.row_tiles, plan.cols_per_tile, plan.waves_per_wg, max(plan.k_splits, 1))
            assert plan.engine == 2 and got == want
    assert_prefill(oracle_mod, d, m, "prefill", None)


@pytest.mark.parametrize("rt", [1, 2, 4])
@pytest.mark.parametrize("cols,waves", [(64, 2), (128, 4), (256, 4), (256, 8)])
def test_prefill_every_tiling_and_small_grids(oracle_mod, rt, cols, waves):
    """One, two or four 32-row tiles; four waves of 32 or 64 columns or
    eight of 32; fewer workgroups than tiles (each walks several (row block,
    column block) tiles), ragged rows, columns and K."""
    m, K, N = 32 * rt + 5, 32 * 61, 300
    d = W.generate(m, K, N, W.F16 if rt % 2 else W.BF16, rt != 2, 0.002, 0.02, 1.0,
                   720 + rt + cols + waves)
    for wg in (1, 3, 13):
        plan = dict(engine=2, row_tiles=rt, cols_per_tile=cols, waves_per_wg=waves, workgroups=wg)
        assert_prefill(oracle_mod, d, m, "prefill rt=%d cols=%d waves=%d wg=%d" % (rt, cols, waves, wg),
                       plan)


@pytest.mark.parametrize("m,K,N,a_dtype,asym", [
    (261, 32 * 61, 300, W.BF16, True),     # ragged rows, columns, odd block count
    (40, 4096, 513, W.F16, False),         # one partial row block, zero point 8
    (512, 14336, 260, W.BF16, True),       # two row blocks, long K
    (300, 0, 600, W.BF16, True),           # K = 0: every output +0
    (300, 32, 600, W.F16, True),           # one block: half of the only stage
])
def test_prefill_lds_staged_tiles(oracle_mod, m, K, N, a_dtype, asym):
    """256 x 256 tiles with the weights dequantized once per workgroup into
    LDS (row_tiles 8, eight waves), with 1, 3 and 13 workgroups."""
    d = W.generate(m, K, N, a_dtype, asym, 0.002, 0.02, 1.0, 800 + m)
    for wg in (1, 3, 13):
        plan = dict(engine=2, row_tiles=8, cols_per_tile=256, waves_per_wg=8, workgroups=wg)
        assert_prefill(oracle_mod, d, m, "prefill lds-staged wg=%d" % wg, plan)


@pytest.mark.parametrize("cols,waves", [(32, 4), (16, 4), (16, 8)])
@pytest.mark.parametrize("m,K,N", [(5, 32 * 61, 300), (37, 32 * 61, 300), (100, 32 * 61, 300),
                                   (40, 32, 77), (33, 0, 64), (64, 4096, 1000), (20, 32 * 13, 90)])
def test_prefill_k_split_tiles(oracle_mod, m, K, N, cols, waves):
    """32-row tiles of 32 columns whose K four waves split, or of 16 columns
    split over four or eight waves (slice s takes quads s, s + waves, ...; an odd quad count, fewer quads
    than slices, a single block, K = 0), with 1, 3 and 13 workgroups and the
    default grid; ragged rows and columns."""
    d = W.generate(m, K, N, W.BF16 if m % 2 else W.F16, m != 40, 0.002, 0.02, 1.0, 900 + m)
    for wg in (1, 3, 13, -(-m // 32) * -(-N // cols)):
        plan = dict(engine=2, row_tiles=1, cols_per_tile=cols, waves_per_wg=waves, workgroups=wg)
        assert_prefill(oracle_mod, d, m, "prefill k-split %dx%d wg=%d" % (cols, waves, wg), plan)


@pytest.mark.parametrize("m", [16, 23, 32, 48, 64, 128])
def test_down_projection_k_split_default(oracle_mod, m):
    """The down projection (K = 14336, N = 4096) with 16..128 rows: the
    default plan splits K over workgroups (two launches: the tiles, then the
    sum of their slices); check 1 on sampled columns, check 2 on every
    output."""
    K, N = 14336, 4096
    d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, 920 + m)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = mnb.plan_for_device(m, K, N, cus)
    assert plan.engine == 2
    if cus == 256:
        assert plan.k_splits > 1
    G.log("[parity] down m=%d k-split, plan %s" % (m, plan.as_dict()))
    y16, c = run(d, m, W.F16)
    assert c["launches"] == (2 if plan.k_splits > 1 else 1)
    ybf, _ = run(d, m, W.BF16)
    assert not np.any(y16 == 0xFFFF)
    assert G.check2(ybf, y16, oracle_mod).all()
    cols = np.unique(np.concatenate([[0, 1, 31, 32, N - 1], np.random.default_rng(921).choice(N, 20, replace=False)]))
    ref = oracle_mod.matmul_nbits(d["A"][:m], True, d["B"], d["scales"], d["zp"], m, K, N, cols=cols)
    ok, _ = G.check1(y16[:, cols], ref, oracle_mod)
    assert ok.all()


@pytest.mark.parametrize("m", [9, 16])
def test_decode_plan_runs_per_8_rows(oracle_mod, m):
    """The down projection's K over 512 columns with 9..16 rows under the
    8-row decode plan (an explicit plan; the default splits K over
    workgroups there, 12.0 us against 17.6-20.3 for the decode launches):
    launches of 8 rows against the oracle, and each block of 8 rows
    bit-equal to its own launch."""
    K, N = 14336, 512
    d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, 860 + m)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert mnb.plan_for_device(m, K, N, cus).engine == 2
    plan = mnb.plan_for_device(8, K, N, cus)
    assert plan.engine == 3
    y16 = assert_prefill(oracle_mod, d, m, "decode per 8 rows", plan.as_dict())
    for r0 in range(0, m, 8):
        mc = min(8, m - r0)
        y, _ = run(dict(d, A=d["A"][r0:r0 + mc]), mc, W.F16, plan.as_dict())
        assert np.array_equal(y, y16[r0:r0 + mc])


@pytest.mark.parametrize("m", [9, 16])
def test_lm_head_few_rows_on_tiles(oracle_mod, m):
    """The lm_head shape (K = 4096, N = 151936) with 9 and 16 rows runs one
    launch of 32-row tiles: check 1 on sampled columns, check 2 on every
    output, and rows 0..8 equal to a 9-row launch of the same plan."""
    K, N = 4096, 151936
    d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, 880 + m)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = mnb.plan_for_device(m, K, N, cus)
    assert plan.engine == 2 and plan.row_tiles == 1
    G.log("[parity] lm_head m=%d on tiles, plan %s" % (m, plan.as_dict()))
    y16, c = run(d, m, W.F16)
    assert c["launches"] == 1
    ybf, _ = run(d, m, W.BF16)
    assert not np.any(y16 == 0xFFFF)
    assert G.check2(ybf, y16, oracle_mod).all()
    cols = np.unique(np.concatenate([[0, 1, 2, 3, N - 1], np.random.default_rng(881).choice(N, 24, replace=False)]))
    ref = oracle_mod.matmul_nbits(d["A"][:m], True, d["B"], d["scales"], d["zp"], m, K, N, cols=cols)
    ok, _ = G.check1(y16[:, cols], ref, oracle_mod)
    assert ok.all()
    y9, _ = run(dict(d, A=d["A"][:9]), 9, W.F16, plan.as_dict())
    assert np.array_equal(y9, y16[:9])


def test_prefill_engine_for_decode_heights(oracle_mod):
    """The prefill engine also serves m <= 8 when asked for explicitly."""
    d = W.generate(3, 4096, 129, W.BF16, True, 0.001, 0.01, 0.5, 730)
    plan = dict(engine=2, row_tiles=1, cols_per_tile=128, waves_per_wg=4, workgroups=2)
    assert_prefill(oracle_mod, d, 3, "prefill m=3", plan)


def test_prefill_rows_do_not_depend_on_launch_height():
    """Rows 0..16 of a 40-row launch equal a 17-row launch of the same rows,
    under different row tilings."""
    d = W.generate(40, 14336, 96, W.BF16, True, 0.001, 0.01, 0.5, 740)
    y40, _ = run(d, 40, W.BF16, dict(engine=2, row_tiles=2, cols_per_tile=128, waves_per_wg=4, workgroups=1))
    p17 = dict(engine=2, row_tiles=4, cols_per_tile=256, waves_per_wg=4, workgroups=5)
    y17, _ = run(dict(d, A=d["A"][:17]), 17, W.BF16, p17)
    assert np.array_equal(y40[:17], y17)


@pytest.mark.parametrize("name,K,N,m", [("gate_up", 4096, 28672, 2048), ("gate_up", 4096, 28672, 512),
                                        ("down", 14336, 4096, 512)])
def test_prefill_full_size_sampled(oracle_mod, name, K, N, m):
    """The benchmarked prefill shapes at full size under the default plan:
    check 1 and the fp16-weight bound on a sample of whole columns (every
    row), check 2 on every output."""
    d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, 750 + m)
    G.log("[parity] prefill %s m=%d K=%d N=%d default plan" % (name, m, K, N))
    plan = mnb.plan_for_device(m, K, N, torch.cuda.get_device_properties(0).multi_processor_count)
    y16, c16 = run(d, m, W.F16)
    ybf, _ = run(d, m, W.BF16)
    assert c16["launches"] == (2 if plan.k_splits > 1 else 1)
    assert not np.any(y16 == 0xFFFF) and not np.any(ybf == 0xFFFF)
    assert G.check2(ybf, y16, oracle_mod).all()
    rng = np.random.default_rng(751)
    cols = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.choice(N, 28, replace=False)]))
    A = d["A"][:m]
    ref = oracle_mod.matmul_nbits(A, True, d["B"], d["scales"], d["zp"], m, K, N, cols=cols)
    ok, max_ulps = G.check1(y16[:, cols], ref, oracle_mod)
    assert ok.all(), "check 1 failed at %d of %d outputs" % ((~ok).sum(), ok.size)
    ref16 = oracle_mod.matmul_nbits(A, True, d["B"], d["scales"], d["zp"], m, K, N, cols=cols,
                                    weights_f16=True)
    err = np.abs(G.f16_values(y16[:, cols]) - ref16["f64"])
    assert (err <= fp16_weight_tol(oracle_mod, ref16, K, plan.k_splits)).all()
    G.log("[parity] prefill %s m=%d ok: max err %.3f fp16 ulp vs exact weights" % (name, m, max_ulps))


@pytest.mark.parametrize("m,K,N", [(9, 0, 5), (40, 32, 1), (33, 96, 257), (100, 32 * 3, 3)])
def test_prefill_edge_shapes(oracle_mod, m, K, N):
    """K = 0 (every output +0), a single column, one block, an odd block
    count with a ragged last quad, under the default plan."""
    d = W.generate(m, K, N, W.BF16, True, 0.002, 0.02, 1.0, 780 + m + K)
    assert_prefill(oracle_mod, d, m, "prefill edge", None)
    if K == 0:
        y, _ = run(d, m, W.F16)
        assert np.all(y == 0)


def test_prefill_longest_rows(oracle_mod):
    """K = 2^24 (the largest K), where a two-row-tile workgroup's 64
    activation rows span 2^31 bytes of 32-bit buffer offsets: sampled rows
    (the first and last of each 32-row tile) and both columns against the
    oracle, with a four-row-tile plan rejected."""
    m, K, N = 64, 1 << 24, 2
    q4 = dict(engine=2, row_tiles=4, cols_per_tile=128, waves_per_wg=4, workgroups=1)
    assert mnb.mnb_plan_check(m, K, N, mnb.mnb_plan(**q4)) == 9
    rng = np.random.default_rng(790)
    # Activations: a few nonzero stretches per row (at the start, in the
    # middle and in the last block), so the sums reach every part of K.
    A = np.zeros((m, K), np.uint16)
    for r in range(m):
        for start in (0, K // 2 + 32 * r, K - 32):
            A[r, start:start + 32] = (rng.standard_normal(32) * 0.5).astype(np.float16).view(np.uint16)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    S = rng.uniform(0.002, 0.02, (N, K // 32)).astype(np.float16).view(np.uint16)
    Z = rng.integers(0, 256, (N, K // 64), dtype=np.uint8)
    d = dict(A=A, B=B, scales=S, zp=Z, m=m, K=K, N=N, a_dtype=W.F16)
    plan = dict(engine=2, row_tiles=2, cols_per_tile=128, waves_per_wg=4, workgroups=1)
    y16, c16 = run(d, m, W.F16, plan)
    ybf, _ = run(d, m, W.BF16, plan)
    assert c16["launches"] == 1
    assert G.check2(ybf, y16, oracle_mod).all()
    rows = np.array([0, 1, 31, 32, 62, 63])
    ref = oracle_mod.matmul_nbits(A[rows], False, B, S, Z, len(rows), K, N)
    ok, max_ulps = G.check1(y16[rows], ref, oracle_mod)
    assert ok.all(), max_ulps
    ref16 = oracle_mod.matmul_nbits(A[rows], False, B, S, Z, len(rows), K, N, weights_f16=True)
    err = np.abs(G.f16_values(y16[rows]) - ref16["f64"])
    assert (err <= (K // 32 + 32) * 2.0 ** -24 * ref16["abs"] + oracle_mod.f16_ulp(ref16["f16"])).all()


HAND = load_cases()


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
def test_hand_case_through_prefill_engine(case):
    """Every hand case's weights are fp16 numbers, so the prefill kernel's
    fp16 dequant changes nothing and the golden bits must hold exactly: the
    case's rows alone, and repeated to 40 rows (two row tiles of 32)."""
    c = build_case(case)
    for reps in (1, -(-40 // c["m"])):
        A = np.tile(c["A"], (reps, 1))
        m = A.shape[0]
        d = dict(A=A, B=c["B"], scales=c["scales"], zp=c["zp"], m=m, K=c["K"], N=c["N"],
                 a_dtype=W.BF16 if c["a_is_bf16"] else W.F16)
        plan = dict(engine=2, row_tiles=1, cols_per_tile=128, waves_per_wg=4, workgroups=1)
        y16, _ = run(d, m, W.F16, plan)
        ybf, _ = run(d, m, W.BF16, plan)
        assert np.array_equal(y16, np.tile(c["f16"], (reps, 1))), [hex(v) for v in y16[:c["m"]].ravel()]
        assert np.array_equal(ybf, np.tile(c["bf16"], (reps, 1))), [hex(v) for v in ybf[:c["m"]].ravel()]


@pytest.mark.parametrize("rt,cols,waves", [(1, 128, 4), (2, 128, 4), (4, 128, 4), (1, 256, 8), (2, 256, 8),
                                           (1, 64, 2), (1, 32, 4), (1, 16, 8)])
@pytest.mark.parametrize("m,K,N,splits", [(37, 32 * 61, 300, 3),    # ragged rows, columns, odd block count
                                          (9, 4096, 513, 7),        # 32 steps in 7 unequal slices
                                          (70, 32 * 13, 90, 4),     # 4 steps, one per slice (the last ragged)
                                          (20, 14336, 260, 16)])    # long K, 16 slices
def test_prefill_k_split_over_workgroups(oracle_mod, rt, cols, waves, m, K, N, splits):
    """K split over workgroups: each workgroup takes one slice of K for its
    tile and leaves fp32 partial sums, a second launch adds the slices in
    order and narrows.  Every tiling that takes a split, with 1, 3 and 13
    workgroups and the full grid; zero points absent in one case."""
    d = W.generate(m, K, N, W.BF16 if m % 2 else W.F16, m != 70, 0.002, 0.02, 1.0, 960 + m + rt + cols)
    tiles = -(-m // (32 * rt)) * -(-N // cols) * splits
    for wg in (1, 3, 13, tiles):
        plan = dict(engine=2, row_tiles=rt, cols_per_tile=cols, waves_per_wg=waves, workgroups=wg,
                    k_splits=splits)
        assert_prefill(oracle_mod, d, m, "prefill %dx%dx%d split %d wg=%d" % (rt, cols, waves, splits, wg), plan)


def test_k_split_is_deterministic_across_workspace_reuse():
    """Split plans of different workspace sizes in a row on one stream, then
    on a second stream: every call of a plan gives the same bits, and the
    launch counter counts the tiles and the sum of the slices."""
    m, K, N = 40, 14336, 1000
    d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, 990)
    big = dict(engine=2, row_tiles=2, cols_per_tile=128, waves_per_wg=4, workgroups=256, k_splits=16)
    small = dict(engine=2, row_tiles=1, cols_per_tile=256, waves_per_wg=8, workgroups=64, k_splits=2)
    y_big, c = run(d, m, W.BF16, big)
    assert c["launches"] == 2
    y_small, _ = run(d, m, W.BF16, small)
    y_big2, _ = run(d, m, W.BF16, big)
    assert np.array_equal(y_big, y_big2)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y_small2, _ = run(d, m, W.BF16, small)
        y_big3, _ = run(d, m, W.BF16, big)
    torch.cuda.synchronize()
    assert np.array_equal(y_small, y_small2) and np.array_equal(y_big, y_big3)
    _, c1 = run(d, m, W.BF16, dict(big, k_splits=1))
    assert c1["launches"] == 1


def test_k_split_default_few_columns(oracle_mod):
    """9 and 16 rows of the down projection's K over 2048 columns: the
    default plan splits K over workgroups; full parity."""
    for m in (9, 16):
        K, N = 14336, 2048
        d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, 995 + m)
        plan = mnb.plan_for_device(m, K, N, torch.cuda.get_device_properties(0).multi_processor_count)
        G.log("[parity] %dx%dx%d default plan %s" % (m, K, N, plan.as_dict()))
        assert_prefill(oracle_mod, d, m, "split default m=%d" % m, None)


def test_k_split_workspace_growth_and_eviction():
    """The per-stream workspace: a small split call and then a larger one on
    a new stream (the buffer grows after the stream drains), and split calls
    on more streams than the library's table holds (the least recently used
    buffer is given up after the device drains): every output equals the
    same call on the default stream."""
    small = dict(engine=2, row_tiles=1, cols_per_tile=128, waves_per_wg=4, workgroups=64, k_splits=2)
    big = dict(engine=2, row_tiles=2, cols_per_tile=128, waves_per_wg=4, workgroups=256, k_splits=16)
    d_small = W.generate(9, 4096, 300, W.BF16, True, 0.001, 0.01, 0.5, 1101)
    d_big = W.generate(40, 14336, 1000, W.BF16, True, 0.001, 0.01, 0.5, 1102)
    ref_small, _ = run(d_small, 9, W.BF16, small)
    ref_big, _ = run(d_big, 40, W.BF16, big)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1, _ = run(d_small, 9, W.BF16, small)      # 9 * 300 * 2 floats
        y2, _ = run(d_big, 40, W.BF16, big)         # 40 * 1000 * 16 floats: grows
        y3, _ = run(d_small, 9, W.BF16, small)
    assert np.array_equal(y1, ref_small) and np.array_equal(y2, ref_big) and np.array_equal(y3, ref_small)
    streams = [torch.cuda.Stream() for _ in range(40)]   # more than the 32 entries of the table
    outs = []
    for st in streams:
        with torch.cuda.stream(st):
            y, _ = run(d_small, 9, W.BF16, small)
            outs.append(y)
    with torch.cuda.stream(streams[0]):               # its entry was given up: a new one
        y, _ = run(d_big, 40, W.BF16, big)
    torch.cuda.synchronize()
    assert all(np.array_equal(o, ref_small) for o in outs)
    assert np.array_equal(y, ref_big)


@pytest.mark.parametrize("m,K,N", [(5, 32 * 611, 150), (8, 28672, 600), (3, 36864, 300), (2, 65568, 70)])
def test_long_k_rows_run_prefill_tiles(oracle_mod, m, K, N):
    """Two to eight rows whose K the decode lane split would walk in chunks
    (K > 16384 at five or more rows, > 32768 at three or four, > 65536 at
    two): the default plan runs the prefill tiles instead, with K split over
    workgroups where the model prices it lower; full parity, including a
    ragged K."""
    d = W.generate(m, K, N, W.BF16, True, 0.001, 0.01, 0.5, 1300 + m)
    plan = mnb.plan_for_device(m, K, N, torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan.engine == 2, plan.as_dict()
    G.log("[parity] long K m=%d K=%d N=%d plan %s" % (m, K, N, plan.as_dict()))
    assert_prefill(oracle_mod, d, m, "long K rows", None)

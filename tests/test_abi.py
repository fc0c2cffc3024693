"""C ABI checks that need no GPU: the library loads, exports every symbol
the header declares, validates arguments before touching the device, and
plans launches consistently."""
import ctypes
import os
import re

import pytest

import block_wise_int4_matmulnbits_amd as mnb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mnb.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*"
                       r"([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_symbols_exported():
    names = _declared_functions()
    assert "matmul_nbits" in names and len(names) >= 10
    lib = ctypes.CDLL(mnb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), "libmnb.so does not export %s" % n
    assert set(mnb.EXPORTS) == set(names)


def test_abi_version_matches_header():
    v = int(re.search(r"#define MNB_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert mnb.mnb_abi_version() == v


FAKE = 0x10000  # never dereferenced: validation fails first


@pytest.mark.parametrize("args,status", [
    (dict(m=(1 << 20) + 1), 6), (dict(m=-1), 6), (dict(K=33), 2), (dict(K=-32), 2),
    (dict(N=-1), 2), (dict(block=64), 3), (dict(a_dtype=2), 4),
    (dict(out_dtype=-1), 4), (dict(A=0), 1), (dict(B=0), 1), (dict(S=0), 1),
    (dict(out=0), 1), (dict(A=FAKE + 8), 5), (dict(B=FAKE * 3 + 4), 5),
    (dict(S=FAKE * 5 + 1), 5), (dict(out=FAKE * 7 + 1), 5),
    (dict(out=FAKE + 64), 8), (dict(K=1 << 25), 2),
])
def test_validation_without_gpu(args, status):
    a = dict(A=FAKE, a_dtype=0, m=1, K=64, N=4, B=FAKE * 3, S=FAKE * 5, Z=None,
             block=32, out=FAKE * 7, out_dtype=0)
    a.update(args)
    c0 = mnb.mnb_counters_get()
    st = mnb.matmul_nbits_raw(a["A"], a["a_dtype"], a["m"], a["K"], a["N"], a["B"],
                              a["S"], a["Z"], a["block"], a["out"], a["out_dtype"])
    assert st == status, mnb.mnb_status_string(st)
    assert mnb.mnb_counters_get() == c0
    assert mnb.mnb_status_string(st) != "unknown status"


def test_empty_problem_is_ok_without_gpu():
    c0 = mnb.mnb_counters_get()
    assert mnb.matmul_nbits_raw(0, 0, 0, 64, 4, 0, 0, 0, 32, 0, 0) == 0
    assert mnb.matmul_nbits_raw(0, 1, 3, 64, 0, 0, 0, 0, 32, 0, 1) == 0
    c1 = mnb.mnb_counters_get()
    assert c1["calls"] == c0["calls"] + 2 and c1["launches"] == c0["launches"]


SHAPES = [(m, K, N) for m in range(1, 9)
          for K in (0, 32, 96, 1024, 4096, 14336, 32 * 611, 65536, 262144)
          for N in (1, 7, 1024, 4096, 28672, 151936)]


def test_default_plans_are_valid_and_cover_k():
    split3 = {}
    for m, K, N in SHAPES:
        for cus, occ in ((1, 0), (80, 3), (256, 0), (256, 5), (304, 1)):
            p = mnb.mnb_plan_default(m, K, N, cus, occ)
            q = mnb.mnb_plan(**{f: getattr(p, f) for f, _ in mnb.mnb_plan._fields_})
            assert mnb.mnb_plan_check(m, K, N, q) == 0
            nb = K // 32
            if p.engine == 3:
                # The 4x4x4 MFMA kernel: four or more rows, K in one pass of
                # the workgroup's 16 * waves lane groups; its lane split
                # depends on K only.
                assert 2 <= m <= 8 and 1 <= nb <= 512
                w, bpl = p.waves_per_wg, p.blocks_per_lane
                assert bpl in (1, 2, 4) and 16 * w * bpl >= nb
                if w <= 4:      # the fewest waves, and the fewest blocks for <= 4 waves
                    assert nb > 16 * (w - 1) * bpl and (bpl == 1 or 16 * 4 * (bpl // 2) < nb)
                else:           # more than four waves of four: eight (some of three blocks)
                    assert w == 8 and bpl == 4 and nb > 256
                assert p.cols_per_tile == 4
                assert split3.setdefault(K, (w, bpl)) == (w, bpl)
                assert q.k_chunks == 1 and q.threads_per_wg == 64 * w
                assert p.cols_per_tile in (4, 8) and not (m > 4 and bpl * p.cols_per_tile // 4 > 4)
                tiles = -(-(-(-N // 4)) // (p.cols_per_tile // 4))
                assert 1 <= p.workgroups <= max(1, -(-tiles // 2))   # two tiles per workgroup
                continue
            if p.engine == 2:
                # Two or more rows whose K the decode lane split would walk
                # in chunks (more blocks than 512 lanes of 8 // m blocks
                # each): the prefill tiles, K split over workgroups.
                assert 2 <= m <= 8 and nb > 512 * max(1, min(4, 8 // m)), (m, K)
                assert q.threads_per_wg == 64 * p.waves_per_wg and q.k_chunks == (nb + 3) // 4
                continue
            assert p.engine == 0 and not (m >= 2 and 1 <= nb <= 512)
            lpc, bpl, nc = p.lanes_per_col, p.blocks_per_lane, p.cols_per_tile
            assert m == 1 or p.k_chunks == 1      # chunked passes only at one row
            assert lpc * bpl * p.k_chunks >= K // 32
            assert m * bpl <= 8 and nc * bpl <= 8 and nc * m <= 32
            assert p.threads_per_wg in (256, lpc) and p.threads_per_wg <= 512
            gpw = 256 // lpc if lpc <= 64 else 1
            groups = p.workgroups * gpw
            assert 1 <= groups <= N + gpw - 1   # no workgroup without columns


PREFILL_SHAPES = [(m, K, N) for m in (9, 16, 17, 100, 1000, 4096, 1 << 20)
                  for K in (0, 32, 96, 4096, 14336, 32 * 611)
                  for N in (1, 63, 64, 4096, 151936)]


def test_default_prefill_plans():
    """m > 8: a prefill tiling, or the 8-row decode plan run per 8 rows,
    whichever the planner's cost model prices lowest (the model itself is
    checked against measured times in test_planner_model.py).  Here: every
    choice is a plan the check accepts, no more workgroups than tiles, one
    resident generation at most, and the benchmark's prefill shapes on the
    tilings measured fastest for them."""
    for m, K, N in PREFILL_SHAPES:
        for cus, occ in ((1, 0), (256, 0), (256, 2), (304, 1)):
            p = mnb.mnb_plan_default(m, K, N, cus, occ)
            if p.engine != 2:
                assert p.as_dict() == mnb.mnb_plan_default(8, K, N, cus, occ).as_dict(), (m, K, N, cus)
                continue
            q = mnb.mnb_plan(**{f: getattr(p, f) for f, _ in mnb.mnb_plan._fields_})
            assert mnb.mnb_plan_check(m, K, N, q) == 0
            assert q.threads_per_wg == 64 * p.waves_per_wg and q.k_chunks == (K // 32 + 3) // 4
            rows = 256 if p.row_tiles == 8 else 32 * p.row_tiles
            splits = max(p.k_splits, 1)
            tiles = -(-m // rows) * -(-N // p.cols_per_tile) * splits
            assert 1 <= p.workgroups <= min(tiles, max(occ, 1) * cus), (m, K, N, cus)
            if splits > 1:   # to fill the device: under four rounds, within the workspace bound
                assert tiles < 4 * cus and splits * m * N * 4 <= mnb.MNB_MAX_SPLIT_WORKSPACE, (m, K, N, cus)
    # The benchmark's prefill shapes (gate_up m = 512 and 2048, down m = 16,
    # 64, 512 and 2048), on the tilings measured fastest for them.
    for m, K, N, want in ((512, 4096, 28672, (8, 256, 8, 1)), (2048, 4096, 28672, (8, 256, 8, 1)),
                          (16, 14336, 4096, (1, 128, 4, 8)), (64, 14336, 4096, (2, 128, 4, 8)),
                          (512, 14336, 4096, (2, 128, 4, 1)), (2048, 14336, 4096, (4, 256, 8, 1))):
        p = mnb.mnb_plan_default(m, K, N, 256, 0)
        assert (p.row_tiles, p.cols_per_tile, p.waves_per_wg, max(p.k_splits, 1)) == want, (m, K, N)


def test_plan_check_engines_and_rows():
    p = mnb.mnb_plan(engine=2, row_tiles=4, cols_per_tile=128, waves_per_wg=4, workgroups=3)
    assert mnb.mnb_plan_check(3, 4096, 100, p) == 0            # engine 2 takes any m >= 1
    assert mnb.mnb_plan_check(5000, 4096, 100, p) == 0
    for rt in (1, 2, 4):
        for cols, waves in ((128, 4), (256, 4), (256, 8)):
            q = mnb.mnb_plan(engine=2, row_tiles=rt, cols_per_tile=cols, waves_per_wg=waves, workgroups=1)
            assert mnb.mnb_plan_check(20, 4096, 100, q) == 0
            assert q.threads_per_wg == 64 * waves
    qs = mnb.mnb_plan(engine=2, row_tiles=1, cols_per_tile=32, waves_per_wg=4, workgroups=7)
    assert mnb.mnb_plan_check(20, 4096, 100, qs) == 0               # 32 columns, K split over 4 waves
    assert qs.threads_per_wg == 256 and qs.k_chunks == 32
    for bad in (dict(row_tiles=2), dict(row_tiles=4), dict(waves_per_wg=2), dict(waves_per_wg=8)):
        q = mnb.mnb_plan(**dict(dict(engine=2, row_tiles=1, cols_per_tile=32, waves_per_wg=4, workgroups=1), **bad))
        assert mnb.mnb_plan_check(20, 4096, 100, q) == 9, bad         # MNB_ERR_PLAN
    for waves in (4, 8):                                               # 16 columns, K split over 4 or 8 waves
        q = mnb.mnb_plan(engine=2, row_tiles=1, cols_per_tile=16, waves_per_wg=waves, workgroups=3)
        assert mnb.mnb_plan_check(20, 4096, 100, q) == 0 and q.threads_per_wg == 64 * waves and q.k_chunks == 32
    for bad in (dict(row_tiles=2), dict(waves_per_wg=2), dict(waves_per_wg=16)):
        q = mnb.mnb_plan(**dict(dict(engine=2, row_tiles=1, cols_per_tile=16, waves_per_wg=4, workgroups=1), **bad))
        assert mnb.mnb_plan_check(20, 4096, 100, q) == 9, bad
    q8 = mnb.mnb_plan(engine=2, row_tiles=8, cols_per_tile=256, waves_per_wg=8, workgroups=1)
    assert mnb.mnb_plan_check(20, 4096, 100, q8) == 0              # 256 x 256, weights through LDS
    for bad in (dict(row_tiles=3), dict(row_tiles=16), dict(row_tiles=8, waves_per_wg=4),
                dict(row_tiles=8, cols_per_tile=128, waves_per_wg=8), dict(cols_per_tile=64), dict(cols_per_tile=96),
                dict(cols_per_tile=512), dict(waves_per_wg=2), dict(waves_per_wg=8),
                dict(waves_per_wg=8, cols_per_tile=512), dict(waves_per_wg=16, cols_per_tile=256),
                dict(workgroups=0)):
        q = mnb.mnb_plan(**dict(dict(engine=2, row_tiles=4, cols_per_tile=128, waves_per_wg=4,
                                     workgroups=3), **bad))
        assert mnb.mnb_plan_check(20, 4096, 100, q) == 9
    # K split over workgroups: 1..64 slices of at least one 128-wide step,
    # not for the 256 x 256 tiles nor the decode engines (0 and 1 mean none).
    for splits in (0, 1, 2, 16, 32):
        q = mnb.mnb_plan(engine=2, row_tiles=2, cols_per_tile=128, waves_per_wg=4, workgroups=1, k_splits=splits)
        assert mnb.mnb_plan_check(20, 4096, 100, q) == 0, splits
    for splits in (-1, 33, 65):   # K = 4096: 32 steps
        q = mnb.mnb_plan(engine=2, row_tiles=2, cols_per_tile=128, waves_per_wg=4, workgroups=1, k_splits=splits)
        assert mnb.mnb_plan_check(20, 4096, 100, q) == 9, splits
    q = mnb.mnb_plan(engine=2, row_tiles=8, cols_per_tile=256, waves_per_wg=8, workgroups=1, k_splits=2)
    assert mnb.mnb_plan_check(20, 4096, 100, q) == 9
    q = mnb.mnb_plan(engine=2, row_tiles=1, cols_per_tile=16, waves_per_wg=8, workgroups=1, k_splits=4)
    assert mnb.mnb_plan_check(20, 4096, 100, q) == 0                 # with the K split over waves too
    for m in (1, 4):
        d = mnb.mnb_plan_default(m, 4096, 4096, 256, 0)
        d.k_splits = 2
        assert mnb.mnb_plan_check(m, 4096, 4096, d) == 9
    # 32-bit activation offsets within a workgroup's rows: 64 * row_tiles * K
    # bytes at most 2^32 - 16.
    big = 1 << 24
    for rt, want in ((4, 9), (2, 0), (1, 0)):
        q = mnb.mnb_plan(engine=2, row_tiles=rt, cols_per_tile=128, waves_per_wg=4, workgroups=1)
        assert mnb.mnb_plan_check(1000, big, 100, q) == want
    p = mnb.mnb_plan_default(1000, big, 100000, 256, 0)   # four row tiles would overflow a resource
    assert p.engine == 2 and p.row_tiles <= 2
    # Decode plans take any m (launches of 8 rows) when they fit 8 rows.
    d = mnb.mnb_plan(lanes_per_col=64, blocks_per_lane=1, cols_per_tile=1, workgroups=1)
    assert mnb.mnb_plan_check(8, 4096, 100, d) == 0
    assert mnb.mnb_plan_check(9, 4096, 100, d) == 0
    d2 = mnb.mnb_plan(lanes_per_col=64, blocks_per_lane=2, cols_per_tile=4, workgroups=1)
    assert mnb.mnb_plan_check(4, 4096, 100, d2) == 0
    assert mnb.mnb_plan_check(9, 4096, 100, d2) == 9           # 8 rows x 2 blocks > 8
    e1 = mnb.mnb_plan(engine=1, cols_per_tile=16, waves_per_wg=4, workgroups=1)
    assert mnb.mnb_plan_check(4, 4096, 100, e1) == 9            # no engine 1
    e3 = mnb.mnb_plan(engine=3, waves_per_wg=7, blocks_per_lane=4, cols_per_tile=8, workgroups=1)
    assert mnb.mnb_plan_check(4, 14336, 100, e3) == 0
    assert mnb.mnb_plan_check(40, 14336, 100, e3) == 9         # 8 rows: registers
    # Activations through LDS: engine 3 only, 0 or 1.
    for m in (1, 4, 8):
        e3 = mnb.mnb_plan(engine=3, waves_per_wg=7, blocks_per_lane=4, cols_per_tile=4, workgroups=1, a_via_lds=1)
        assert mnb.mnb_plan_check(m, 14336, 100, e3) == 0
    e3.a_via_lds = 2
    assert mnb.mnb_plan_check(4, 14336, 100, e3) == 9
    d.a_via_lds = 1
    assert mnb.mnb_plan_check(8, 4096, 100, d) == 9
    q = mnb.mnb_plan(engine=2, row_tiles=1, cols_per_tile=128, waves_per_wg=4, workgroups=1, a_via_lds=1)
    assert mnb.mnb_plan_check(40, 4096, 100, q) == 9


def test_summation_order_does_not_depend_on_n_or_device():
    """Up to 8 rows, the engine is a function of (m, K) (the prefill tiles
    only where the decode lane split would need K in chunks at two or more
    rows), and the decode lane split (which fixes the fp32 summation order
    of a column) depends only on (m, K): the same inputs give the same bits
    for any N and on any compute-unit count."""
    for m in range(1, 9):
        for K in (32, 1024, 4096, 14336, 32768, 65536, 131072):
            plans = [mnb.mnb_plan_default(m, K, N, cus, occ)
                     for N in (1, 1000, 151936) for cus in (1, 256, 304) for occ in (0, 1, 5)]
            engines = {p.engine for p in plans}
            assert engines == {2} or 2 not in engines, (m, K, engines)
            if engines == {2}:
                continue
            splits = {(p.engine, p.lanes_per_col, p.waves_per_wg, p.blocks_per_lane, p.k_chunks) for p in plans}
            assert len(splits) == 1, (m, K, splits)


@pytest.mark.parametrize("fields", [
    dict(lanes_per_col=8), dict(lanes_per_col=96), dict(lanes_per_col=576),
    dict(blocks_per_lane=3), dict(blocks_per_lane=16), dict(cols_per_tile=16),
    dict(workgroups=0), dict(blocks_per_lane=8, cols_per_tile=2),
])
def test_plan_check_rejects(fields):
    base = dict(lanes_per_col=64, blocks_per_lane=1, cols_per_tile=1, workgroups=1)
    base.update(fields)
    p = mnb.mnb_plan(**base)
    assert mnb.mnb_plan_check(1, 4096, 100, p) == 9


def test_default_plan_shapes():
    """The tuned plan shapes for the measured workloads."""
    p = mnb.mnb_plan_default(1, 4096, 151936, 256, 6)
    assert (p.lanes_per_col, p.blocks_per_lane, p.cols_per_tile, p.interleave) == (64, 2, 2, 1)
    assert p.workgroups == 15 * 256             # ~5 tiles per group, whole rounds of CUs
    p = mnb.mnb_plan_default(1, 4096, 28672, 256, 6)
    assert p.workgroups == 6 * 256 // 2         # about five tiles per group, >= half a generation
    # Two or more rows: the 4x4x4 MFMA kernel, eight waves for the 14336-long
    # K (four of four blocks per lane group and four of three), four waves of
    # two for 4096; four columns per tile; whole workgroups per CU, about
    # 12 * K/4096 tiles each within one resident generation (the grids
    # measured fastest or within 7% of it).
    for m, K, N, occ, shape in ((2, 14336, 4096, 1, (8, 4, 4, 256)), (8, 14336, 4096, 1, (8, 4, 4, 256)),
                                (4, 4096, 28672, 4, (4, 2, 4, 768)), (8, 4096, 151936, 4, (4, 2, 4, 1024)),
                                (8, 4096, 6144, 4, (4, 2, 4, 256)), (4, 8192, 8192, 3, (4, 4, 4, 256)),
                                (4, 4096, 14336, 4, (4, 2, 4, 512)),
                                # K = 2048: two waves of two blocks up to four rows, in
                                # multiples of four workgroups per CU; four waves of one
                                # from five rows
                                (2, 2048, 28672, 10, (2, 2, 4, 1024)), (4, 2048, 151936, 10, (2, 2, 4, 2048)),
                                (3, 2048, 8192, 10, (2, 2, 4, 1024)), (8, 2048, 28672, 7, (4, 1, 4, 1280)),
                                # K = 5120 and 6144: five and six waves of two blocks
                                (4, 5120, 4096, 3, (5, 2, 4, 256)), (8, 6144, 14336, 2, (6, 2, 4, 256))):
        p = mnb.mnb_plan_default(m, K, N, 256, occ)
        assert p.engine == 3
        assert (p.waves_per_wg, p.blocks_per_lane, p.cols_per_tile, p.workgroups) == shape
    # Activations through LDS from three rows up where K or N exceeds 8192.
    for m, K, N, via in ((2, 14336, 4096, 0), (3, 14336, 4096, 1), (8, 14336, 4096, 1), (4, 4096, 28672, 1),
                         (8, 4096, 151936, 1), (6, 8192, 8192, 0), (8, 4096, 6144, 0), (5, 4096, 4096, 0),
                         (2, 4096, 151936, 0), (1, 4096, 151936, 0)):
        assert mnb.mnb_plan_default(m, K, N, 256, 2).a_via_lds == via, (m, K, N)


def test_plan_check_rows_limit():
    p = mnb.mnb_plan(lanes_per_col=64, blocks_per_lane=2, cols_per_tile=4, workgroups=1)
    assert mnb.mnb_plan_check(4, 4096, 100, p) == 0
    p = mnb.mnb_plan(lanes_per_col=64, blocks_per_lane=2, cols_per_tile=4, workgroups=1)
    assert mnb.mnb_plan_check(5, 4096, 100, p) == 9


@pytest.mark.parametrize("args,status", [
    (dict(src_layout=2), 10), (dict(dst_layout=-1), 10), (dict(K=48), 2), (dict(K=-32), 2),
    (dict(N=-1), 2), (dict(src=0), 1), (dict(dst=0), 1), (dict(src=FAKE + 8), 5),
    (dict(dst=FAKE * 3 + 4), 5), (dict(dst=FAKE + 64), 8), (dict(K=1 << 25), 2),
])
def test_repack_validation_without_gpu(args, status):
    """mnb_repack_weights rejects bad arguments on the host and launches
    nothing; dst == src (in place) and an empty matrix are accepted."""
    a = dict(src=FAKE, src_layout=0, dst=FAKE * 3, dst_layout=1, N=4, K=64)
    a.update(args)
    L = mnb.lib()
    c0 = mnb.mnb_counters_get()
    st = L.mnb_repack_weights(a["src"], a["src_layout"], a["dst"], a["dst_layout"], a["N"], a["K"], 0)
    assert st == status, mnb.mnb_status_string(st)
    assert mnb.mnb_counters_get() == c0
    assert mnb.mnb_status_string(st) != "unknown status"
    assert L.mnb_repack_weights(0, 0, 0, 1, 0, 64, 0) == 0        # nothing to convert
    assert L.mnb_repack_weights(0, 0, 0, 1, 5, 0, 0) == 0


def test_plan_layouts():
    """The even/odd layout is read by engines 0 and 3 only."""
    for eng, fields in ((0, dict(lanes_per_col=64, blocks_per_lane=2, cols_per_tile=2)),
                        (2, dict(row_tiles=1, cols_per_tile=128, waves_per_wg=4)),
                        (3, dict(waves_per_wg=4, blocks_per_lane=2, cols_per_tile=4))):
        for layout in (0, 1, 2):
            q = mnb.mnb_plan(engine=eng, workgroups=1, b_layout=layout, **fields)
            want = 0 if layout == 0 or (layout == 1 and eng in (0, 3)) else 9
            assert mnb.mnb_plan_check(4, 4096, 100, q) == want, (eng, layout)
    assert mnb.mnb_plan_default(1, 4096, 100, 256, 0).b_layout == mnb.MNB_LAYOUT_NATURAL

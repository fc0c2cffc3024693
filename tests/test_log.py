"""MNB_LOG: each call prints its shape and plan to stderr, one line.

The library's host front end is built here with host-only stand-ins for the
HIP side (tests/sanitize/mnb_hip_stub.cpp: every device entry reports that
no device is present), so a call plans, logs and returns MNB_ERR_HIP
without touching a device, also on a machine that has one."""
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_wise_int4_matmulnbits_amd", "csrc")

CHILD = textwrap.dedent("""
    import ctypes, sys
    sys.path.insert(0, {root!r})
    import block_wise_int4_matmulnbits_amd as mnb
    mnb.LIB_PATH = {lib!r}
    L = mnb.lib()
    # Aligned, disjoint addresses that are never dereferenced: the host-only
    # build reports that no device is present when the launch is queued.
    A, B, S, O = 0x100000, 0x200000, 0x300000, 0x400000
    p = mnb.mnb_plan(lanes_per_col=64, blocks_per_lane=2, cols_per_tile=2, workgroups=7)
    st = L.matmul_nbits_planned(A, mnb.MNB_F16, 3, 4096, 100, B, S, None, 32, O, mnb.MNB_BF16, None,
                                ctypes.byref(p))
    print("status", st)
""")


def _host_lib(tmp_path):
    lib = tmp_path / "libmnb_host.so"
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-O1", "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, "-o", str(lib), os.path.join(CSRC, "mnb_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "mnb_hip_stub.cpp")], check=True)
    return lib


def _call(lib, log):
    env = dict(os.environ)
    env.pop("MNB_LOG", None)
    if log is not None:
        env["MNB_LOG"] = log
    p = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(lib))], env=env,
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    assert "status 7" in p.stdout, p.stdout   # MNB_ERR_HIP: no device behind the stand-ins
    return [line for line in p.stderr.splitlines() if line.startswith("mnb: ")]


def test_mnb_log_prints_the_plan(tmp_path):
    lib = _host_lib(tmp_path)
    lines = _call(lib, "1")
    assert len(lines) == 1, lines
    assert lines[0].startswith("mnb: m=3 K=4096 N=100 a=f16 out=bf16 explicit plan: engine=0 lanes_per_col=64 "
                               "blocks_per_lane=2 cols_per_tile=2 "), lines[0]
    assert "workgroups=7 threads_per_wg=256 k_chunks=1 launches=1" in lines[0], lines[0]
    for off in (None, "0", ""):
        assert _call(lib, off) == [], off

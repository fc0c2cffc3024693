"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/mnb_oracle.c) is rebuilt with -fsanitize=address,
  undefined in a copy of the oracle package and the whole pin suite
  (tests/test_oracle_pins.py) runs against that build.
* The library's host front end (csrc/mnb_api.cpp: argument validation,
  launch planning, counters, status strings) is built the same way with
  host-only stand-ins for the HIP side (tests/sanitize/mnb_hip_stub.cpp),
  and tests/test_abi.py runs against it.

Each run happens in a child process with the sanitizer runtimes preloaded;
any sanitizer report aborts it (halt_on_error), which fails the test.
"""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_wise_int4_matmulnbits_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()


def _env(extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    # Python and its extension modules are not built with the sanitizer:
    # their allocations are not leak-checked, and their globals are not
    # checked for one-definition violations.
    env["ASAN_OPTIONS"] = "detect_leaks=0:detect_odr_violation=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    env.update(extra)
    return env


def _pytest(test_file, env, tmp_path):
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", test_file)]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = p.stdout[-3000:] + p.stderr[-3000:]
    assert p.returncode == 0, out
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, out
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    root = tmp_path / "sanitized"
    dst = root / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__"))
    lib = dst / "libmnb_oracle.so"
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra"] + SAN +
                   ["-o", str(lib), str(dst / "mnb_oracle.c"), "-lm"], check=True)
    os.utime(lib)   # newer than the source: the package loads it as built
    out = _pytest("test_oracle_pins.py", _env({"MNB_ORACLE_ROOT": str(root)}), tmp_path)
    assert "passed" in out


def test_host_front_end_under_asan_ubsan(tmp_path):
    lib = tmp_path / "libmnb_host_sanitized.so"
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra"] + SAN +
                   ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(lib),
                    os.path.join(CSRC, "mnb_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "mnb_hip_stub.cpp")], check=True)
    out = _pytest("test_abi.py", _env({"MNB_HOST_LIB": str(lib)}), tmp_path)
    assert "passed" in out

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (tests/sanitize/oracle_driver.c) and the library's host code --
the fp64 table fit in every mode, the neighbour-map fit and blob validation
(tests/sanitize/host_driver.cpp) -- are compiled with gcc/g++ and both
sanitizers and driven through round trips and through damaged, truncated
and random inputs.  The table blob and the container are parsed from
untrusted bytes, so any out-of-bounds read, overflow or leak there is a bug.
No GPU code is built or run here.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def _run(cmd, exe, tmp_path):
    if shutil.which(cmd[0]) is None:
        pytest.skip(f"{cmd[0]} not available")
    subprocess.run(cmd, check=True, cwd=tmp_path, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], cwd=tmp_path, capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "ok" in r.stdout, out[-4000:]


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
          os.path.join(HERE, "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "skv_oracle.c"),
          "-o", exe, "-lm"], exe, tmp_path)


def test_host_fit_and_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    _run(["g++", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN,
          os.path.join(HERE, "sanitize", "host_driver.cpp"),
          os.path.join(ROOT, "lossless_kv_cache_amd", "csrc", "skv_fit.cpp"), "-o", exe], exe, tmp_path)

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The oracle (oracle/oracle.c), built with gcc and both sanitizers, driven over
  every function and edge-case shapes by tests/sanitize/oracle_check.c.
* The library's host code -- argument validation of every call, launch
  planning up to the first device call, the selection counts, the calibration
  search and the cost-model fit -- built with both sanitizers on the host
  pass only (tests/sanitize/build_abi_check.sh) and driven by
  tests/sanitize/abi_check.c.
Any report is fatal (-fno-sanitize-recover), so a clean run exits 0."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, (cmd[0], r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-fopenmp", os.path.join(SAN, "oracle_check.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4")
    r = _run([exe], env=env)
    assert "0 failed checks" in r.stdout


def test_abi_host_code_under_sanitizers(tmp_path):
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = str(tmp_path / "abi")
    _run(["bash", os.path.join(SAN, "build_abi_check.sh"), out], timeout=900)
    # leak checking stays off: the HIP runtime keeps allocations until exit
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = _run([os.path.join(out, "abi_check")], env=env)
    assert "0 failed checks" in r.stdout

"""AddressSanitizer + UndefinedBehaviorSanitizer on the host code, CPU only
(tests/sanitize): the CPU reference driven over every mode, shape kind and
special input on exactly sized buffers; the C-ABI validation layer of
libnvfp4 on stub launchers with valid, invalid and extreme arguments; and the
reference's own test suite against a sanitizer build of it.  Any report
aborts the program (no recovery), which fails the test."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))
import build as san  # noqa: E402

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")


@pytest.fixture(scope="module")
def programs():
    return san.build()


def _run(cmd, **kw):
    r = subprocess.run(cmd, env=kw.pop("env", ENV), capture_output=True, text=True, **kw)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


def test_oracle_under_sanitizers(programs):
    assert "0 unexpected" in _run([programs[0]])


def test_abi_validation_under_sanitizers(programs):
    out = _run([programs[1]])
    assert "unexpected statuses: 0" in out


def test_oracle_suite_against_sanitizer_build(programs):
    env = dict(ENV, LD_PRELOAD=san.preload(), NVFP4_ORACLE_LIB=san.ORACLE_LIB)
    files = ["test_oracle_formats.py", "test_oracle_quantize.py", "test_oracle_gemm.py",
             "test_oracle_rht.py", "test_oracle_mxfp4.py", "test_scale_ties.py",
             "test_near_points_construction.py", "test_sr_decision_host.py"]
    out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p",
                "no:cacheprovider", *[os.path.join(HERE, f) for f in files]],
               env=env, cwd=os.path.dirname(HERE))
    assert " passed" in out and "failed" not in out

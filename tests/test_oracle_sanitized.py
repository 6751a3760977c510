"""The oracle's C sources under AddressSanitizer and UndefinedBehaviorSanitizer.

A sanitizer build of oracle/gdr_ref.c and oracle/gdr_ref_bwd.c (gcc, host code) runs
the oracle's pin suites in a child process with the sanitizer runtimes preloaded, so an
out-of-bounds access, a use after free or undefined behaviour anywhere the pins reach
in the forward recurrence or its reverse pass stops the run and fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py",
              "tests/test_oracle_invariants.py"]


def _runtime(name):
    path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    from oracle import build

    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = build.build(out=str(tmp_path / "libgdr_ref_san.so"), sanitize=True)
    # the reports go to files: a sanitizer stops the child before pytest prints anything
    log = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", GDR_ORACLE_LIB=lib,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:verify_asan_link_order=0:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}",
               OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *PIN_SUITES]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    reports = "".join(open(os.path.join(tmp_path, f)).read()[:3000]
                      for f in sorted(os.listdir(tmp_path)) if f.startswith("san."))
    assert r.returncode == 0 and not reports, reports + r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout

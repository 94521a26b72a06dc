"""AddressSanitizer and UndefinedBehaviorSanitizer builds (host code only, no
GPU): the oracle driven through every entry point on small seeded inputs
(tests/sanitize/oracle_driver.c, gcc), and the library's host entry points --
argument checks, size limits, workspace layout, the commit step's digests --
(tests/sanitize/host_driver.cpp with sv_api.hip and sv_commit.hip, hipcc, each
-fsanitize= after -Xarch_host so that device code is built without it).  A
sanitizer report fails the run (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    b = run(["gcc", "-std=c11", "-g", "-O1", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-o", exe, os.path.join(HERE, "oracle_driver.c"), "-lm"])
    assert b.returncode == 0, b.stderr
    r = run([exe], env=ENV)
    assert r.returncode == 0 and "rc=0" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_host_entry_points_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "host_driver")
    csrc = os.path.join(ROOT, "token_sampling_amd", "csrc")
    b = run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
             "-I", csrc, "-o", exe, os.path.join(HERE, "host_driver.cpp"),
             os.path.join(csrc, "sv_api.hip"), os.path.join(csrc, "sv_commit.hip")])
    assert b.returncode == 0, b.stderr[-4000:]
    r = run([exe], env=ENV)
    assert r.returncode == 0 and "0 failures" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr

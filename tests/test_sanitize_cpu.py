"""The oracle and the library's host code under AddressSanitizer + UndefinedBehaviorSanitizer.

Both are rebuilt here with the sanitizers (on the host pass only, for the HIP sources) and
driven by small programs beside this file that need no GPU: the oracle over seeded paged
cases and its refusals (`sanitize/oracle_checks.c`); the library's status strings, its
size queries over a sweep of problem shapes and planner options with extreme values, and
every argument check made before a launch (`sanitize/host_checks.cpp`).  A sanitizer
report, or any unexpected status, fails the test."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host pass only (the device code is built as usual)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    return r.returncode, msg


def _check_clean(rc, msg):
    assert "runtime error:" not in msg and "ERROR: AddressSanitizer" not in msg, msg
    assert rc == 0 and "ALL OK" in msg, msg


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    rc, msg = _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "mla_oracle.c"), os.path.join(HERE, "sanitize", "oracle_checks.c"),
                    "-lm", "-o", exe])
    assert rc == 0, msg
    _check_clean(*_run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1")))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_library_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "mla_decode_03_amd", "csrc")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + csrc]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN, *inc]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src).replace(".", "_") + ".o"))
        rc, msg = _run([HIPCC, *flags, "-c", src, "-o", obj])
        assert rc == 0, msg
        return obj

    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    srcs.append(os.path.join(HERE, "sanitize", "host_checks.cpp"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_checks")
    rc, msg = _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, *objs, "-o", exe])
    assert rc == 0, msg
    _check_clean(*_run([exe], env=ENV))

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* ``tests/native/host_checks.cpp`` with the library's packed-sequence index helpers
  (``csrc/seqmath.h``, the same header the kernels include) and the C entry points of
  ``csrc/gdn_api.cpp``, both compiled with the sanitizers on the host side (the kernels' launchers
  come from the built ``libgdn.so``): malformed ``cu_seqlens`` arrays (decreasing, negative, past T,
  extreme values) must give token ranges inside [0, T] and chunk slots inside the workspace, and
  rejected arguments and extreme sizes must be handled without a sanitizer report.
* ``tests/native/oracle_checks.c`` with the C oracle, compiled with gcc and the same sanitizers.

A planted mistake (the clamp of a sequence's end to its start removed) must make the host checks
fail, so the checks are known to bite.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "gated_deltanet_delta_amd", "csrc")
PKG = os.path.join(ROOT, "gated_deltanet_delta_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host side only: device code cannot be built with them
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build_host_checks(tmp_path, include_first=None):
    if not os.path.exists(os.path.join(PKG, "libgdn.so")):
        pytest.skip("libgdn.so is not built")
    out = str(tmp_path / "host_checks")
    inc = ([f"-I{include_first}"] if include_first else []) + [f"-I{ROOT}/include", f"-I{CSRC}"]
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *HOST_SAN, *inc,
           os.path.join(NATIVE, "host_checks.cpp"), os.path.join(CSRC, "gdn_api.cpp"), f"-L{PKG}", "-lgdn",
           f"-Wl,-rpath,{PKG}", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_host_index_math_and_abi_checks_under_sanitizers(tmp_path):
    exe = _build_host_checks(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0 and "host checks passed" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_host_checks_catch_a_planted_clamp_mistake(tmp_path):
    mut = tmp_path / "mutant"
    mut.mkdir()
    src = open(os.path.join(CSRC, "seqmath.h")).read()
    good = "b = b < a ? a : (b > T ? T : b);"
    assert good in src
    (mut / "seqmath.h").write_text(src.replace(good, "b = b > T ? T : b;"))
    exe = _build_host_checks(tmp_path, include_first=str(mut))
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode != 0 and "FAIL" in r.stderr, r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_checks")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(NATIVE, "oracle_checks.c"),
           os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True,
                       env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"), timeout=120)
    assert r.returncode == 0 and "oracle checks passed" in r.stdout, r.stdout + r.stderr

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* libdeepselect's host part (argument checks, split planner, layouts, status
  strings, rejected calls) built host-only with the sanitizers on the host
  pass, linked into tests/host_check.cpp;
* the C oracle with tests/oracle_check.c, built by gcc with the same
  sanitizers and OpenMP;
* the workspace cache (csrc/ds_workspace.hpp) driven from 8 threads with
  fake streams by tests/ws_check.cpp, once under AddressSanitizer and
  UndefinedBehaviorSanitizer and once under ThreadSanitizer.
Each program exits non-zero on a failed expectation; a sanitizer finding
aborts it. The GPU code is not part of these builds."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    return res


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_library_host_code_under_sanitizers(tmp_path):
    obj = str(tmp_path / "ds_host.o")
    exe = str(tmp_path / "host_check")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "--offload-host-only", "-std=c++17", "-O1", "-g",
          "-fno-omit-frame-pointer", *san, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "top_selection_row_amd", "csrc", "deepselect.hip"), "-o", obj])
    # a host-only object refers to the device code's fat binary; no kernel is
    # launched here, so an empty array of that name stands in for it
    nm = shutil.which("nm") or shutil.which("llvm-nm") or "/opt/rocm/llvm/bin/llvm-nm"
    syms = re.findall(r"__hip_fatbin_[0-9a-f]+", _run([nm, obj]).stdout)
    stub = str(tmp_path / "fatbin_stub.cpp")
    with open(stub, "w") as f:
        f.write("".join(f'extern "C" {{ char {sym}[64]; }}\n' for sym in sorted(set(syms))))
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "--offload-host-only", "-std=c++17", "-O1", "-g",
          "-fno-omit-frame-pointer", *san, "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "host_check.cpp"), "-x", "c++", stub, "-x", "none", obj, "-o", exe])
    res = _run([exe], env=SAN_ENV)
    assert "0 failures" in res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fopenmp", os.path.join(ROOT, "oracle", "topk_sort.c"),
          os.path.join(ROOT, "tests", "oracle_check.c"), "-o", exe])
    res = _run([exe], env=SAN_ENV)
    assert "0 failures" in res.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
@pytest.mark.parametrize("san", [["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
                                 ["-fsanitize=thread"]], ids=["asan-ubsan", "tsan"])
def test_workspace_cache_under_threads(tmp_path, san):
    # every call frees a buffer only after synchronising its stream, while
    # holding the lock from the choice of the workspace until its use is queued
    exe = str(tmp_path / "ws_check")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *san, "-pthread",
          os.path.join(ROOT, "tests", "ws_check.cpp"), "-o", exe])
    env = dict(SAN_ENV, TSAN_OPTIONS="halt_on_error=1")
    res = _run([exe], env=env)
    assert "no free of a queued buffer" in res.stdout

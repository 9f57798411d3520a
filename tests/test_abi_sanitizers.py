"""The C ABI layer's host code (csrc/ps_api.hip: validation, overflow-checked
sizing, dispatch) built for the host only with the address and
undefined-behaviour sanitizers, linked with counting stand-ins of the kernel
launchers (tests/abi/stubs.cpp), and driven through every entry point by
tests/abi/driver.cpp (CPU only; no device code is built or run)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_page_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "abi")


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                     else None)


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_abi_host_code_under_sanitizers(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17",
              f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    objs = []
    for src in (os.path.join(CSRC, "ps_api.hip"), os.path.join(HERE, "stubs.cpp"),
                os.path.join(HERE, "driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"]
        subprocess.run([_hipcc(), *lang, *common, *san, "-c", src, "-o", obj], check=True,
                       capture_output=True, text=True)
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    subprocess.run([_hipcc(), "--offload-arch=gfx950", *san, *objs, "-o", exe], check=True,
                   capture_output=True, text=True)
    syms = subprocess.run(["nm", exe], capture_output=True, text=True, check=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms  # both are really built in
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr

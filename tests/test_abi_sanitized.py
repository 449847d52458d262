"""The C ABI's host-side checks built with AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

dsc_api.hip (argument validation, no kernels) is compiled with the host
sanitizers and linked with the library's other objects;
tests/abi_sanitize_driver.c then calls every entry point with arguments that
fail validation before any HIP call, including sizes at the int64 limits.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_abi_checks_under_sanitizers(tmp_path):
    from input_dependent_short_amd import build
    objdir = os.path.join(build.PKG, "_build")
    others = [os.path.join(objdir, os.path.basename(s) + ".o") for s in build.sources()
              if os.path.basename(s) != "dsc_api.hip"]
    if not all(os.path.exists(o) for o in others):
        build.build()
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    obj, lib, exe = str(tmp_path / "dsc_api.o"), str(tmp_path / "libdsc_san.so"), str(tmp_path / "driver")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-O3")] + ["-O1", "-g"]
    subprocess.run([hipcc, *flags, *san, f"-I{os.path.join(ROOT, 'include')}", "-c",
                    os.path.join(build.CSRC, "dsc_api.hip"), "-o", obj], check=True, capture_output=True)
    subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={build.ARCH}", obj, *others, *san, "-o", lib],
                   check=True, capture_output=True)
    subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "abi_sanitize_driver.c"), lib,
                    f"-Wl,-rpath,{tmp_path}", "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi checks ok" in r.stdout
    assert "runtime error" not in r.stderr

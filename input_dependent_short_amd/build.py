"""Build libdsc.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m input_dependent_short_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsc.so")
ARCH = os.environ.get("DSC_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are disabled on purpose for every device pass
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wno-unused-command-line-argument",
]


# Extra flags per source file.  The wide low-rank forward keeps its
# matrix-core results in ordinary VGPRs (measured faster there); the other
# kernels keep the compiler's default register form.
FILE_FLAGS = {
    "lowrank_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with code {res.returncode}: {' '.join(cmd)}")


def build(out: str = LIB, verbose: bool = False, extra: list[str] | None = None, objdir: str | None = None) -> str:
    """Compile every HIP source (in parallel) and link libdsc.so (extra flags
    and a separate object folder build variants of the library)."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = f"-I{os.path.join(ROOT, 'include')}"
    objdir = objdir or os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        per_file = FILE_FLAGS.get(os.path.basename(src), [])
        jobs.append(([hipcc, *compile_flags, *per_file, *(extra or []), inc, "-c", src, "-o", obj], obj))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    _run([hipcc, *FLAGS, *(extra or []), *[o for _, o in jobs], "-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

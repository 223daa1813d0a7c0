"""Compile the HIP library ``libcoda.so`` for gfx950 (in-tree, no JIT cache).

    python -m gemm_epilogue_transformer_amd.build

Every translation unit under ``csrc/`` is compiled with hipcc (in parallel) into
``_build/`` and linked into ``gemm_epilogue_transformer_amd/libcoda.so``.  Packed fp32
VALU instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcoda.so")
ARCH = os.environ.get("CODA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, save_temps: bool = False, defines=(), out: str = LIB,
          build_dir: str = BUILD, host_flags=()) -> str:
    """Compile and link; host_flags (e.g. the tests' host-only sanitizer options, each
    preceded by -Xarch_host) go on every compile and on the link line."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    objs = []

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *host_flags, *(f"-D{d}" for d in defines), "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if save_temps:
            cmd.append("-save-temps=obj")
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                         and "not a recognized feature" not in l)
        if verbose and warn.strip():
            print(warn, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *host_flags, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))

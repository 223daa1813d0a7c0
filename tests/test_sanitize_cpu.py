"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only, no GPU code is
instrumented):

- the library's host code (the C ABI's validation, sizing and launch set-up) built with
  host-side ASan/UBSan, then the ABI validation tests and the binding's checks run against
  it in a child process with the sanitizer runtime preloaded;
- the fp64 oracle built with ASan/UBSan, then the oracle's pins and the checker tests run
  against it in another child process.

Any sanitizer report aborts the child (halt_on_error, no recovery), which fails the test.
Marked slow: it compiles the library a second time (about a minute).
"""

import glob
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = [pytest.mark.slow,
              pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="host sanitizer runs use fake-pointer validation cases: GPU-less hosts only")]

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _clang_runtime(name):
    hits = sorted(glob.glob(f"/opt/rocm/lib/llvm/lib/clang/*/lib/linux/{name}") +
                  glob.glob(f"/opt/rocm/llvm/lib/clang/*/lib/linux/{name}"))
    if not hits:
        pytest.skip(f"{name} not found")
    return hits[-1]


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not p or not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"{name} not found")
    return p


def _run(args, env_extra, cwd=ROOT):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *args],
                       cwd=cwd, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    return tail


def test_abi_host_code_under_asan_ubsan(tmp_path):
    from gemm_epilogue_transformer_amd import build as b

    lib = str(tmp_path / "libcoda_san.so")
    flags = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer")
    b.build(out=lib, build_dir=str(tmp_path / "obj"), host_flags=flags)
    out = _run(["tests/test_abi_cpu.py", "tests/test_binding_cpu.py"],
               {"LD_PRELOAD": _clang_runtime("libclang_rt.asan-x86_64.so"), "CODA_LIB": lib})
    assert "passed" in out


def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liborcl_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                           "-shared", "-fPIC", os.path.join(ROOT, "oracle", "coda_oracle.c"), "-o", lib, "-lm"])
    pre = ":".join([_gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")])
    out = _run(["tests/test_oracle_codecs.py", "tests/test_oracle_chain.py", "tests/test_oracle_textbook.py",
                "tests/test_oracle_mlpin_bwd.py", "tests/test_oracle_chain_bwd.py", "tests/test_oracle_rope.py",
                "tests/test_oracle_cross_entropy.py", "tests/test_harness_cpu.py"],
               {"LD_PRELOAD": pre, "ORC_LIB": lib, "OMP_NUM_THREADS": "4"})
    assert "passed" in out

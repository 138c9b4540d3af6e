"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only, no GPU needed).

* The fp64 oracle (oracle/oracle.c) is built with gcc -fsanitize=address,undefined together
  with tests/sanitize/oracle_check.c, which drives every oracle function over small inputs and
  their edge cases (empty visibility, k above and below n_vis, ties, -1 padding, clipped
  windows, sinks, every dtype).
* The C ABI's argument validation (api.cpp, host code) is built with the same sanitizers on its
  host pass only (the gfx950 device code is compiled without them) and driven from C by
  tests/sanitize/abi_check.c, which also compiles include/dsa.h as C. Every call there fails
  validation before a launch, so nothing runs on a GPU.
"""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "lightning_indexer_top_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
# host-pass-only sanitizer flags for hipcc: each -fsanitize= right after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(HERE, "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle_check: ok" in r.stdout


def _asan_runtime_dir():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return os.path.dirname(hits[0]) if hits else None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm clang")
def test_abi_validation_under_asan_ubsan(tmp_path):
    import importlib.util

    rt = _asan_runtime_dir()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    spec = importlib.util.spec_from_file_location(
        "_dsa_build", os.path.join(ROOT, "lightning_indexer_top_03_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    objs = []
    for src in b.SOURCES:
        if src == "api.cpp":
            continue
        obj = os.path.join(ROOT, "_build", "dsa", os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(
                os.path.join(CSRC, src)):
            os.makedirs(os.path.dirname(obj), exist_ok=True)
            obj = b._compile(src, str(tmp_path))
        objs.append(obj)
    api = str(tmp_path / "api_san.o")
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([HIPCC, *flags, *HOST_SAN, "-c", os.path.join(CSRC, "api.cpp"), "-o", api])
    lib = str(tmp_path / "libdsa_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *HOST_SAN, api,
          *objs, "-o", lib])
    exe = str(tmp_path / "abi_check")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-shared-libsan", "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include"),
          os.path.join(HERE, "abi_check.c"), lib, "-Wl,-rpath," + str(tmp_path),
          "-Wl,-rpath," + rt, "-o", exe])
    import torch

    args = [] if torch.cuda.is_available() else ["--no-gpu"]
    r = _run([exe, *args], env=ENV)
    assert "abi_check: ok" in r.stdout

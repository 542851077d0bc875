"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU work): api.hip is rebuilt with
the sanitizers on its host code, linked with the library's other objects,
and the ABI tests (every rejection path, workspace sizing, exported symbols)
run against that build in a child process with the sanitizer runtime
preloaded.  Any sanitizer report fails the test."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_32_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitized")


def _runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def _build():
    from block_sparse_attention_32_amd import build as Bld
    hipcc = Bld.hipcc()
    objs = os.path.join(ROOT, "_build")
    others = [os.path.join(objs, os.path.basename(s) + ".o") for s in Bld.sources()
              if not s.endswith("api.hip")]
    if not all(os.path.exists(o) for o in others):
        Bld.build(incremental=True)
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "api.hip.o")
    # the sanitizers instrument the host code only (-Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-g"]
    flags = [f for f in Bld.HIPCC_FLAGS if f != "-O3"] + ["-O1"]
    subprocess.run([hipcc, *flags, *san, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o],
                   check=True, capture_output=True, text=True)
    lib = os.path.join(OUT, "libqsa_sanitized.so")
    clang = os.path.join(os.path.dirname(hipcc), "..", "lib", "llvm", "bin", "clang++")
    subprocess.run([clang, "-shared", "-fPIC", "-shared-libsan",
                    "-fsanitize=address,undefined", api_o, *others,
                    "-L/opt/rocm/lib", "-lamdhip64", "-o", lib],
                   check=True, capture_output=True, text=True)
    return lib


def test_abi_validation_clean_under_asan_and_ubsan():
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm")
    try:
        lib = _build()
    except subprocess.CalledProcessError as e:
        pytest.fail(f"sanitized build failed:\n{e.stdout}\n{e.stderr}")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "build is not instrumented"
    env = dict(os.environ, QSA_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout

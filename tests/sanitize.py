"""The CPU test suite against address- and undefined-behaviour-sanitised
builds of the host code: the C-ABI library's host side (argument
validation, workspace layouts, token tiling, the workgroup-trace setting),
the oracle and the input generator.

    python tests/sanitize.py [extra pytest arguments]

builds the three libraries under tests/_san/ with clang's AddressSanitizer
and UndefinedBehaviorSanitizer (any report aborts the run), then runs
``pytest tests -m "not gpu"`` in a child process that loads them in place of
the normal builds (DSA_LIBRARY, DSA_ORACLE_LIBRARY, DSA_SYNTH_LIBRARY) with
the sanitiser runtime preloaded (the library's device code is built as
usual, uninstrumented; the CPU suite makes no GPU call).  Exits with
pytest's status.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "tests", "_san")
LLVM = "/opt/rocm/lib/llvm"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = os.path.join(LLVM, "bin", "clang")


def asan_runtime() -> str:
    found = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not found:
        raise SystemExit("clang's AddressSanitizer runtime was not found under " + LLVM)
    return found[-1]


def build() -> dict:
    os.makedirs(OUT, exist_ok=True)
    libs = {"DSA_LIBRARY": os.path.join(OUT, "libdsa_san.so"),
            "DSA_ORACLE_LIBRARY": os.path.join(OUT, "liboracle_san.so"),
            "DSA_SYNTH_LIBRARY": os.path.join(OUT, "libsynth_san.so")}
    csrc = os.path.join(ROOT, "indexed_sparse_attention_amd", "csrc")
    srcs = [os.path.join(csrc, s) for s in
            ("index_score.hip", "topk.hip", "sparse_mla.hip", "noalloc_ws.hip", "dsa_api.cpp")]
    # host code only, instrumented (each sanitiser flag applies to the host pass alone)
    subprocess.check_call([
        HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
        *srcs, "-o", libs["DSA_LIBRARY"]])
    for name, src in (("DSA_ORACLE_LIBRARY", os.path.join(ROOT, "oracle", "oracle.c")),
                      ("DSA_SYNTH_LIBRARY", os.path.join(ROOT, "synth", "gen.c"))):
        subprocess.check_call([
            CLANG, "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", src, "-o", libs[name], "-lm"])
    return libs


def main(argv) -> int:
    libs = build()
    env = dict(os.environ)
    env.update(libs)
    env["LD_PRELOAD"] = asan_runtime()
    # Python's own allocations are never freed at exit: leak checking is off
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["LD_LIBRARY_PATH"] = os.path.join(LLVM, "lib") + os.pathsep + env.get("LD_LIBRARY_PATH", "")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider", "--ignore", os.path.join(ROOT, "tests", "test_sanitizers.py"), *argv]
    print("sanitised libraries:", ", ".join(f"{k}={v}" for k, v in libs.items()), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

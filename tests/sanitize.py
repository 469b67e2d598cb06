"""Run the CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

    python tests/sanitize.py [extra pytest arguments]

Builds, before anything is preloaded, instrumented copies of the three native
libraries the CPU tests load, under ``_build/sanitize/``:

  * the oracle (``oracle/ssta_oracle.c``) and the input generator
    (``synthetic_inputs/philox_gen.c``), with clang, single-threaded (no
    OpenMP), every undefined-behaviour check fatal;
  * ``libssta.so`` with its host half instrumented (its device code is built
    as usual; the CPU tests never launch it).

It then runs ``pytest -m "not gpu"`` in a child process with clang's ASan
runtime preloaded (its UBSan handlers included) and the loaders pointed at
the instrumented libraries (SSTA_ORACLE_LIB, SSTA_SYNTH_LIB, SSTA_LIB); no
compiler runs under the preload.  The instrumented oracle and generator run
on one thread (they are built without OpenMP); numpy and torch keep their own
threads.  Leak checking is off: the Python interpreter itself holds memory
until exit.  Exits with pytest's status.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
C_FLAGS = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-mfma",
           "-fno-omit-frame-pointer", "-Wno-unknown-pragmas",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def runtime() -> str:
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hits:
        raise SystemExit("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found")
    return hits[0]


def build_c(src: str, name: str) -> str:
    out = os.path.join(OUT, name)
    subprocess.run([CLANG, *C_FLAGS, src, "-o", out, "-lm"], check=True)
    return out


def main() -> int:
    os.makedirs(OUT, exist_ok=True)
    orc = build_c(os.path.join(ROOT, "oracle", "ssta_oracle.c"), "libssta_oracle.so")
    syn = build_c(os.path.join(ROOT, "synthetic_inputs", "philox_gen.c"), "libsynth.so")
    sys.path.insert(0, ROOT)
    from video_dit_block_tile_amd import build as hip_build
    lib = hip_build.build(lib=os.path.join(OUT, "libssta.so"),
                          build_dir=os.path.join(OUT, "obj"),
                          host_flags=["-fsanitize=address", "-fsanitize=undefined",
                                      "-fno-sanitize-recover=undefined",
                                      "-fno-omit-frame-pointer"])
    env = dict(os.environ,
               LD_PRELOAD=runtime(),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               SSTA_ORACLE_LIB=orc, SSTA_SYNTH_LIB=syn, SSTA_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q",
           "-p", "no:cacheprovider", *sys.argv[1:]]
    print("[sanitize] %s" % " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())

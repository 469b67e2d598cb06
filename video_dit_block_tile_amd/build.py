"""Build libssta.so (gfx950) in-tree with hipcc.

Each translation unit is compiled to an object under ``_build/`` and the
objects are linked into ``video_dit_block_tile_amd/libssta.so``.  Packed fp32
VALU instructions are disabled for all device code.  The scoring and tiling
units are compiled without floating-point contraction (their results must not
depend on the compiler's choice to fuse).  The attention unit is compiled with
-fno-honor-nans: its inputs are finite, and IEEE NaN semantics would make
every fmaxf of a matrix-core result pay an extra canonicalising instruction.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssta.so")

ARCH = "gfx950"
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-I", INCLUDE, "-I", CSRC]
SOURCES = {
    "ssta_api.cpp": ["-x", "hip"],
    "k_tile.hip": ["-ffp-contract=off"],
    "k_score.hip": ["-ffp-contract=off"],
    "k_mask.hip": [],
    "k_attn.hip": ["-fno-honor-nans"],
    "k_calib.hip": [],
    "k_attn_bwd.hip": ["-fno-honor-nans"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libssta.so")
    return path


def _host_only(flags) -> list:
    """Each flag for the host compilation only (device code is built as usual)."""
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def _compile(src: str, extra: list, build_dir: str = BUILD, host_flags=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, *_host_only(host_flags), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(jobs: int = 8, lib: str = LIB, build_dir: str = BUILD, host_flags=()) -> str:
    """Compile every HIP source for gfx950 and link libssta.so; returns its path.

    ``lib``, ``build_dir`` and ``host_flags`` (applied to the host compilation
    only, e.g. for an instrumented host build) default to the in-tree library.
    """
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], build_dir, host_flags),
                           SOURCES.items()))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build())

"""Seeded synthetic inputs for the SSTA workloads, shared by the oracle and the GPU path.

This module draws numbers and builds workload presets; it holds no step of the
attention method.  Arrays are returned as bf16 bit patterns (``numpy.uint16``)
with layout ``[batch, heads, T*H*W, head_dim]``, tokens row-major over (t, y, x).

Generator recipe (the C file beside this one implements it):
  * kind 0 ("iid"):    x = noise_std * N(0, 1)
  * kind 1 ("field"):  x = sin(2*pi*(ft*t/T + fy*y/H + fx*x/W) + phi[h, d]) + noise_std * N(0, 1),
    ft, fy, fx ~ U[0.5, 2.0] cycles per grid extent, drawn per (batch, head);
    phi ~ U[0, 2*pi) per (batch, head, channel).
  * Philox4x32-10 counters keyed by (seed, tensor id), tensor id 0/1/2 = Q/K/V.
  * value -> fp32 -> bf16 round-to-nearest-even.
  * Joint sequences (text_len > 0): the clip's tokens are followed by text_len
    text tokens, drawn i.i.d. N(0, 1) with tensor id 16 + (the clip tensor's id),
    so the layout is [batch, heads, T*H*W + text_len, head_dim].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox_gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
# A prebuilt library (e.g. an instrumented build for sanitizer runs) named by
# SSTA_SYNTH_LIB is loaded instead, and build() leaves it alone.
_PREBUILT = os.environ.get("SSTA_SYNTH_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile the generator with gcc into ``libsynth.so`` (next to the source)."""
    global _lib
    if _PREBUILT:
        return _PREBUILT
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _PREBUILT:
            lib = ctypes.CDLL(_PREBUILT)
        else:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
        lib.synth_generate.restype = ctypes.c_int
        lib.synth_generate.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint32,
            ctypes.c_double, ctypes.c_double, ctypes.c_double]
        lib.synth_philox_block.restype = None
        lib.synth_philox_block.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def philox4x32_10(counter, key):
    """One Philox4x32-10 block (exposed for the generator's known-answer test)."""
    lib = _load()
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.synth_philox_block(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


@dataclass(frozen=True)
class Workload:
    """One SSTA workload: geometry, selection parameters and input recipe."""
    name: str
    batch: int
    heads: int
    T: int
    H: int
    W: int
    tile: tuple = (2, 8, 8)
    win: tuple = (1, 1, 1)
    topk: int = 2
    head_dim: int = 128
    kind: int = 1             # 0 = iid Gaussian, 1 = smooth field + noise
    noise_std: float = 0.5
    seed: int = 0
    dup_tiles: tuple = field(default=())   # ((src_tile, dst_tile), ...) copies for exact ties
    text_len: int = 0         # text tokens after the clip's tokens

    @property
    def n_tokens(self) -> int:
        """Clip tokens per (batch, head)."""
        return self.T * self.H * self.W

    @property
    def seq_len(self) -> int:
        """Tokens per (batch, head): the clip's, then the text's."""
        return self.n_tokens + self.text_len

    @property
    def tile_tokens(self) -> int:
        """Tokens per block (128 for 2x8x8, 64 for 4x4x4)."""
        return self.tile[0] * self.tile[1] * self.tile[2]

    @property
    def n_text_blocks(self) -> int:
        return -(-self.text_len // self.tile_tokens)

    @property
    def n_rows(self) -> int:
        """Blocks per (batch, head): clip blocks, then text blocks."""
        return self.n_tiles + self.n_text_blocks

    @property
    def tile_grid(self) -> tuple:
        """Blocks per axis, rounded up: edge blocks of a ragged grid are partial."""
        return tuple(-(-n // t) for n, t in zip((self.T, self.H, self.W), self.tile))

    @property
    def n_tiles(self) -> int:
        a, b, c = self.tile_grid
        return a * b * c

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five measured shapes (latent grids of 480p/720p clips; 2x8x8 = 128-token tiles).
CONFIGS = {
    "tiny": Workload("tiny", 1, 2, 4, 16, 16, topk=2, kind=0, noise_std=1.0, seed=0),
    "480p-short": Workload("480p-short", 1, 16, 6, 32, 56, topk=8, seed=1),
    "480p-5s": Workload("480p-5s", 1, 16, 20, 32, 56, topk=16, seed=2),
    "720p-5s": Workload("720p-5s", 1, 16, 30, 48, 80, topk=32, seed=3),
    "720p-10s": Workload("720p-10s", 1, 16, 60, 48, 80, topk=48, seed=4),
}

# Small cases that exercise what the five shapes do not: a top-k that matters on a
# small grid, window 0, k = 0, exact score ties, batch > 1, odd head count, tile
# grids with odd extents and tile counts that are not multiples of 64.
EXTRA = {
    "grid32-w1-k2": Workload("grid32-w1-k2", 1, 2, 4, 32, 32, tile=(2, 8, 8), win=(1, 1, 1),
                             topk=2, seed=10),
    "grid32-w0-k3": Workload("grid32-w0-k3", 1, 2, 4, 32, 32, win=(0, 0, 0), topk=3, seed=11),
    "grid32-w0-k0": Workload("grid32-w0-k0", 1, 2, 4, 32, 32, win=(0, 0, 0), topk=0, seed=12),
    "dup-ties": Workload("dup-ties", 1, 2, 4, 32, 32, win=(0, 0, 0), topk=3, kind=0,
                         noise_std=1.0, seed=13,
                         dup_tiles=((5, 0), (5, 9), (5, 17), (5, 30), (12, 3), (12, 21))),
    "ragged": Workload("ragged", 2, 3, 6, 24, 40, win=(1, 0, 2), topk=5, seed=14),
    "wide-k": Workload("wide-k", 1, 2, 6, 24, 40, win=(1, 1, 1), topk=100, seed=15),
    # grids the 2x8x8 block does not divide: partial edge blocks on t and y (5x20x24),
    # and on x only (4x16x20)
    "partial": Workload("partial", 1, 2, 5, 20, 24, win=(1, 1, 1), topk=4, seed=16),
    "partial-x": Workload("partial-x", 2, 1, 4, 16, 20, win=(1, 0, 1), topk=3, seed=17),
}

# The real latent grid of a 10 s 720p clip (61 latent frames from 241 frames; 720/16 = 45
# rows): ragged in t and y for the 2x8x8 block.
LATENT = {
    "720p-10s-latent": Workload("720p-10s-latent", 1, 16, 61, 45, 80, topk=48, seed=5),
}

# Joint video + text sequences: clip tokens followed by text tokens (a single-stream
# block's input).  Text lengths: a partial text block (77), two full blocks (256), and a
# ragged grid with a text tail of one full block plus 2 tokens (130).
JOINT = {
    "joint-tiny": Workload("joint-tiny", 1, 2, 4, 16, 16, topk=2, kind=0, noise_std=1.0,
                           seed=20, text_len=77),
    "joint-grid32": Workload("joint-grid32", 1, 2, 4, 32, 32, win=(1, 1, 1), topk=2, seed=21,
                             text_len=256),
    "joint-partial": Workload("joint-partial", 2, 1, 5, 20, 24, win=(1, 0, 1), topk=3,
                              seed=22, text_len=130),
    "720p-10s-text": Workload("720p-10s-text", 1, 16, 60, 48, 80, topk=48, seed=23,
                              text_len=256),
}

# 64-token blocks (4x4x4, the block the pages use as their example): a small grid, a
# ragged grid with a text tail, and the 720p 10 s clip (top-k 96 selects as many tokens
# as top-k 48 of 128-token blocks).
TILE64 = {
    "t64-grid": Workload("t64-grid", 1, 2, 8, 16, 16, tile=(4, 4, 4), win=(1, 1, 1), topk=3,
                         seed=24),
    "t64-partial": Workload("t64-partial", 2, 1, 6, 10, 18, tile=(4, 4, 4), win=(1, 0, 1),
                            topk=4, seed=25, text_len=70),
    "720p-10s-t64": Workload("720p-10s-t64", 1, 16, 60, 48, 80, tile=(4, 4, 4), topk=96,
                             seed=26),
}

# The largest block grid the selection takes (4096 blocks in one head: 16 x 16 x 16).
LIMITS = {
    "max-tiles": Workload("max-tiles", 1, 1, 32, 128, 128, topk=64, seed=27),
}

ALL = {**CONFIGS, **EXTRA, **LATENT, **JOINT, **TILE64, **LIMITS}


def _copy_tiles(x: np.ndarray, wl: Workload) -> None:
    """Overwrite whole tiles with copies of others (tokens and all channels)."""
    tt, th, tw = wl.tile
    _, ny, nx = wl.tile_grid
    xg = x.reshape(x.shape[0], x.shape[1], wl.T, wl.H, wl.W, x.shape[-1])
    for src, dst in wl.dup_tiles:
        st, sy, sx = src // (ny * nx), (src // nx) % ny, src % nx
        dt, dy, dx = dst // (ny * nx), (dst // nx) % ny, dst % nx
        xg[:, :, dt * tt:(dt + 1) * tt, dy * th:(dy + 1) * th, dx * tw:(dx + 1) * tw, :] = \
            xg[:, :, st * tt:(st + 1) * tt, sy * th:(sy + 1) * th, sx * tw:(sx + 1) * tw, :]


def generate(wl: Workload, tensor: int) -> np.ndarray:
    """bf16 bits [batch, heads, N + text_len, head_dim] for tensor 0/1/2 (Q/K/V) of
    workload ``wl`` (other ids: other tensors of the same shape, e.g. 3 for dO)."""
    lib = _load()
    out = np.empty((wl.batch, wl.heads, wl.n_tokens, wl.head_dim), dtype=np.uint16)
    rc = lib.synth_generate(out.ctypes.data, wl.batch, wl.heads, wl.T, wl.H, wl.W, wl.head_dim,
                            wl.kind, wl.seed, tensor, wl.noise_std, 0.5, 2.0)
    if rc != 0:
        raise ValueError("synth_generate rejected workload %r" % (wl,))
    if wl.dup_tiles:
        _copy_tiles(out, wl)
    if wl.text_len == 0:
        return out
    txt = np.empty((wl.batch, wl.heads, wl.text_len, wl.head_dim), dtype=np.uint16)
    rc = lib.synth_generate(txt.ctypes.data, wl.batch, wl.heads, 1, 1, wl.text_len,
                            wl.head_dim, 0, wl.seed, 16 + tensor, 1.0, 0.5, 2.0)
    if rc != 0:
        raise ValueError("synth_generate rejected the text of workload %r" % (wl,))
    return np.concatenate([out, txt], axis=2)


def make_qkv(wl: Workload):
    """(q, k, v) bf16-bit arrays of workload ``wl``."""
    return generate(wl, 0), generate(wl, 1), generate(wl, 2)


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a bit shift, no rounding)."""
    return (x.astype(np.uint32) << 16).view(np.float32)

"""SSTA CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU implementation of the Selective and Sliding
Tile Attention (SSTA) forward, used to check the GPU library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it; the GPU library never does, and this package never imports the GPU library.

The arithmetic lives in ``ssta_oracle.c`` (plain C, built with gcc,
``-ffp-contract=off``); this module only marshals numpy arrays.  Each function
cites the passage it follows:

  [TR]   "HunyuanVideo 1.5 Technical Report" summary page, section
         "SSTA: Selective and Sliding Tile Attention" (attention equation; Steps 1-4).
  [BLOG] "HunyuanVideo-1.5: An 8.3B-Parameter Video Diffusion Model Built for
         Consumer GPUs", section "Under the Hood: SSTA and Muon in Detail"
         (the importance_sampling excerpt).

Readings of the pages that the oracle fixes (each pinned by a test):
  * blocks numbered row-major over the (t, h, w) block grid, tokens row-major inside;
  * block mean = fp32 sum over in-block tokens in ascending order / token count;
  * scores in fp32 with fmaf dot chains in ascending channel order;
  * redundancy averaged over the other n - 1 key blocks;
  * top-k over all key blocks, ties to the lower block id, output ascending;
  * window clipped at the grid edge; window and top-k combined by union;
  * attention from the exact fp32 widening of bf16, fp64 accumulation.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssta_oracle.c")
_LIB = os.path.join(_HERE, "libssta_oracle.so")
# A prebuilt library (e.g. an instrumented build for sanitizer runs) named by
# SSTA_ORACLE_LIB is loaded instead, and build() leaves it alone.
_PREBUILT = os.environ.get("SSTA_ORACLE_LIB")
_lib = None

COMBINE_AND = 1 << 0
TOPK_EXCLUDE_WINDOW = 1 << 1

# [BLOG] lambda_ defaults to 0.9 and the redundancy weight is 1 - lambda_;
# both are applied to fp32 tensors, so they act as the fp32 values below.
DEFAULT_LAMBDA = np.float32(0.9)
DEFAULT_BETA = np.float32(1.0 - 0.9)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``libssta_oracle.so`` next to its source."""
    global _lib
    if _PREBUILT:
        return _PREBUILT
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-mfma", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "head_dim", "T", "H", "W", "tile_t", "tile_h", "tile_w",
                 "text_len")]


def _geom(wl) -> _Geom:
    return _Geom(wl.batch, wl.heads, wl.head_dim, wl.T, wl.H, wl.W, *wl.tile,
                 getattr(wl, "text_len", 0))


def _p(a: np.ndarray):
    return a.ctypes.data


def _load():
    global _lib
    if _lib is None:
        if _PREBUILT:
            lib = ctypes.CDLL(_PREBUILT)
        else:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
        G = ctypes.POINTER(_Geom)
        vp, i32, i64, f32, f64, u32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_float, ctypes.c_double, ctypes.c_uint32)
        sig = {
            "orc_n_tiles": (i64, [G]),
            "orc_n_rows": (i64, [G]),
            "orc_tile_tokens": (i32, [G]),
            "orc_token_to_tile": (None, [G, i64, vp, vp]),
            "orc_tile_to_token": (i64, [G, i64, i32]),
            "orc_permute": (None, [G, vp, vp]),
            "orc_pool": (None, [G, vp, vp]),
            "orc_normalize": (None, [i64, i32, vp, vp]),
            "orc_redundancy": (None, [i64, i64, i32, vp, vp]),
            "orc_scores": (None, [i64, i64, i32, vp, vp, vp, f32, f32, vp]),
            "orc_window": (i32, [G, i32, i32, i32, i64, vp]),
            "orc_topk": (ctypes.c_int, [G, i32, i32, i32, i32, i64, i64, vp, i32, i32, vp]),
            "orc_build_lists": (ctypes.c_int, [G, i32, i32, i32, u32, vp, i32, i32, vp, vp, vp]),
            "orc_attention": (None, [G, f64, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp]),
            "orc_attention_bwd": (None, [G, f64, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, i64,
                                         vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


# ---------------------------------------------------------------- geometry

def n_tiles(wl) -> int:
    """[TR] Step 1: number of 3D blocks."""
    return int(_load().orc_n_tiles(ctypes.byref(_geom(wl))))


def n_rows(wl) -> int:
    """Blocks per (batch, head) of a joint sequence: the clip's n_tiles, then
    ceil(text_len / tile_tokens) text blocks ([BLOG] "Architecture: From Prompt
    to Video": single-stream blocks concatenate text and video tokens)."""
    return int(_load().orc_n_rows(ctypes.byref(_geom(wl))))


def tile_tokens(wl) -> int:
    return int(_load().orc_tile_tokens(ctypes.byref(_geom(wl))))


def token_to_tile(wl, n: int):
    t, r = ctypes.c_int64(), ctypes.c_int32()
    _load().orc_token_to_tile(ctypes.byref(_geom(wl)), n, ctypes.byref(t), ctypes.byref(r))
    return t.value, r.value


def tile_to_token(wl, tile: int, r: int) -> int:
    return int(_load().orc_tile_to_token(ctypes.byref(_geom(wl)), tile, r))


def window(wl, i: int, win=None) -> np.ndarray:
    """[TR] Step 3: the clipped sliding-tile window of block i, ascending ids."""
    wt, wh, ww = wl.win if win is None else win
    out = np.empty(n_tiles(wl), dtype=np.int32)
    c = _load().orc_window(ctypes.byref(_geom(wl)), wt, wh, ww, i, _p(out))
    return out[:c].copy()


def k_eff(wl, topk=None, flags: int = 0) -> int:
    """Width of the per-row top-k output: min(k, candidates)  ([BLOG] clamp)."""
    k = wl.topk if topk is None else topk
    n = n_tiles(wl)
    if flags & TOPK_EXCLUDE_WINDOW:
        wmin = min(len(window(wl, i)) for i in range(n))
        return max(0, min(k, n - wmin))
    return max(0, min(k, n))


def max_kept(wl, topk=None, flags: int = 0) -> int:
    """Row capacity of the kept list: the largest |window| combined with k_eff."""
    n = n_tiles(wl)
    wmax = max(len(window(wl, i)) for i in range(n))
    ke = k_eff(wl, topk, flags)
    if flags & COMBINE_AND:
        return min(wmax, ke)
    return min(n, wmax + ke)


# ---------------------------------------------------------------- steps

def permute(wl, x: np.ndarray) -> np.ndarray:
    """Token-major [B,h,S,D] -> tile-major [B,h,n_rows,tile_tokens,D] (bf16 bits):
    the clip's blocks, then the text's (S = N + text_len; n_rows = n_tiles without text)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty((wl.batch, wl.heads, n_rows(wl), tile_tokens(wl), wl.head_dim), np.uint16)
    _load().orc_permute(ctypes.byref(_geom(wl)), _p(x), _p(out))
    return out


def pool(wl, x: np.ndarray) -> np.ndarray:
    """[TR] Step 2: fp32 block means [B,h,n_tiles,D] of token-major bf16 bits
    (clip blocks only: [BLOG] text masking keeps the text out of scoring)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty((wl.batch, wl.heads, n_tiles(wl), wl.head_dim), np.float32)
    _load().orc_pool(ctypes.byref(_geom(wl)), _p(x), _p(out))
    return out


def normalize(p: np.ndarray) -> np.ndarray:
    """[BLOG] divide each vector by its L2 norm (fp32, fixed order)."""
    p = np.ascontiguousarray(p, dtype=np.float32)
    out = np.empty_like(p)
    _load().orc_normalize(p.size // p.shape[-1], p.shape[-1], _p(p), _p(out))
    return out


def redundancy(khat: np.ndarray) -> np.ndarray:
    """[TR] Score_r / [BLOG] mean redundancy, shape [..., n] from khat [..., n, D]."""
    khat = np.ascontiguousarray(khat, dtype=np.float32)
    n, D = khat.shape[-2], khat.shape[-1]
    bh = khat.size // (n * D)
    out = np.empty(khat.shape[:-1], np.float32)
    _load().orc_redundancy(bh, n, D, _p(khat), _p(out))
    return out


def scores(qhat, khat, red, lambda_=DEFAULT_LAMBDA, beta=DEFAULT_BETA) -> np.ndarray:
    """[TR] Score_i = lambda * Score_s - beta * Score_r, shape [..., n, n]."""
    qhat = np.ascontiguousarray(qhat, dtype=np.float32)
    khat = np.ascontiguousarray(khat, dtype=np.float32)
    red = np.ascontiguousarray(red, dtype=np.float32)
    n, D = khat.shape[-2], khat.shape[-1]
    bh = khat.size // (n * D)
    out = np.empty(khat.shape[:-1] + (n,), np.float32)
    _load().orc_scores(bh, n, D, _p(qhat), _p(khat), _p(red), float(lambda_), float(beta),
                       _p(out))
    return out


def topk(wl, sc: np.ndarray, topk=None, flags: int = 0) -> np.ndarray:
    """[TR] Topk / [BLOG] top-k: ascending block ids [B,h,n,k_eff], -1 padded."""
    k = wl.topk if topk is None else topk
    sc = np.ascontiguousarray(sc, dtype=np.float32)
    n = sc.shape[-1]
    ko = k_eff(wl, k, flags)
    out = np.empty(sc.shape[:-1] + (ko,), np.int32)
    rc = _load().orc_topk(ctypes.byref(_geom(wl)), *wl.win,
                          1 if flags & TOPK_EXCLUDE_WINDOW else 0,
                          sc.size // (n * n), n, _p(sc), k, ko, _p(out))
    if rc != 0:
        raise RuntimeError("orc_topk failed")
    return out


def build_lists(wl, topk_idx: np.ndarray, flags: int = 0, topk=None):
    """[TR] Step 4 mask combination -> (kv_idx [B,h,n,max_kept], kv_cnt [B,h,n], bitmask)."""
    n = n_tiles(wl)
    mk = max_kept(wl, topk, flags)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    ks = topk_idx.shape[-1]
    kv_idx = np.empty((wl.batch, wl.heads, n, mk), np.int32)
    kv_cnt = np.empty((wl.batch, wl.heads, n), np.int32)
    bitmask = np.empty((wl.batch, wl.heads, n, (n + 31) // 32), np.uint32)
    rc = _load().orc_build_lists(ctypes.byref(_geom(wl)), *wl.win, flags, _p(topk_idx), ks, mk,
                                 _p(kv_idx), _p(kv_cnt), _p(bitmask))
    if rc != 0:
        raise RuntimeError("orc_build_lists: a row exceeds max_kept")
    return kv_idx, kv_cnt, bitmask


def default_scale(wl) -> float:
    """[TR] attention equation: 1/sqrt(d_k), as the fp32 value the library receives."""
    return float(np.float32(1.0 / math.sqrt(wl.head_dim)))


def attention(wl, q, k, v, kv_idx, kv_cnt, rows=None, scale=None):
    """[TR] Step 4: block-sparse softmax attention over the kept blocks.

    ``rows``: flat row ids (b*heads + h)*n_rows + i to compute (default: all);
    on a joint sequence rows i >= n_tiles are text query blocks, every clip row
    also keeps every text block and a text row keeps every block.
    Returns (o [len(rows), tile_tokens, D] fp64, lse [len(rows), tile_tokens] fp64),
    rows of o in in-tile token order.
    """
    n = n_rows(wl)
    R = tile_tokens(wl)
    if rows is None:
        rows = np.arange(wl.batch * wl.heads * n, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    q, k, v = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v))
    kv_idx = np.ascontiguousarray(kv_idx, dtype=np.int32)
    kv_cnt = np.ascontiguousarray(kv_cnt, dtype=np.int32)
    mk = kv_idx.shape[-1]
    o = np.empty((rows.size, R, wl.head_dim), np.float64)
    lse = np.empty((rows.size, R), np.float64)
    sc = default_scale(wl) if scale is None else float(scale)
    _load().orc_attention(ctypes.byref(_geom(wl)), sc, _p(q), _p(k), _p(v), _p(kv_idx),
                          _p(kv_cnt), mk, rows.size, _p(rows), _p(o), _p(lse))
    return o, lse


def attention_bwd(wl, q, k, v, dout, kv_idx, kv_cnt, q_rows=None, k_rows=None, scale=None):
    """Gradients of Step 4's block-sparse attention with the kept lists held
    fixed ([TR] section "SSTA: Selective and Sliding Tile Attention": the
    attention equation, Step 4 and the paragraph on integrating SSTA during
    distillation training).

    ``q_rows``: flat query-block rows (b*heads + h)*n_rows + i whose dq is
    wanted; ``k_rows``: key-block rows whose dk, dv are wanted (defaults: all).
    Returns (dq [len(q_rows), R, D], dk [len(k_rows), R, D], dv [len(k_rows), R, D])
    in fp64, rows in in-block token order.
    """
    n = n_rows(wl)
    R = tile_tokens(wl)
    allrows = np.arange(wl.batch * wl.heads * n, dtype=np.int64)
    q_rows = allrows if q_rows is None else np.ascontiguousarray(q_rows, dtype=np.int64)
    k_rows = allrows if k_rows is None else np.ascontiguousarray(k_rows, dtype=np.int64)
    q, k, v, dout = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v, dout))
    kv_idx = np.ascontiguousarray(kv_idx, dtype=np.int32)
    kv_cnt = np.ascontiguousarray(kv_cnt, dtype=np.int32)
    mk = kv_idx.shape[-1]
    D = wl.head_dim
    dq = np.empty((q_rows.size, R, D), np.float64)
    dk = np.empty((k_rows.size, R, D), np.float64)
    dv = np.empty((k_rows.size, R, D), np.float64)
    sc = default_scale(wl) if scale is None else float(scale)
    _load().orc_attention_bwd(ctypes.byref(_geom(wl)), sc, _p(q), _p(k), _p(v), _p(dout),
                              _p(kv_idx), _p(kv_cnt), mk, q_rows.size, _p(q_rows), _p(dq),
                              k_rows.size, _p(k_rows), _p(dk), _p(dv))
    return dq, dk, dv


def select(wl, q, k, flags: int = 0, topk=None, lambda_=DEFAULT_LAMBDA, beta=DEFAULT_BETA):
    """Steps 1-4 up to the kept lists; returns a dict of every intermediate."""
    qp, kp = pool(wl, q), pool(wl, k)
    qh, kh = normalize(qp), normalize(kp)
    red = redundancy(kh)
    sc = scores(qh, kh, red, lambda_, beta)
    tk = topk_fn(wl, sc, topk, flags)
    kv_idx, kv_cnt, bitmask = build_lists(wl, tk, flags, topk)
    return dict(q_pooled=qp, k_pooled=kp, q_hat=qh, k_hat=kh, red=red, scores=sc, topk=tk,
                kv_idx=kv_idx, kv_cnt=kv_cnt, bitmask=bitmask)


topk_fn = topk


def forward(wl, q, k, v, rows=None, flags: int = 0, scale=None):
    """The whole SSTA forward; attention only for ``rows`` (default all)."""
    out = select(wl, q, k, flags)
    o, lse = attention(wl, q, k, v, out["kv_idx"], out["kv_cnt"], rows, scale)
    out.update(o=o, lse=lse)
    return out

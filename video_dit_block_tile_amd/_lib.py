"""ctypes binding of libssta.so: the C ABI of include/ssta.h, one Python
function per entry point with the same name.

Marshalling only: tensors become device pointers, the stream defaults to
PyTorch's current HIP stream, and a non-zero status raises ``SstaError``.
Shapes, dtypes and contiguity are checked here because the C ABI receives
bare pointers and cannot.  Every step of the computation runs in the HIP
kernels; there is no fallback when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

# SSTA_LIB may name another build of the same library (e.g. one with an
# instrumented host half for sanitizer runs).
_LIB_PATH = os.environ.get("SSTA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                       "libssta.so")

SSTA_OK = 0
STATUS_NAMES = {0: "SSTA_OK", -1: "SSTA_ERR_ARG", -2: "SSTA_ERR_SHAPE", -3: "SSTA_ERR_ALIGN",
                -4: "SSTA_ERR_NO_DEVICE", -5: "SSTA_ERR_ARCH", -6: "SSTA_ERR_HIP",
                -7: "SSTA_ERR_WORKSPACE"}
COMBINE_AND = 1 << 0
TOPK_EXCLUDE_WINDOW = 1 << 1
LAYOUT_TOKEN_MAJOR = 0
LAYOUT_DIM_MAJOR = 1

# Every function that libssta.so exports, with its ctypes signature.
_vp, _i32, _i64, _u32, _f = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                             ctypes.c_float)


class SstaGeom(ctypes.Structure):
    """ssta_geom_t"""
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "head_dim", "T", "H", "W", "tile_t", "tile_h", "tile_w",
                 "text_len")]

    @property
    def n_tokens(self) -> int:
        """Clip tokens per (batch, head)."""
        return self.T * self.H * self.W

    @property
    def seq_len(self) -> int:
        """Tokens per (batch, head) of the token-major tensors: the clip's, then the text's."""
        return self.n_tokens + self.text_len

    @property
    def n_rows(self) -> int:
        """Blocks per (batch, head): the clip's n_tiles, then the text's blocks of tile_tokens."""
        return self.n_tiles + -(-self.text_len // self.tile_tokens)

    @property
    def n_tiles(self) -> int:
        """Blocks per (batch, head); each axis rounds up (ragged grids have partial edge blocks)."""
        return (-(-self.T // self.tile_t)) * (-(-self.H // self.tile_h)) * (-(-self.W // self.tile_w))

    @property
    def tile_tokens(self) -> int:
        return self.tile_t * self.tile_h * self.tile_w


class SstaParams(ctypes.Structure):
    """ssta_params_t"""
    _fields_ = [("win_t", _i32), ("win_h", _i32), ("win_w", _i32), ("topk", _i32),
                ("lambda_", _f), ("beta", _f), ("scale", _f), ("flags", _u32)]


_G = ctypes.POINTER(SstaGeom)
_P = ctypes.POINTER(SstaParams)
SIGNATURES = {
    "ssta_block_rows": (_i64, [_G]),
    "ssta_tile_pool": (ctypes.c_int, [_G, _vp, _vp, _i32, _vp, _vp]),
    "ssta_tile_unpermute": (ctypes.c_int, [_G, _vp, _vp, _vp]),
    "ssta_topk_width": (_i32, [_G, _P]),
    "ssta_max_kept": (_i32, [_G, _P]),
    "ssta_workspace_bytes": (_i64, [_G, _P]),
    "ssta_score_select": (ctypes.c_int, [_G, _P, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "ssta_score_select_noalloc": (ctypes.c_int, [_G, _P, _vp, _vp, _vp, _vp]),
    "ssta_scores": (ctypes.c_int, [_G, _P, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "ssta_build_mask": (ctypes.c_int, [_G, _P, _vp, _vp, _vp, _vp, _vp]),
    "ssta_attention_fwd": (ctypes.c_int, [_G, _P, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "ssta_attention_fwd_tokens": (ctypes.c_int,
                                  [_G, _P, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "ssta_calibrate_mfma": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp]),
    "ssta_attention_bwd_workspace_bytes": (_i64, [_G]),
    "ssta_attention_bwd": (ctypes.c_int, [_G, _P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                          _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "ssta_default_params": (ctypes.c_int, [_P, _i32]),
    "ssta_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssta_last_hip_error": (ctypes.c_int, []),
}

_lib = None


class SstaError(RuntimeError):
    def __init__(self, name: str, status: int):
        lib = load()
        text = lib.ssta_status_string(status).decode()
        extra = ""
        if status == -6:
            extra = " (hipError %d)" % lib.ssta_last_hip_error()
        super().__init__("%s failed: %s [%s]%s" % (name, STATUS_NAMES.get(status, status), text,
                                                   extra))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libssta.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libssta.so is not built (%s): run __graft_entry__.build() or "
                               "python video_dit_block_tile_amd/build.py" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


# ------------------------------------------------------------------ helpers

def make_geom(batch, heads, T, H, W, tile=(2, 8, 8), head_dim=128, text_len=0) -> SstaGeom:
    return SstaGeom(batch, heads, head_dim, T, H, W, *tile, text_len)


def make_params(win=(1, 1, 1), topk=0, lambda_=None, beta=None, scale=None, flags=0,
                head_dim=128) -> SstaParams:
    """ssta_default_params (the pages' lambda, redundancy weight and 1/sqrt(d)
    scale, from the library) with the given fields overridden."""
    p = SstaParams()
    _call("ssta_default_params", ctypes.byref(p), head_dim)
    p.win_t, p.win_h, p.win_w = win
    p.topk = topk
    p.flags = flags
    if lambda_ is not None:
        p.lambda_ = lambda_
    if beta is not None:
        p.beta = beta
    if scale is not None:
        p.scale = scale
    return p


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _expect(name, t, shape, dtype, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor, got %s" % (name, t.device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _call(name, *args):
    rc = getattr(load(), name)(*args)
    if rc != SSTA_OK:
        raise SstaError(name, rc)


def _tiled_shape(g):
    """Tile-major copies hold the clip's blocks, then the text's."""
    return (g.batch, g.heads, g.n_rows, g.tile_tokens, g.head_dim)


def _kept_lists(g, kv_idx, kv_cnt) -> int:
    """Checks the kept lists and returns their row stride max_kept (0: dense,
    both None)."""
    if kv_cnt is None:
        if kv_idx is not None:
            raise ValueError("dense attention takes neither kv_idx nor kv_cnt")
        return 0
    if not isinstance(kv_idx, torch.Tensor) or kv_idx.dim() != 4:
        raise ValueError("kv_idx must be an int32 [B, h, n_tiles, max_kept] tensor with kv_cnt")
    _expect("kv_cnt", kv_cnt, (g.batch, g.heads, g.n_tiles), torch.int32)
    mk = kv_idx.shape[-1]
    _expect("kv_idx", kv_idx, (g.batch, g.heads, g.n_tiles, mk), torch.int32)
    return mk


def _workspace(workspace) -> int:
    """Checks a device byte buffer and returns its size."""
    if not isinstance(workspace, torch.Tensor):
        raise ValueError("workspace must be a uint8 device tensor")
    _expect("workspace", workspace, (workspace.numel(),), torch.uint8)
    return workspace.numel()


# ------------------------------------------------------------------ entry points

def ssta_block_rows(g: SstaGeom) -> int:
    """Blocks per (batch, head): clip blocks, then text blocks."""
    v = load().ssta_block_rows(ctypes.byref(g))
    if v < 0:
        raise SstaError("ssta_block_rows", v)
    return v


def ssta_topk_width(g: SstaGeom, p: SstaParams) -> int:
    v = load().ssta_topk_width(ctypes.byref(g), ctypes.byref(p))
    if v < 0:
        raise SstaError("ssta_topk_width", v)
    return v


def ssta_max_kept(g: SstaGeom, p: SstaParams) -> int:
    v = load().ssta_max_kept(ctypes.byref(g), ctypes.byref(p))
    if v < 0:
        raise SstaError("ssta_max_kept", v)
    return v


def ssta_workspace_bytes(g: SstaGeom, p: SstaParams) -> int:
    v = load().ssta_workspace_bytes(ctypes.byref(g), ctypes.byref(p))
    if v < 0:
        raise SstaError("ssta_workspace_bytes", v)
    return v


def ssta_tile_pool(g: SstaGeom, x, x_tiled=None, layout=LAYOUT_TOKEN_MAJOR, pooled=None,
                   stream=None):
    _expect("x", x, (g.batch, g.heads, g.seq_len, g.head_dim), torch.bfloat16)
    shp = _tiled_shape(g)
    if layout == LAYOUT_DIM_MAJOR:
        shp = (g.batch, g.heads, g.n_rows, g.head_dim, g.tile_tokens)
    _expect("x_tiled", x_tiled, shp, torch.bfloat16, allow_none=True)
    _expect("pooled", pooled, (g.batch, g.heads, g.n_tiles, g.head_dim), torch.float32,
            allow_none=True)
    _call("ssta_tile_pool", ctypes.byref(g), _ptr(x), _ptr(x_tiled), layout, _ptr(pooled),
          _stream(stream))


def ssta_tile_unpermute(g: SstaGeom, x_tiled, x, stream=None):
    _expect("x_tiled", x_tiled, _tiled_shape(g), torch.bfloat16)
    _expect("x", x, (g.batch, g.heads, g.seq_len, g.head_dim), torch.bfloat16)
    _call("ssta_tile_unpermute", ctypes.byref(g), _ptr(x_tiled), _ptr(x), _stream(stream))


def ssta_score_select(g: SstaGeom, p: SstaParams, q_pooled, k_pooled, topk_idx, workspace,
                      stream=None):
    pshape = (g.batch, g.heads, g.n_tiles, g.head_dim)
    _expect("q_pooled", q_pooled, pshape, torch.float32)
    _expect("k_pooled", k_pooled, pshape, torch.float32)
    _expect("topk_idx", topk_idx, (g.batch, g.heads, g.n_tiles, ssta_topk_width(g, p)),
            torch.int32)
    ws_bytes = _workspace(workspace)
    _call("ssta_score_select", ctypes.byref(g), ctypes.byref(p), _ptr(q_pooled), _ptr(k_pooled),
          _ptr(topk_idx), _ptr(workspace), ws_bytes, _stream(stream))


def ssta_score_select_noalloc(g: SstaGeom, p: SstaParams, q_pooled, k_pooled, topk_idx,
                              stream=None):
    pshape = (g.batch, g.heads, g.n_tiles, g.head_dim)
    _expect("q_pooled", q_pooled, pshape, torch.float32)
    _expect("k_pooled", k_pooled, pshape, torch.float32)
    _expect("topk_idx", topk_idx, (g.batch, g.heads, g.n_tiles, ssta_topk_width(g, p)),
            torch.int32)
    _call("ssta_score_select_noalloc", ctypes.byref(g), ctypes.byref(p), _ptr(q_pooled),
          _ptr(k_pooled), _ptr(topk_idx), _stream(stream))


def ssta_scores(g: SstaGeom, p: SstaParams, q_pooled, k_pooled, scores, red, workspace,
                stream=None):
    pshape = (g.batch, g.heads, g.n_tiles, g.head_dim)
    _expect("q_pooled", q_pooled, pshape, torch.float32)
    _expect("k_pooled", k_pooled, pshape, torch.float32)
    _expect("scores", scores, (g.batch, g.heads, g.n_tiles, g.n_tiles), torch.float32)
    _expect("red", red, (g.batch, g.heads, g.n_tiles), torch.float32, allow_none=True)
    ws_bytes = _workspace(workspace)
    _call("ssta_scores", ctypes.byref(g), ctypes.byref(p), _ptr(q_pooled), _ptr(k_pooled),
          _ptr(scores), _ptr(red), _ptr(workspace), ws_bytes, _stream(stream))


def ssta_build_mask(g: SstaGeom, p: SstaParams, topk_idx, kv_idx, kv_cnt, bitmask=None,
                    stream=None):
    n = g.n_tiles
    _expect("topk_idx", topk_idx, (g.batch, g.heads, n, ssta_topk_width(g, p)), torch.int32)
    _expect("kv_idx", kv_idx, (g.batch, g.heads, n, ssta_max_kept(g, p)), torch.int32)
    _expect("kv_cnt", kv_cnt, (g.batch, g.heads, n), torch.int32)
    _expect("bitmask", bitmask, (g.batch, g.heads, n, (n + 31) // 32), torch.int32,
            allow_none=True)
    _call("ssta_build_mask", ctypes.byref(g), ctypes.byref(p), _ptr(topk_idx), _ptr(kv_idx),
          _ptr(kv_cnt), _ptr(bitmask), _stream(stream))


def ssta_attention_fwd(g: SstaGeom, p: SstaParams, q_t, k_t, v_t, kv_idx, kv_cnt, o_t, lse=None,
                       stream=None):
    """kv_idx = kv_cnt = None runs dense attention (every block kept)."""
    _expect("q_t", q_t, _tiled_shape(g), torch.bfloat16)
    _expect("k_t", k_t, _tiled_shape(g), torch.bfloat16)
    _expect("v_t", v_t, (g.batch, g.heads, g.n_rows, g.head_dim, g.tile_tokens),
            torch.bfloat16)
    _expect("o_t", o_t, _tiled_shape(g), torch.bfloat16)
    _expect("lse", lse, (g.batch, g.heads, g.n_rows, g.tile_tokens), torch.float32,
            allow_none=True)
    mk = _kept_lists(g, kv_idx, kv_cnt)
    _call("ssta_attention_fwd", ctypes.byref(g), ctypes.byref(p), _ptr(q_t), _ptr(k_t), _ptr(v_t),
          _ptr(kv_idx), _ptr(kv_cnt), mk, _ptr(o_t), _ptr(lse), _stream(stream))


def ssta_attention_fwd_tokens(g: SstaGeom, p: SstaParams, q, k, v, kv_idx, kv_cnt, o,
                              lse=None, stream=None):
    """Attention with token-major q, k, v and o (block gathers and output
    scatter inside the kernel)."""
    tok = (g.batch, g.heads, g.seq_len, g.head_dim)
    _expect("q", q, tok, torch.bfloat16)
    _expect("k", k, tok, torch.bfloat16)
    _expect("v", v, tok, torch.bfloat16)
    _expect("o", o, tok, torch.bfloat16)
    _expect("lse", lse, (g.batch, g.heads, g.n_rows, g.tile_tokens), torch.float32,
            allow_none=True)
    mk = _kept_lists(g, kv_idx, kv_cnt)
    _call("ssta_attention_fwd_tokens", ctypes.byref(g), ctypes.byref(p), _ptr(q), _ptr(k),
          _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), mk, _ptr(o), _ptr(lse), _stream(stream))


def ssta_calibrate_mfma(operands, sink, grid: int, iters: int, stream=None):
    """Measurement aid: grid x 4 waves x iters x 4 bf16 32x32x16 products on
    register-resident operands (operands: 256x8 bf16, sink: grid*256 fp32)."""
    _expect("operands", operands, (256, 8), torch.bfloat16)
    _expect("sink", sink, (grid * 256,), torch.float32)
    _call("ssta_calibrate_mfma", _ptr(operands), _ptr(sink), grid, iters, _stream(stream))


def ssta_attention_bwd_workspace_bytes(g: SstaGeom) -> int:
    v = load().ssta_attention_bwd_workspace_bytes(ctypes.byref(g))
    if v < 0:
        raise SstaError("ssta_attention_bwd_workspace_bytes", v)
    return v


def ssta_attention_bwd(g: SstaGeom, p: SstaParams, q, k, v, o, dout, lse, kv_idx, kv_cnt, dq, dk,
                       dv, workspace, stream=None):
    """Gradients of the block-sparse attention with the kept lists fixed; all
    tensors token-major bf16 [B, h, S, 128] except lse (tile-major fp32)."""
    tok = (g.batch, g.heads, g.seq_len, g.head_dim)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _expect(name, t, tok, torch.bfloat16)
    _expect("lse", lse, (g.batch, g.heads, g.n_rows, g.tile_tokens), torch.float32)
    mk = _kept_lists(g, kv_idx, kv_cnt)
    ws_bytes = _workspace(workspace)
    _call("ssta_attention_bwd", ctypes.byref(g), ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
          _ptr(o), _ptr(dout), _ptr(lse), _ptr(kv_idx), _ptr(kv_cnt), mk, _ptr(dq), _ptr(dk),
          _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream))

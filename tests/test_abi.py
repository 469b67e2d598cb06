"""The C ABI on the host: libssta.so loads, exports every function that
include/ssta.h declares, and rejects bad arguments before any HIP call.
No kernel is launched here (the pointers passed are never valid buffers, and
every call is built to fail validation)."""
import ctypes
import os
import re

import numpy as np
import pytest

import video_dit_block_tile_amd as m
from video_dit_block_tile_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ARG, SHAPE, ALIGN, NO_DEV, WS = -1, -2, -3, -4, -7


def _declared():
    text = open(os.path.join(ROOT, "include", "ssta.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssta_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = m.load()
    names = _declared()
    assert "ssta_attention_fwd" in names and len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(L.SIGNATURES)


def test_header_is_plain_c(tmp_path):
    """include/ssta.h compiles as C11 and a C program links against the
    library and calls its host-side entry points (no device needed)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_ssta.c"
    src.write_text(r"""
#include <stdio.h>
#include "ssta.h"
int main(void) {
  ssta_geom_t g = {1, 2, 128, 4, 16, 16, 2, 8, 8, 77};
  ssta_params_t p;
  if (ssta_default_params(&p, 128) != SSTA_OK) return 1;
  if (ssta_default_params(NULL, 128) != SSTA_ERR_ARG) return 2;
  p.topk = 2;
  printf("%lld %d %d %a %a %a %d %d %d %u %s\n", (long long)ssta_block_rows(&g),
         ssta_topk_width(&g, &p), ssta_max_kept(&g, &p), (double)p.lambda_, (double)p.beta,
         (double)p.scale, p.win_t, p.win_h, p.win_w, p.flags,
         ssta_status_string(SSTA_ERR_SHAPE));
  return 0;
}
""")
    lib = m.library_path()
    exe = tmp_path / "use_ssta"
    # The compiler runs without any preloaded runtime.  A sanitizer run preloads
    # one, and its instrumented library leaves the runtime's symbols to it.
    cc_env = {k: v for k, v in os.environ.items() if k != "LD_PRELOAD"}
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), lib, "-Wl,--allow-shlib-undefined", "-o", str(exe)], check=True,
                   env=cc_env)
    env = dict(os.environ, LD_LIBRARY_PATH=os.path.dirname(lib))
    out = subprocess.run([str(exe)], capture_output=True, text=True, env=env, check=True).stdout
    rows, width, kept, lam, beta, scale, wt, wh, ww, flags, text = out.split(maxsplit=10)
    assert (int(rows), int(width), int(kept)) == (9, 2, 8)
    # the pages' defaults as the library states them: lambda 0.9 and 1 - 0.9 as
    # fp32 values, the attention equation's 1/sqrt(128), window +-1, no flags
    assert float.fromhex(lam) == float(np.float32(0.9))
    assert float.fromhex(beta) == float(np.float32(1.0 - 0.9))
    assert float.fromhex(scale) == float(np.float32(1.0 / np.sqrt(128.0)))
    assert (int(wt), int(wh), int(ww), int(flags)) == (1, 1, 1, 0)
    assert text.strip() == lib_status_text(SHAPE)


def lib_status_text(code):
    return m.load().ssta_status_string(code).decode()


def test_status_strings():
    lib = m.load()
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.ssta_status_string(code)
    assert lib.ssta_status_string(99) == b"unknown status"


def _g(**kw):
    base = dict(batch=1, heads=2, T=4, H=16, W=16, tile=(2, 8, 8))
    base.update(kw)
    return m.make_geom(base["batch"], base["heads"], base["T"], base["H"], base["W"],
                       tile=base["tile"], head_dim=base.get("head_dim", 128))


def test_geometry_validation():
    lib = m.load()
    good = 16
    cases = [
        (_g(head_dim=64), SHAPE),
        (_g(tile=(4, 8, 8)), SHAPE),          # 256 tokens per block
        (_g(tile=(3, 8, 8)), SHAPE),          # does not divide T
        (_g(T=0), ARG),
        (_g(batch=-1), ARG),
        (_g(tile=(0, 8, 8)), ARG),
    ]
    for g, want in cases:
        assert lib.ssta_tile_pool(ctypes.byref(g), good, good, 0, None, None) == want
    assert lib.ssta_tile_pool(None, good, good, 0, None, None) == ARG


def test_block_rows_of_joint_sequences():
    """Text blocks follow the clip's blocks, 128 tokens each; the selection
    sizes do not see the text."""
    lib = m.load()
    assert m.ssta_block_rows(m.make_geom(1, 2, 4, 16, 16)) == 8
    assert m.ssta_block_rows(m.make_geom(1, 2, 4, 16, 16, text_len=77)) == 9
    assert m.ssta_block_rows(m.make_geom(1, 2, 4, 16, 16, text_len=256)) == 10
    assert m.ssta_block_rows(m.make_geom(1, 2, 4, 16, 16, text_len=257)) == 11
    assert m.ssta_block_rows(m.make_geom(1, 2, 5, 20, 24, text_len=1)) == 28   # ragged grid
    g = m.make_geom(1, 16, 60, 48, 80, text_len=256)
    p = m.make_params(topk=48)
    assert m.ssta_topk_width(g, p) == 48 and m.ssta_max_kept(g, p) == 27 + 48
    bad = m.make_geom(1, 2, 4, 16, 16, text_len=-1)
    assert lib.ssta_block_rows(ctypes.byref(bad)) == ARG
    assert lib.ssta_tile_pool(ctypes.byref(bad), 16, 16, 0, None, None) == ARG


def test_pointer_validation():
    lib = m.load()
    g = _g()
    assert lib.ssta_tile_pool(ctypes.byref(g), None, 16, 0, None, None) == ARG
    assert lib.ssta_tile_pool(ctypes.byref(g), 17, 16, 0, None, None) == ALIGN
    assert lib.ssta_tile_pool(ctypes.byref(g), 16, 24, 0, None, None) == ALIGN
    assert lib.ssta_tile_pool(ctypes.byref(g), 16, None, 0, None, None) == ARG
    assert lib.ssta_tile_pool(ctypes.byref(g), 16, 32, 5, None, None) == ARG   # layout
    assert lib.ssta_tile_unpermute(ctypes.byref(g), 16, 8, None) == ALIGN


def test_params_validation():
    lib = m.load()
    g = _g()
    for kw in (dict(win=(-1, 0, 0)), dict(topk=-3), dict(scale=0.0), dict(scale=float("inf")),
               dict(lambda_=float("nan")), dict(flags=1 << 5)):
        p = m.make_params(**kw)
        assert lib.ssta_max_kept(ctypes.byref(g), ctypes.byref(p)) == ARG
        assert lib.ssta_build_mask(ctypes.byref(g), ctypes.byref(p), 16, 16, 16, None,
                                   None) == ARG


def test_widths_and_capacity():
    g = m.make_geom(1, 16, 60, 48, 80)                  # 30 x 6 x 10 blocks
    p = m.make_params(topk=48)
    assert m.ssta_topk_width(g, p) == 48
    assert m.ssta_max_kept(g, p) == 27 + 48
    p = m.make_params(topk=5000)
    assert m.ssta_topk_width(g, p) == 1800 and m.ssta_max_kept(g, p) == 1800
    p = m.make_params(topk=48, flags=m.COMBINE_AND)
    assert m.ssta_max_kept(g, p) == 27
    p = m.make_params(win=(0, 0, 0), topk=2000, flags=m.TOPK_EXCLUDE_WINDOW)
    assert m.ssta_topk_width(g, p) == 1799
    gt = m.make_geom(1, 2, 4, 16, 16)                   # 2 x 2 x 2 blocks
    assert m.ssta_max_kept(gt, m.make_params(topk=2)) == 8
    # the normalised means, Score_r, its partial sums per group of 128 key
    # blocks and Score_i (16 x 1800 x 1800 fp32), each region 256-byte aligned
    ws = m.ssta_workspace_bytes(g, m.make_params(topk=48))
    need = 2 * 16 * 1800 * 128 * 4 + 16 * 1800 * 4 + 16 * 15 * 1800 * 4 + 16 * 1800 * 1800 * 4
    assert need <= ws < need + 5 * 256


def test_workspace_and_score_validation():
    lib = m.load()
    g = _g()
    p = m.make_params(topk=2)
    need = m.ssta_workspace_bytes(g, p)
    assert lib.ssta_score_select(ctypes.byref(g), ctypes.byref(p), 16, 16, 16, None, need,
                                 None) == WS
    assert lib.ssta_score_select(ctypes.byref(g), ctypes.byref(p), 16, 16, 16, 16, need - 1,
                                 None) == WS
    big = m.make_geom(1, 1, 80, 64, 128)                # 40 x 8 x 16 = 5120 blocks
    assert lib.ssta_score_select(ctypes.byref(big), ctypes.byref(p), 16, 16, 16, 16, 1 << 40,
                                 None) == SHAPE


def test_default_params_through_the_binding():
    """make_params takes its defaults from ssta_default_params (no formula in
    the binding) and agrees with the oracle's constants."""
    import oracle
    p = m.make_params(topk=7)
    assert np.float32(p.lambda_) == oracle.DEFAULT_LAMBDA
    assert np.float32(p.beta) == oracle.DEFAULT_BETA
    assert np.float32(p.scale) == np.float32(1.0 / np.sqrt(128.0))
    assert (p.win_t, p.win_h, p.win_w, p.topk, p.flags) == (1, 1, 1, 7, 0)
    q = m.make_params(head_dim=64)
    assert np.float32(q.scale) == np.float32(0.125)
    assert m.load().ssta_default_params(None, 128) == ARG
    r = L.SstaParams()
    assert m.load().ssta_default_params(ctypes.byref(r), 0) == ARG


def test_score_heads_limit():
    """The scoring grids put batch*heads on a grid axis: more than 65535 is a
    shape error, not a launch failure."""
    lib = m.load()
    p = m.make_params(topk=2)
    ok = m.make_geom(5, 13107, 2, 8, 8)                  # 65535 heads, one block each
    over = m.make_geom(2, 32768, 2, 8, 8)                # 65536
    assert lib.ssta_score_select(ctypes.byref(ok), ctypes.byref(p), 16, 16, 16, 16, 1,
                                 None) == WS
    assert lib.ssta_score_select(ctypes.byref(over), ctypes.byref(p), 16, 16, 16, 16, 1 << 40,
                                 None) == SHAPE
    assert lib.ssta_scores(ctypes.byref(over), ctypes.byref(p), 16, 16, 16, None, 16, 1 << 40,
                           None) == SHAPE


def test_size_limits_at_the_boundary():
    """ssta_score_select takes up to 4096 blocks; the attention entry points up
    to 65535 blocks per head (one head's K/V addressed with 32-bit offsets)."""
    lib = m.load()
    p = m.make_params(topk=2)
    at_limit = m.make_geom(1, 1, 32, 128, 128)           # 16 x 16 x 16 = 4096 blocks
    over = m.make_geom(1, 1, 34, 8, 1928)                # 17 x 1 x 241 = 4097 blocks
    assert at_limit.n_tiles == 4096 and over.n_tiles == 4097
    # accepted shape: the call gets as far as the (too small) workspace
    assert lib.ssta_score_select(ctypes.byref(at_limit), ctypes.byref(p), 16, 16, 16, 16, 1,
                                 None) == WS
    assert lib.ssta_score_select(ctypes.byref(over), ctypes.byref(p), 16, 16, 16, 16, 1 << 40,
                                 None) == SHAPE
    rows_max = m.make_geom(1, 1, 510, 2056, 8)            # 255 x 257 x 1 = 65535 blocks
    rows_over = m.make_geom(1, 1, 512, 2048, 8)           # 256 x 256 x 1 = 65536 blocks
    assert rows_max.n_tiles == 65535 and rows_over.n_tiles == 65536
    # a negative list width is rejected after the size check, so ARG means
    # the shape was accepted (and nothing is ever launched)
    args = (16, 16, 16, 16, 16, -1, 16, None, None)
    assert lib.ssta_attention_fwd(ctypes.byref(rows_max), ctypes.byref(p), *args) == ARG
    assert lib.ssta_attention_fwd(ctypes.byref(rows_over), ctypes.byref(p), *args) == SHAPE
    # text blocks count towards the attention limit
    rows_text = m.make_geom(1, 1, 510, 2056, 8, text_len=1)
    assert lib.ssta_attention_fwd(ctypes.byref(rows_text), ctypes.byref(p), *args) == SHAPE


def test_attention_argument_rules():
    lib = m.load()
    g = _g()
    p = m.make_params(topk=2)
    # dense takes neither list; a list needs its count array
    assert lib.ssta_attention_fwd(ctypes.byref(g), ctypes.byref(p), 16, 16, 16, 16, None, 0,
                                  16, None, None) == ARG
    assert lib.ssta_attention_fwd(ctypes.byref(g), ctypes.byref(p), 16, 16, 16, None, None, 3,
                                  16, None, None) == ARG
    assert lib.ssta_attention_fwd(ctypes.byref(g), ctypes.byref(p), 16, 16, 16, 16, 16, 9,
                                  16, None, None) == ARG          # max_kept > n_tiles


def test_calibration_argument_rules():
    lib = m.load()
    assert lib.ssta_calibrate_mfma(16, 16, 0, 10, None) == ARG       # empty grid
    assert lib.ssta_calibrate_mfma(16, 16, 4, 0, None) == ARG        # no iterations
    assert lib.ssta_calibrate_mfma(None, 16, 4, 10, None) == ARG
    assert lib.ssta_calibrate_mfma(8, 16, 4, 10, None) == ALIGN


def test_no_device_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path")
    lib = m.load()
    g = _g()
    assert lib.ssta_tile_pool(ctypes.byref(g), 16, 32, 0, None, None) == NO_DEV
    assert lib.ssta_calibrate_mfma(16, 16, 4, 10, None) == NO_DEV
    with pytest.raises(m.SstaError):
        L._call("ssta_tile_pool", ctypes.byref(g), 16, 32, 0, None, None)


def test_noalloc_scratch_limit():
    """The entry point without a workspace scores at least one head per pass
    of its 64 MiB scratch: a 4,096-block head (64 MiB of Score_i alone) is a
    shape error; a 3,600-block head fits, and the call gets as far as the
    output pointer's check (a misaligned one here, so nothing runs)."""
    lib = m.load()
    p = m.make_params(topk=2)
    big = m.make_geom(1, 1, 32, 128, 128)                # 16 x 16 x 16 = 4096 blocks
    fits = m.make_geom(1, 16, 60, 48, 80, tile=(4, 4, 4))  # 15 x 12 x 20 = 3600 blocks
    assert big.n_tiles == 4096 and fits.n_tiles == 3600
    assert lib.ssta_score_select_noalloc(ctypes.byref(big), ctypes.byref(p), 16, 16, 16,
                                         None) == SHAPE
    assert lib.ssta_score_select_noalloc(ctypes.byref(fits), ctypes.byref(p), 16, 16, 8,
                                         None) == ALIGN
    assert lib.ssta_score_select_noalloc(ctypes.byref(fits), ctypes.byref(p), None, 16, 16,
                                         None) == ARG

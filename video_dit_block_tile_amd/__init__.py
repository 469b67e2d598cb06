"""MI355X-native (gfx950) SSTA forward: Selective and Sliding Tile Attention.

The computation runs in hand-written HIP kernels inside ``libssta.so`` behind
the C ABI of ``include/ssta.h``; this package is the Python binding (same
function names) plus a plan object that chains the calls.  PyTorch supplies
device memory and the HIP stream only.
"""
from ._lib import (COMBINE_AND, LAYOUT_DIM_MAJOR, LAYOUT_TOKEN_MAJOR, TOPK_EXCLUDE_WINDOW,
                   SstaError, SstaGeom, SstaParams, library_path, load, make_geom, make_params,
                   ssta_attention_bwd, ssta_attention_bwd_workspace_bytes, ssta_attention_fwd,
                   ssta_attention_fwd_tokens, ssta_block_rows, ssta_build_mask,
                   ssta_calibrate_mfma, ssta_max_kept, ssta_score_select,
                   ssta_score_select_noalloc, ssta_scores,
                   ssta_tile_pool, ssta_tile_unpermute, ssta_topk_width, ssta_workspace_bytes)
from .pipeline import SstaPlan, ssta_forward

__all__ = [
    "COMBINE_AND", "LAYOUT_DIM_MAJOR", "LAYOUT_TOKEN_MAJOR", "TOPK_EXCLUDE_WINDOW", "SstaError",
    "SstaGeom", "SstaParams", "SstaPlan", "library_path", "load", "make_geom", "make_params",
    "ssta_attention_fwd", "ssta_attention_fwd_tokens", "ssta_calibrate_mfma", "ssta_attention_bwd",
    "ssta_attention_bwd_workspace_bytes", "ssta_block_rows", "ssta_build_mask", "ssta_forward", "ssta_max_kept",
    "ssta_score_select", "ssta_score_select_noalloc", "ssta_scores", "ssta_tile_pool",
    "ssta_tile_unpermute",
    "ssta_topk_width", "ssta_workspace_bytes",
]

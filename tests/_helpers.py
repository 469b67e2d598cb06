"""Helpers shared by the GPU tests: host<->device marshalling of generator
arrays and the comparison bars.

Tolerances for the bf16 attention output against the fp64 oracle: max-abs
2e-2 and mean-abs 2e-3 (bf16 inputs and output, fp32 accumulation); LSE
1e-3 absolute.  Everything integer (tile copies, top-k ids, kept lists,
bitmasks) and the fp32 block means and scores must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synthetic_inputs as si

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def to_dev(x: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device bf16 tensor, bit for bit."""
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def geom_of(wl):
    import video_dit_block_tile_amd as m
    return m.make_geom(wl.batch, wl.heads, wl.T, wl.H, wl.W, tile=wl.tile, head_dim=wl.head_dim)


def params_of(wl, flags=0, topk=None):
    import video_dit_block_tile_amd as m
    return m.make_params(win=wl.win, topk=wl.topk if topk is None else topk,
                         lambda_=float(oracle.DEFAULT_LAMBDA), beta=float(oracle.DEFAULT_BETA),
                         scale=oracle.default_scale(wl), flags=flags)


def sample_rows(wl, count: int, seed: int = 0) -> np.ndarray:
    """Deterministic sample of (batch*head, query block) rows: every corner and
    edge-centre block of the block grid in the first and last head, plus random rows."""
    nt, ny, nx = wl.tile_grid
    n = wl.n_tiles
    special = set()
    for t in {0, nt // 2, nt - 1}:
        for y in {0, ny // 2, ny - 1}:
            for x in {0, nx // 2, nx - 1}:
                special.add((t * ny + y) * nx + x)
    bh_all = wl.batch * wl.heads
    rows = set()
    for bh in {0, bh_all - 1}:
        for i in special:
            rows.add(bh * n + i)
    rng = np.random.default_rng(seed)
    extra = rng.choice(bh_all * n, size=min(count, bh_all * n), replace=False)
    rows.update(int(r) for r in extra)
    return np.array(sorted(rows), dtype=np.int64)


def compare_o(o_gpu_rows: np.ndarray, o_ref: np.ndarray):
    err = np.abs(o_gpu_rows.astype(np.float64) - o_ref)
    return float(err.max()), float(err.mean())


def token_rows(wl, rows):
    """[len(rows), 128] token indices of the query rows (b*heads+h)*n_tiles + i, in in-block order."""
    n = wl.n_tiles
    return np.array([[oracle.tile_to_token(wl, int(r) % n, t) for t in range(128)] for r in rows])


def o_rows(wl, o_tok: torch.Tensor, rows) -> np.ndarray:
    """fp32 O rows [len(rows), 128, 128] gathered from a token-major output."""
    o = o_tok.float().cpu().numpy().reshape(wl.batch * wl.heads, wl.n_tokens, 128)
    tok = token_rows(wl, rows)
    bh = np.asarray(rows) // wl.n_tiles
    return o[bh[:, None], tok]

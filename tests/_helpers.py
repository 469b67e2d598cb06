"""Helpers shared by the GPU tests: host<->device marshalling of generator
arrays and the comparison bars.

Tolerances for the bf16 attention output against the fp64 oracle: max-abs
2e-2 and mean-abs 2e-3 (bf16 inputs and output, fp32 accumulation).  The LSE
is held to a per-query bound derived from the kernel's arithmetic (see
lse_bound; rows with nothing kept must be exactly -inf).  Everything integer (tile copies, top-k
ids, kept lists, bitmasks) and the fp32 block means and scores must match bit
for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synthetic_inputs as si

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3


def to_dev(x: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device bf16 tensor, bit for bit."""
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def geom_of(wl):
    import video_dit_block_tile_amd as m
    return m.make_geom(wl.batch, wl.heads, wl.T, wl.H, wl.W, tile=wl.tile, head_dim=wl.head_dim,
                       text_len=wl.text_len)


def params_of(wl, flags=0, topk=None, lambda_=None, beta=None):
    import video_dit_block_tile_amd as m
    return m.make_params(win=wl.win, topk=wl.topk if topk is None else topk,
                         lambda_=float(oracle.DEFAULT_LAMBDA if lambda_ is None else lambda_),
                         beta=float(oracle.DEFAULT_BETA if beta is None else beta),
                         scale=oracle.default_scale(wl), flags=flags)


def sample_rows(wl, count: int, seed: int = 0) -> np.ndarray:
    """Deterministic sample of (batch*head, query block) rows: every corner and
    edge-centre block of the block grid and every text block, in the first and
    last head, plus random rows.  Rows are (b*heads + h)*n_rows + block."""
    nt, ny, nx = wl.tile_grid
    n = wl.n_rows
    special = set(range(wl.n_tiles, n))
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
    """[len(rows), 128] token indices of the query rows (b*heads+h)*n_rows + i, in in-block
    order (-1 where a ragged grid or the text has no token)."""
    n = wl.n_rows
    return np.array([[oracle.tile_to_token(wl, int(r) % n, t) for t in range(128)] for r in rows])


def o_rows(wl, o_tok: torch.Tensor, rows) -> np.ndarray:
    """fp32 O rows [len(rows), 128, 128] gathered from a token-major output;
    positions beyond a ragged grid (no token) read as zero."""
    o = o_tok.float().cpu().numpy().reshape(wl.batch * wl.heads, wl.seq_len, 128)
    tok = token_rows(wl, rows)
    bh = np.asarray(rows) // wl.n_rows
    out = o[bh[:, None], np.maximum(tok, 0)]
    out[tok < 0] = 0.0
    return out


def lse_bound(wl, q, k, rows) -> np.ndarray:
    """[len(rows), 128] bound on |LSE - LSE_oracle| (natural log) per query.

    Three error sources, each bounded generously:
    - the denominator sums the probabilities after rounding them to bf16 (the
      same weights the P.V product uses): relative error at most 2^-9, so
      the LSE moves by at most log(1 + 2^-9);
    - each score is a 128-term fp32 accumulation on the matrix cores: error at
      most 128 * 2^-23 * sum_d |q_d k_d| <= 2^-16 * |q| * |k| (Cauchy-Schwarz),
      times the softmax scale; the LSE, a smooth maximum of the scores, moves
      by at most the largest score error, so |k| is the head's largest key norm;
    - fp32 exp2/log2, the scaling fma and the fp32 running sum: at most 2^-12.
    """
    bh_all = wl.batch * wl.heads
    qn = np.linalg.norm(si.bf16_bits_to_f32(q).reshape(bh_all, wl.seq_len, 128)
                        .astype(np.float64), axis=-1)
    kmax = np.linalg.norm(si.bf16_bits_to_f32(k).reshape(bh_all, wl.seq_len, 128)
                          .astype(np.float64), axis=-1).max(axis=-1)
    rows = np.asarray(rows)
    bh = rows // wl.n_rows
    tok = token_rows(wl, rows)
    scale = oracle.default_scale(wl)
    return (np.log1p(2.0 ** -9) + 2.0 ** -16 * scale * qn[bh[:, None], tok] * kmax[bh][:, None]
            + 2.0 ** -12)


def check_lse(wl, q, k, rows, lse: np.ndarray, lse_ref: np.ndarray):
    """Empty rows (-inf) must match exactly; the rest must lie within lse_bound.
    Returns the largest error as a fraction of its bound."""
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty)
    if empty.all():
        return 0.0
    err = np.abs(lse[~empty] - lse_ref[~empty])
    ratio = float((err / lse_bound(wl, q, k, rows)[~empty]).max())
    assert ratio <= 1.0, ratio
    return ratio

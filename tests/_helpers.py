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
    """[len(rows), R] token indices of the query rows (b*heads+h)*n_rows + i, in in-block
    order (-1 where a ragged grid or the text has no token)."""
    n = wl.n_rows
    return np.array([[oracle.tile_to_token(wl, int(r) % n, t) for t in range(wl.tile_tokens)]
                     for r in rows])


def o_rows(wl, o_tok: torch.Tensor, rows) -> np.ndarray:
    """fp32 O rows [len(rows), R, 128] gathered from a token-major output;
    positions beyond a ragged grid (no token) read as zero."""
    o = o_tok.float().cpu().numpy().reshape(wl.batch * wl.heads, wl.seq_len, 128)
    tok = token_rows(wl, rows)
    bh = np.asarray(rows) // wl.n_rows
    out = o[bh[:, None], np.maximum(tok, 0)]
    out[tok < 0] = 0.0
    return out


def lse_bound(wl, q, k, rows) -> np.ndarray:
    """[len(rows), R] bound on |LSE - LSE_oracle| (natural log) per query.

    Three error sources, each bounded generously:
    - the denominator sums the probabilities after rounding them to bf16 (the
      same weights the P.V product uses): round-to-nearest bf16 keeps 8
      significand bits, so each weight is off by at most a relative 2^-8
      (the unit roundoff), and the LSE moves by at most log(1 + 2^-8);
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
    return (np.log1p(2.0 ** -8) + 2.0 ** -16 * scale * qn[bh[:, None], tok] * kmax[bh][:, None]
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


def _token_map(wl):
    """[n_rows, R] token of every (block, in-block position), -1 where none."""
    n = wl.n_rows
    return token_rows(wl, np.arange(n))


def _row_keys(wl, tmap, kv_idx, kv_cnt, b, h, i):
    """Key tokens (within the head) of query block i, in the oracle's order."""
    n = wl.n_tiles
    if i >= n:
        blocks = np.arange(wl.n_rows)
    else:
        blocks = np.concatenate([kv_idx[b, h, i, :kv_cnt[b, h, i]], np.arange(n, wl.n_rows)])
    toks = tmap[blocks.astype(np.int64)].reshape(-1)
    return toks[toks >= 0]


def _row_terms(wl, qf, kf, vf, dof, b, h, qtok, keys, scale):
    """fp64 softmax-row quantities of the queries qtok over keys."""
    Q, K, V, dO = qf[b, h, qtok], kf[b, h, keys], vf[b, h, keys], dof[b, h, qtok]
    s = Q @ K.T * scale
    s -= s.max(axis=1, keepdims=True)
    P = np.exp(s)
    P /= P.sum(axis=1, keepdims=True)
    O = P @ V
    D = (dO * O).sum(axis=1)
    dS = P * (dO @ V.T - D[:, None])
    # D is formed from the bf16-rounded O: |error| <= 2^-8 sum_d |dO_d| |O_d|;
    # dP = dO . v is a 128-term fp32 sum: |error| <= 2^-16 |dO| |v|
    eps_d = (2.0 ** -8 * (np.abs(dO) * np.abs(O)).sum(axis=1)
             + 2.0 ** -16 * np.linalg.norm(dO, axis=1) * np.linalg.norm(V, axis=1).max())
    return Q, K, dO, P, dS, eps_d


def bwd_bounds(wl, q, k, v, do, kv_idx, kv_cnt, q_rows, k_rows):
    """Per-element error bounds [len(rows), R, 128] on dq (q_rows) and dk, dv
    (k_rows) of the GPU backward, derived from its arithmetic (worst case,
    every error of one sign):
      - dS and P enter the products rounded to bf16 (relative 2^-8, the unit
        roundoff of an 8-bit significand) and P is
        recomputed from an LSE that carries its own small error; both are
        covered by 2^-7 relative on each term, so dq gets
        scale * 2^-7 * sum_b |dS_ab| |k_b| (dk likewise with |q_a|, dv with
        2^-7 * sum_a P_ab |dO_a|);
      - D = dO . O uses the bf16 output O: |dD_a| <= 2^-8 sum |dO_a| |O_a|,
        and dP_ab is an fp32 sum (<= 2^-16 |dO_a| |v_b|); either moves dS_ab by
        at most P_ab |dD_a| (both folded into dD_a): scale * sum_b P_ab |dD_a| |k_b|
        for dq, scale * sum_a P_ab |dD_a| |q_a| for dk;
      - the bf16 output rounding: 2^-8 |value| (with margin).
    Positions without a token, query rows that keep nothing and key blocks
    that no row keeps get bound 0 (their gradients must be exactly 0)."""
    R, scale = wl.tile_tokens, oracle.default_scale(wl)
    tmap = _token_map(wl)
    sh = (wl.batch, wl.heads, wl.seq_len, 128)
    qf, kf, vf, dof = (si.bf16_bits_to_f32(x).reshape(sh).astype(np.float64)
                       for x in (q, k, v, do))
    bq = np.zeros((len(q_rows), R, 128))
    for a, row in enumerate(q_rows):
        bh, i = divmod(int(row), wl.n_rows)
        b, h = divmod(bh, wl.heads)
        qt = tmap[i]
        there = qt >= 0
        keys = _row_keys(wl, tmap, kv_idx, kv_cnt, b, h, i)
        if keys.size == 0:
            continue          # a row that keeps nothing: dq is exactly 0 (bound 0)
        Q, K, dO, P, dS, eps_d = _row_terms(wl, qf, kf, vf, dof, b, h, qt[there], keys, scale)
        dq = scale * dS @ K
        bq[a, there] = (scale * (2.0 ** -7 * np.abs(dS) @ np.abs(K)
                                 + (P * eps_d[:, None]) @ np.abs(K)) + 2.0 ** -8 * np.abs(dq))
    bk = np.zeros((len(k_rows), R, 128))
    bv = np.zeros((len(k_rows), R, 128))
    for a, row in enumerate(k_rows):
        bh, j = divmod(int(row), wl.n_rows)
        b, h = divmod(bh, wl.heads)
        kt = tmap[j]
        there = kt >= 0
        acc_k = np.zeros((int(there.sum()), 128))
        acc_v = np.zeros_like(acc_k)
        dk = np.zeros_like(acc_k)
        dv = np.zeros_like(acc_k)
        # query blocks whose keys hold block j: clip rows listing it (every
        # clip row for a text block j), and every text row
        if j >= wl.n_tiles:
            users = np.arange(wl.n_rows)
        else:
            lists = kv_idx[b, h]
            listed = (lists == j) & (np.arange(lists.shape[1])[None, :] < kv_cnt[b, h][:, None])
            users = np.concatenate([np.nonzero(listed.any(axis=1))[0],
                                    np.arange(wl.n_tiles, wl.n_rows)])
        for i in users:
            keys = _row_keys(wl, tmap, kv_idx, kv_cnt, b, h, int(i))
            sel = np.nonzero(np.isin(keys, kt[there]))[0]
            qt = tmap[i]
            qt = qt[qt >= 0]
            Q, K, dO, P, dS, eps_d = _row_terms(wl, qf, kf, vf, dof, b, h, qt, keys, scale)
            # columns of this key block, in the block's position order
            col = {int(t): c for c, t in zip(sel, keys[sel])}
            cols = np.array([col[int(t)] for t in kt[there]])
            Pj, dSj = P[:, cols], dS[:, cols]
            acc_k += scale * (2.0 ** -7 * np.abs(dSj).T @ np.abs(Q)
                              + (Pj * eps_d[:, None]).T @ np.abs(Q))
            acc_v += 2.0 ** -7 * Pj.T @ np.abs(dO)
            dk += scale * dSj.T @ Q
            dv += Pj.T @ dO
        bk[a, there] = acc_k + 2.0 ** -8 * np.abs(dk)
        bv[a, there] = acc_v + 2.0 ** -8 * np.abs(dv)
    return bq, bk, bv

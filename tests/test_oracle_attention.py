"""Oracle pins for the block-sparse attention of Step 4.

Pinned against PyTorch's scaled_dot_product_attention in float64 on the CPU
(a library routine): with every block kept it must equal dense attention; in
general it must equal dense attention under the token-level mask expanded from
the kept-block lists; window 0 with k = 0 reduces it to attention inside each
block.  Also: V = 1 gives O = 1, and the log-sum-exp matches torch.logsumexp.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle
import synthetic_inputs as si


def _f64(x):
    return torch.from_numpy(si.bf16_bits_to_f32(x).astype(np.float64))


def _token_rows(wl, rows):
    """Token indices (token-major) of every query row in the oracle's output order."""
    n, R = wl.n_tiles, oracle.tile_tokens(wl)
    return np.array([[oracle.tile_to_token(wl, row % n, r) for r in range(R)] for row in rows])


def _token_mask(wl, kv_idx, kv_cnt, b, h):
    """Boolean [N, N] mask: query token may see key token iff its block is kept."""
    N = wl.n_tokens
    blk = np.array([oracle.token_to_tile(wl, t)[0] for t in range(N)])
    keep = np.zeros((wl.n_tiles, wl.n_tiles), bool)
    for i in range(wl.n_tiles):
        keep[i, kv_idx[b, h, i, :kv_cnt[b, h, i]]] = True
    return torch.from_numpy(keep[blk][:, blk])


def _sdpa(q, k, v, mask=None, scale=None):
    return Fnn.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)


def test_all_kept_equals_dense():
    wl = si.CONFIGS["tiny"]                 # the +-1 window covers all 8 blocks
    q, k, v = si.make_qkv(wl)
    out = oracle.forward(wl, q, k, v)
    assert np.all(out["kv_cnt"] == wl.n_tiles)
    rows = np.arange(wl.batch * wl.heads * wl.n_tiles)
    tok = _token_rows(wl, rows)
    sc = oracle.default_scale(wl)
    dense = _sdpa(_f64(q), _f64(k), _f64(v), scale=sc).numpy()
    for a, row in enumerate(rows):
        bh = row // wl.n_tiles
        np.testing.assert_allclose(out["o"][a], dense[0, bh][tok[a]], rtol=0, atol=1e-12)
    # the library's default scale is the fp32 value of 1/sqrt(d)
    assert abs(sc - 1 / math.sqrt(128)) < 1e-8


@pytest.mark.parametrize("name", ["grid32-w1-k2", "grid32-w0-k3", "dup-ties"])
def test_sparse_equals_token_masked_dense(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    out = oracle.forward(wl, q, k, v)
    rows = np.arange(wl.batch * wl.heads * wl.n_tiles)
    tok = _token_rows(wl, rows)
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    sc = oracle.default_scale(wl)
    for b in range(wl.batch):
        for h in range(wl.heads):
            mask = _token_mask(wl, out["kv_idx"], out["kv_cnt"], b, h)
            ref = _sdpa(qf[b, h], kf[b, h], vf[b, h], mask, sc).numpy()
            s = (qf[b, h] @ kf[b, h].T * sc).masked_fill(~mask, -math.inf)
            lse = torch.logsumexp(s, dim=-1).numpy()
            for i in range(wl.n_tiles):
                a = (b * wl.heads + h) * wl.n_tiles + i
                np.testing.assert_allclose(out["o"][a], ref[tok[a]], rtol=0, atol=1e-12)
                np.testing.assert_allclose(out["lse"][a], lse[tok[a]], rtol=0, atol=1e-12)


def test_window0_k0_is_blockwise_local():
    wl = si.ALL["grid32-w0-k0"]
    q, k, v = si.make_qkv(wl)
    out = oracle.forward(wl, q, k, v)
    assert np.all(out["kv_cnt"] == 1)
    sc = oracle.default_scale(wl)
    qt, kt, vt = (torch.from_numpy(si.bf16_bits_to_f32(oracle.permute(wl, x)).astype(np.float64))
                  for x in (q, k, v))
    ref = _sdpa(qt, kt, vt, scale=sc).numpy()          # attention within each block
    np.testing.assert_allclose(out["o"], ref.reshape(out["o"].shape), rtol=0, atol=1e-12)


def test_unit_values_give_unit_output():
    wl = si.ALL["ragged"]
    q, k, v = si.make_qkv(wl)
    ones = np.full_like(v, 0x3F80)                      # bf16 1.0
    rows = np.arange(0, wl.batch * wl.heads * wl.n_tiles, 7)
    out = oracle.forward(wl, q, k, ones, rows=rows)
    np.testing.assert_allclose(out["o"], 1.0, rtol=0, atol=1e-13)


def test_empty_row_under_and():
    wl = si.ALL["grid32-w0-k0"].with_(topk=1)
    q, k, v = si.make_qkv(wl)
    sel = oracle.select(wl, q, k, flags=oracle.COMBINE_AND)
    o, lse = oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"])
    for row in range(wl.batch * wl.heads * wl.n_tiles):
        b_h, i = divmod(row, wl.n_tiles)
        if sel["kv_cnt"].reshape(-1)[row] == 0:
            assert np.all(o[row] == 0) and np.all(np.isneginf(lse[row]))
        else:
            assert sel["kv_idx"].reshape(-1, sel["kv_idx"].shape[-1])[row, 0] == i

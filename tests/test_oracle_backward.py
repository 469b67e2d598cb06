"""Oracle pins for the gradients of Step 4's block-sparse attention (the
kept lists held fixed).

Pinned against PyTorch float64 autograd of dense softmax attention with a
token-level mask expanded from the kept lists (an independent
implementation of the same derivative), and against identities that hold for
any mask: per head the key gradients sum to zero (every row of dS sums to
zero), the value gradients sum to the summed dO of rows that keep anything,
and a constant V gives zero dq and dk.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


def _tok(wl):
    """[n_tiles, R] token index of each in-block position."""
    return np.array([[oracle.tile_to_token(wl, i, r) for r in range(oracle.tile_tokens(wl))]
                     for i in range(wl.n_tiles)])


def _to_tokens(wl, x_rows):
    """[B*h*n, R, D] rows in in-block order -> [B, h, N, D]."""
    bh, n = wl.batch * wl.heads, wl.n_tiles
    out = np.zeros((bh, wl.n_tokens, wl.head_dim))
    tok = _tok(wl)
    x = x_rows.reshape(bh, n, -1, wl.head_dim)
    for b in range(bh):
        out[b, tok.reshape(-1)] = x[b].reshape(-1, wl.head_dim)
    return out.reshape(wl.batch, wl.heads, wl.n_tokens, wl.head_dim)


def _torch_grads(wl, q, k, v, do, kv_idx, kv_cnt):
    f = lambda a: torch.from_numpy(si.bf16_bits_to_f32(a).astype(np.float64))
    qt, kt, vt = (f(a).requires_grad_(True) for a in (q, k, v))
    dot = f(do)
    n, tok = wl.n_tiles, _tok(wl)
    blk = np.empty(wl.n_tokens, np.int64)
    blk[tok.reshape(-1)] = np.repeat(np.arange(n), tok.shape[1])
    mask = np.zeros((wl.batch, wl.heads, wl.n_tokens, wl.n_tokens), bool)
    for b in range(wl.batch):
        for h in range(wl.heads):
            keep = np.zeros((n, n), bool)
            for i in range(n):
                keep[i, kv_idx[b, h, i, :kv_cnt[b, h, i]]] = True
            mask[b, h] = keep[blk][:, blk]
    s = torch.matmul(qt, kt.transpose(-1, -2)) * oracle.default_scale(wl)
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vt)
    (o * dot).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("name", ["tiny", "dup-ties", "grid32-w0-k3"])
def test_matches_torch_autograd(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    sel = oracle.select(wl, q, k)
    dq, dk, dv = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    tq, tk, tv = _torch_grads(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        got = _to_tokens(wl, mine)
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_sum_identities_and_constant_v():
    wl = si.ALL["grid32-w1-k2"]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    sel = oracle.select(wl, q, k)
    dq, dk, dv = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    bh, n, R = wl.batch * wl.heads, wl.n_tiles, 128
    dk = dk.reshape(bh, n * R, 128)
    dv = dv.reshape(bh, n * R, 128)
    dof = si.bf16_bits_to_f32(do).astype(np.float64).reshape(bh, wl.n_tokens, 128)
    assert np.all(sel["kv_cnt"] > 0)
    for b in range(bh):
        assert np.max(np.abs(dk[b].sum(axis=0))) <= 1e-9
        assert np.max(np.abs(dv[b].sum(axis=0) - dof[b].sum(axis=0))) <= 1e-9
    const = np.full_like(v, 0x3FC0)                 # 1.5 in every channel of every key
    dq1, dk1, dv1 = oracle.attention_bwd(wl, q, k, const, do, sel["kv_idx"], sel["kv_cnt"])
    assert np.max(np.abs(dq1)) <= 1e-10 and np.max(np.abs(dk1)) <= 1e-10
    assert np.max(np.abs(dv1.reshape(bh, -1, 128).sum(axis=1) - dof.sum(axis=1))) <= 1e-9


def test_row_selection_and_empty_rows():
    wl = si.ALL["grid32-w1-k2"]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    flags = oracle.COMBINE_AND
    sel = oracle.select(wl, q, k, flags)
    dq, dk, dv = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    rows = np.array([0, 5, 31, 40, 63])
    dq2, dk2, dv2 = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"], rows, rows)
    assert np.array_equal(dq2, dq[rows]) and np.array_equal(dk2, dk[rows])
    assert np.array_equal(dv2, dv[rows])
    cnt = sel["kv_cnt"].reshape(-1)
    assert np.all(dq[cnt == 0] == 0.0)
    kept = np.zeros(cnt.size, bool)
    idx = sel["kv_idx"].reshape(cnt.size, -1)
    bh = np.arange(cnt.size) // wl.n_tiles
    for r in range(cnt.size):
        kept[bh[r] * wl.n_tiles + idx[r, :cnt[r]]] = True
    assert np.all(dk[~kept] == 0.0) and np.all(dv[~kept] == 0.0)

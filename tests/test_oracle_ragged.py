"""Oracle pins for grids the block size does not divide (real latent grids:
61 x 45 x 80 for a 10 s 720p clip).  Reading: the block grid rounds up and the
edge blocks hold only the tokens that exist; block means average those tokens;
attention runs over the existing tokens of the kept blocks.

Pinned by brute force over token coordinates (block membership and counts,
fp64 block means) and against PyTorch float64 dense attention over the real
tokens with the token-level mask expanded from the kept lists (forward output,
log-sum-exp, and autograd gradients).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle
import synthetic_inputs as si

NAMES = ["partial", "partial-x"]


def _f64(x):
    return torch.from_numpy(si.bf16_bits_to_f32(x).astype(np.float64))


def _blocks(wl):
    """Block id of every token, by brute force over (t, y, x)."""
    T, H, W = wl.T, wl.H, wl.W
    tt, th, tw = wl.tile
    nt, ny, nx = (-(-T // tt), -(-H // th), -(-W // tw))
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return (((t // tt) * ny + y // th) * nx + x // tw).reshape(-1), nt * ny * nx


@pytest.mark.parametrize("name", NAMES)
def test_block_grid_and_membership(name):
    wl = si.ALL[name]
    blk, n = _blocks(wl)
    assert oracle.n_tiles(wl) == wl.n_tiles == n
    counts = np.bincount(blk, minlength=n)
    assert counts.min() < 128 < counts.max() + 1          # some blocks are partial
    for i in range(n):
        toks = [oracle.tile_to_token(wl, i, r) for r in range(128)]
        valid = [t for t in toks if t >= 0]
        assert len(valid) == counts[i]
        assert sorted(valid) == sorted(np.nonzero(blk == i)[0].tolist())
        assert all(oracle.token_to_tile(wl, t)[0] == i for t in valid)


@pytest.mark.parametrize("name", NAMES)
def test_permute_and_pool(name):
    wl = si.ALL[name]
    x = si.generate(wl, 1)
    xt = oracle.permute(wl, x)
    pooled = oracle.pool(wl, x).astype(np.float64)
    xf = si.bf16_bits_to_f32(x).astype(np.float64)
    blk, n = _blocks(wl)
    for b in range(wl.batch):
        for h in range(wl.heads):
            for i in range(n):
                for r in range(128):
                    tok = oracle.tile_to_token(wl, i, r)
                    want = x[b, h, tok] if tok >= 0 else np.zeros(128, np.uint16)
                    assert np.array_equal(xt[b, h, i, r], want)
                mean = xf[b, h, blk == i].mean(axis=0)
                assert np.max(np.abs(pooled[b, h, i] - mean)) <= 1e-5 * max(1.0, np.abs(mean).max())


def _mask(wl, sel, b, h):
    blk, n = _blocks(wl)
    keep = np.zeros((n, n), bool)
    for i in range(n):
        keep[i, sel["kv_idx"][b, h, i, :sel["kv_cnt"][b, h, i]]] = True
    return torch.from_numpy(keep[blk][:, blk])


@pytest.mark.parametrize("name", NAMES)
def test_forward_matches_dense_over_real_tokens(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    out = oracle.forward(wl, q, k, v)
    sc = oracle.default_scale(wl)
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    for b in range(wl.batch):
        for h in range(wl.heads):
            mask = _mask(wl, out, b, h)
            ref = Fnn.scaled_dot_product_attention(qf[b, h], kf[b, h], vf[b, h], attn_mask=mask,
                                                   scale=sc).numpy()
            s = (qf[b, h] @ kf[b, h].T * sc).masked_fill(~mask, -math.inf)
            lse = torch.logsumexp(s, dim=-1).numpy()
            for i in range(wl.n_tiles):
                a = (b * wl.heads + h) * wl.n_tiles + i
                for r in range(128):
                    tok = oracle.tile_to_token(wl, i, r)
                    if tok < 0:
                        assert not out["o"][a, r].any() and out["lse"][a, r] == -math.inf
                    else:
                        np.testing.assert_allclose(out["o"][a, r], ref[tok], rtol=0, atol=1e-12)
                        assert abs(out["lse"][a, r] - lse[tok]) <= 1e-12


@pytest.mark.parametrize("name", NAMES)
def test_backward_matches_autograd_over_real_tokens(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    sel = oracle.select(wl, q, k)
    dq, dk, dv = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    sc = oracle.default_scale(wl)
    qf, kf, vf, dof = _f64(q), _f64(k), _f64(v), _f64(do)
    for b in range(wl.batch):
        for h in range(wl.heads):
            qt, kt, vt = (x[b, h].clone().requires_grad_(True) for x in (qf, kf, vf))
            s = (qt @ kt.T * sc).masked_fill(~_mask(wl, sel, b, h), -math.inf)
            (torch.softmax(s, dim=-1) @ vt * dof[b, h]).sum().backward()
            for i in range(wl.n_tiles):
                a = (b * wl.heads + h) * wl.n_tiles + i
                for r in range(128):
                    tok = oracle.tile_to_token(wl, i, r)
                    for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
                        want = ref[tok].numpy() if tok >= 0 else 0.0
                        np.testing.assert_allclose(mine[a, r], want, rtol=0, atol=1e-12)

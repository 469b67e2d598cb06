"""Oracle pins for joint video + text sequences: the clip's tokens followed by
text tokens in one sequence, as single-stream DiT blocks see them ("HunyuanVideo-1.5:
An 8.3B-Parameter Video Diffusion Model Built for Consumer GPUs", section
"Architecture: From Prompt to Video"), with the text kept out of scoring (the
same page, section "Under the Hood: SSTA and Muon in Detail": text masking).

Readings pinned here: scoring and selection see the clip only; every clip query
block keeps every text token on top of its kept blocks; a text query attends to
every token.  The references below are written independently of the oracle: the
token/block map is computed from its definition with numpy, and attention is a
dense fp64 softmax under a token-level mask (numpy) or PyTorch fp64 autograd.

The same pins run on 64-token blocks (4x4x4, the block size the technical
report's summary page gives as its example in Step 1), with and without text.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

JOINT_SMALL = ["joint-tiny", "joint-grid32", "joint-partial", "t64-grid", "t64-partial"]


def _block_map(wl):
    """(block, in-block position) of every token of the joint sequence."""
    tt, th, tw = wl.tile
    R = tt * th * tw
    _, ny, nx = wl.tile_grid
    t, y, x = np.meshgrid(np.arange(wl.T), np.arange(wl.H), np.arange(wl.W), indexing="ij")
    blk = (((t // tt) * ny + y // th) * nx + x // tw).ravel()
    pos = (((t % tt) * th + y % th) * tw + x % tw).ravel()
    u = np.arange(wl.text_len)
    return (np.concatenate([blk, wl.n_tiles + u // R]),
            np.concatenate([pos, u % R]))


def _token_mask(wl, kv_idx, kv_cnt, b, h):
    """[S, S] keys each query token may attend to."""
    n, nr = wl.n_tiles, wl.n_rows
    keep = np.zeros((nr, nr), bool)
    for i in range(n):
        keep[i, kv_idx[b, h, i, :kv_cnt[b, h, i]]] = True
    keep[:, n:] = True          # text blocks: kept by every query block
    keep[n:, :] = True          # text query blocks: keep every block
    blk, _ = _block_map(wl)
    return keep[blk][:, blk]


def _dense(wl, q, k, v, mask):
    """fp64 masked softmax attention of one head: (o [S, D], lse [S])."""
    f = lambda a: si.bf16_bits_to_f32(a).astype(np.float64)
    s = f(q) @ f(k).T * oracle.default_scale(wl)
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ f(v), (mx + np.log(l))[:, 0]


def _rows_to_tokens(wl, x_rows, b, h):
    """Oracle rows of head (b, h) [n_rows, R, ...] -> token order [S, ...]."""
    blk, pos = _block_map(wl)
    bh = b * wl.heads + h
    R = wl.tile[0] * wl.tile[1] * wl.tile[2]
    x = x_rows.reshape((wl.batch * wl.heads, wl.n_rows, R) + x_rows.shape[2:])[bh]
    return x[blk, pos]


@pytest.mark.parametrize("name", JOINT_SMALL)
def test_forward_matches_masked_dense(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    assert q.shape == (wl.batch, wl.heads, wl.seq_len, 128)
    sel = oracle.select(wl, q, k)
    o, lse = oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"])
    assert o.shape[0] == wl.batch * wl.heads * wl.n_rows
    for b in range(wl.batch):
        for h in range(wl.heads):
            mask = _token_mask(wl, sel["kv_idx"], sel["kv_cnt"], b, h)
            ro, rl = _dense(wl, q[b, h], k[b, h], v[b, h], mask)
            got_o = _rows_to_tokens(wl, o, b, h)
            got_l = _rows_to_tokens(wl, lse, b, h)
            assert np.max(np.abs(got_o - ro)) <= 1e-12
            assert np.max(np.abs(got_l - rl)) <= 1e-11


def test_all_kept_is_textbook_dense_attention():
    """Tiny grid: the window covers every block, so the joint sequence is plain
    dense attention over all clip and text tokens."""
    wl = si.ALL["joint-tiny"]
    q, k, v = si.make_qkv(wl)
    sel = oracle.select(wl, q, k)
    assert np.all(sel["kv_cnt"] == wl.n_tiles)
    o, lse = oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"])
    for h in range(wl.heads):
        f = lambda a: torch.from_numpy(si.bf16_bits_to_f32(a).astype(np.float64))
        ref = torch.softmax(f(q[0, h]) @ f(k[0, h]).T * oracle.default_scale(wl), -1) @ f(v[0, h])
        got = _rows_to_tokens(wl, o, 0, h)
        assert np.max(np.abs(got - ref.numpy())) <= 1e-12


@pytest.mark.parametrize("name", ["t64-grid", "t64-partial"])
def test_pool_of_64_token_blocks(name):
    """Block means over the (existing) tokens of each 4x4x4 block, against an
    fp64 mean gathered with the numpy block map."""
    wl = si.ALL[name]
    q, _, _ = si.make_qkv(wl)
    blk, _ = _block_map(wl)
    pooled = oracle.pool(wl, q).astype(np.float64)
    xf = si.bf16_bits_to_f32(q).astype(np.float64)
    for b in range(wl.batch):
        for h in range(wl.heads):
            for i in range(wl.n_tiles):
                mean = xf[b, h, :wl.n_tokens][blk[:wl.n_tokens] == i].mean(axis=0)
                assert np.max(np.abs(pooled[b, h, i] - mean)) <= 1e-5 * max(1.0, np.abs(mean).max())


def test_positions_past_the_text_are_empty():
    wl = si.ALL["joint-tiny"]                          # 77 text tokens: one partial block
    q, k, v = si.make_qkv(wl)
    sel = oracle.select(wl, q, k)
    rows = np.array([wl.n_rows - 1])                   # head 0, the text block
    o, lse = oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"], rows)
    assert np.all(np.isfinite(lse[0, :77])) and np.all(np.isneginf(lse[0, 77:]))
    assert not o[0, 77:].any()


@pytest.mark.parametrize("name", JOINT_SMALL)
def test_text_is_not_scored(name):
    """The selection of a joint sequence equals that of its clip alone, and
    does not move when the text changes."""
    wl = si.ALL[name]
    q, k, _ = si.make_qkv(wl)
    clip = wl.with_(text_len=0)
    a = oracle.select(wl, q, k)
    b = oracle.select(clip, q[:, :, :wl.n_tokens], k[:, :, :wl.n_tokens])
    q2, k2 = q.copy(), k.copy()
    q2[:, :, wl.n_tokens:] ^= 0x1234
    k2[:, :, wl.n_tokens:] ^= 0x0F0F
    c = oracle.select(wl, q2, k2)
    for key in ("q_pooled", "k_pooled", "scores", "topk", "kv_idx", "kv_cnt", "bitmask"):
        assert np.array_equal(a[key], b[key]) and np.array_equal(a[key], c[key]), key


@pytest.mark.parametrize("name", JOINT_SMALL)
def test_permute_appends_text_blocks(name):
    wl = si.ALL[name]
    q, _, _ = si.make_qkv(wl)
    R = wl.tile[0] * wl.tile[1] * wl.tile[2]
    t = oracle.permute(wl, q)
    assert t.shape == (wl.batch, wl.heads, wl.n_rows, R, 128)
    clip = oracle.permute(wl.with_(text_len=0), q[:, :, :wl.n_tokens])
    assert np.array_equal(t[:, :, :wl.n_tiles], clip)
    blk, pos = _block_map(wl.with_(text_len=0))
    assert np.array_equal(clip[:, :, blk, pos], q[:, :, :wl.n_tokens])
    txt = np.zeros((wl.batch, wl.heads, wl.n_text_blocks * R, 128), np.uint16)
    txt[:, :, :wl.text_len] = q[:, :, wl.n_tokens:]
    assert np.array_equal(t[:, :, wl.n_tiles:].reshape(txt.shape), txt)


def _torch_grads(wl, q, k, v, do, kv_idx, kv_cnt):
    f = lambda a: torch.from_numpy(si.bf16_bits_to_f32(a).astype(np.float64))
    qt, kt, vt = (f(a).requires_grad_(True) for a in (q, k, v))
    mask = np.stack([np.stack([_token_mask(wl, kv_idx, kv_cnt, b, h) for h in range(wl.heads)])
                     for b in range(wl.batch)])
    s = torch.matmul(qt, kt.transpose(-1, -2)) * oracle.default_scale(wl)
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vt)
    (o * f(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("name", ["joint-tiny", "joint-partial", "t64-grid", "t64-partial"])
def test_backward_matches_torch_autograd(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    sel = oracle.select(wl, q, k)
    dq, dk, dv = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    tq, tk, tv = _torch_grads(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        for b in range(wl.batch):
            for h in range(wl.heads):
                got = _rows_to_tokens(wl, mine, b, h)
                r = ref[b, h]
                assert np.max(np.abs(got - r)) <= 1e-12 * max(1.0, np.max(np.abs(r)))

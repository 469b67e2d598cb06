"""GPU parity of every step of the SSTA forward against the CPU oracle, through
the C ABI, on small workloads that span several blocks, odd block grids,
batch > 1, exact score ties, window 0, k = 0, k above the block count, and
grids the block size does not divide (partial edge blocks), joint video +
text sequences (text blocks always kept, text query blocks dense), and
64-token (4x4x4) blocks.

Bit-exact: tile copies (both layouts), block means, Score_r, Score_i, top-k
ids, kept lists, bitmasks.  Within tolerance (tests/_helpers.py): the bf16
attention output and its LSE.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from _helpers import (O_MAX_ABS, O_MEAN_ABS, bits, check_lse, compare_o, geom_of, o_rows,
                      params_of, sample_rows, to_dev)

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "grid32-w1-k2", "grid32-w0-k3", "grid32-w0-k0", "dup-ties", "ragged", "wide-k",
         "partial", "partial-x", "joint-tiny", "joint-grid32", "joint-partial", "t64-grid",
         "t64-partial"]
_cache = {}


def _case(name, flags=0):
    key = (name, flags)
    if key not in _cache:
        wl = si.ALL[name]
        q, k, v = si.make_qkv(wl)
        sel = oracle.select(wl, q, k, flags)
        _cache[key] = (wl, q, k, v, sel)
    return _cache[key]


def _plan(wl, flags=0, bitmask=True, dense=False, fused_io=True):
    import video_dit_block_tile_amd as m
    return m.SstaPlan(geom_of(wl), params_of(wl, flags), bitmask=bitmask, dense=dense,
                      fused_io=fused_io)


@pytest.mark.parametrize("name", SMALL)
def test_tile_pool_bit_exact(name):
    import video_dit_block_tile_amd as m
    wl, q, k, v, sel = _case(name)
    g = geom_of(wl)
    for x in (q, v):
        xd = to_dev(x)
        tok = torch.empty(wl.batch, wl.heads, wl.n_rows, wl.tile_tokens, 128, dtype=torch.bfloat16,
                          device="cuda")
        dim = torch.empty(wl.batch, wl.heads, wl.n_rows, 128, wl.tile_tokens,
                          dtype=torch.bfloat16, device="cuda")
        pooled = torch.empty(wl.batch, wl.heads, wl.n_tiles, 128, dtype=torch.float32,
                             device="cuda")
        m.ssta_tile_pool(g, xd, tok, m.LAYOUT_TOKEN_MAJOR, pooled)
        m.ssta_tile_pool(g, xd, dim, m.LAYOUT_DIM_MAJOR, None)
        torch.cuda.synchronize()
        ref = oracle.permute(wl, x)
        assert np.array_equal(bits(tok), ref)
        assert np.array_equal(bits(dim), np.swapaxes(ref, -1, -2))
        assert np.array_equal(pooled.cpu().numpy().view(np.uint32),
                              oracle.pool(wl, x).view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "ragged", "partial", "partial-x", "joint-tiny",
                                  "joint-partial", "t64-grid", "t64-partial"])
def test_unpermute_inverts(name):
    import video_dit_block_tile_amd as m
    wl, q, k, v, sel = _case(name)
    g = geom_of(wl)
    xt = to_dev(oracle.permute(wl, k))
    out = torch.empty(wl.batch, wl.heads, wl.seq_len, 128, dtype=torch.bfloat16, device="cuda")
    m.ssta_tile_unpermute(g, xt, out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), k)


@pytest.mark.parametrize("name", SMALL)
def test_scores_bit_exact(name):
    import video_dit_block_tile_amd as m
    wl, q, k, v, sel = _case(name)
    g, p = geom_of(wl), params_of(wl)
    qp = torch.from_numpy(sel["q_pooled"]).cuda()
    kp = torch.from_numpy(sel["k_pooled"]).cuda()
    sc = torch.empty(wl.batch, wl.heads, wl.n_tiles, wl.n_tiles, dtype=torch.float32,
                     device="cuda")
    red = torch.empty(wl.batch, wl.heads, wl.n_tiles, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.ssta_workspace_bytes(g, p), dtype=torch.uint8, device="cuda")
    m.ssta_scores(g, p, qp, kp, sc, red, ws)
    torch.cuda.synchronize()
    assert np.array_equal(red.cpu().numpy().view(np.uint32), sel["red"].view(np.uint32))
    got = sc.cpu().numpy().view(np.uint32)
    want = sel["scores"].view(np.uint32)
    bad = np.count_nonzero(got != want)
    assert bad == 0, "%d of %d scores differ" % (bad, got.size)


@pytest.mark.parametrize("name", SMALL)
def test_selection_and_lists_bit_exact(name):
    wl, q, k, v, sel = _case(name)
    plan = _plan(wl)
    plan.tile_pool(to_dev(q), to_dev(k), to_dev(v))
    plan.select()
    torch.cuda.synchronize()
    assert np.array_equal(plan.topk_idx.cpu().numpy(), sel["topk"])
    assert np.array_equal(plan.kv_cnt.cpu().numpy(), sel["kv_cnt"])
    assert np.array_equal(plan.kv_idx.cpu().numpy(), sel["kv_idx"])
    assert np.array_equal(plan.bitmask.cpu().numpy().view(np.uint32), sel["bitmask"])


def _check_attention(wl, q, k, v, sel, plan, rows):
    o_ref, lse_ref = oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"], rows)
    mx, mean = compare_o(o_rows(wl, plan.o, rows), o_ref)
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, (mx, mean)
    lse = plan.lse.cpu().numpy().reshape(-1, wl.tile_tokens)[rows]
    ratio = check_lse(wl, q, k, rows, lse, lse_ref)
    print("[%s] %d rows: O max-abs %.3e mean-abs %.3e, LSE error / bound %.3f"
          % (wl.name, len(rows), mx, mean, ratio), flush=True)
    return mx, mean


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("fused", [True, False])
def test_attention_vs_oracle(name, fused):
    wl, q, k, v, sel = _case(name)
    plan = _plan(wl, fused_io=fused)
    plan.run(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    rows = np.arange(wl.batch * wl.heads * wl.n_rows, dtype=np.int64)   # every row
    _check_attention(wl, q, k, v, sel, plan, rows)
    if not fused:
        # the tile-major output holds the same bits as the token-major one
        o_tok = bits(plan.o).reshape(wl.batch * wl.heads, wl.seq_len, 128)
        o_til = bits(plan.o_t).reshape(-1, wl.tile_tokens, 128)
        for row in rows[:8]:
            bh, i = divmod(int(row), wl.n_rows)
            toks = np.array([oracle.tile_to_token(wl, i, r) for r in range(wl.tile_tokens)])
            there = toks >= 0        # an edge block of a ragged grid holds zero rows
            assert np.array_equal(o_tok[bh][toks[there]], o_til[row][there])
            assert not o_til[row][~there].any()


@pytest.mark.parametrize("name", ["grid32-w1-k2", "ragged", "dup-ties", "wide-k", "partial",
                                  "partial-x", "joint-tiny", "joint-grid32", "joint-partial",
                                  "t64-grid", "t64-partial"])
def test_fused_io_matches_materialised(name):
    """Gathering blocks inside the kernel gives the same bits as permuting first."""
    wl, q, k, v, sel = _case(name)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    a = _plan(wl, fused_io=True)
    b = _plan(wl, fused_io=False)
    a.run(qd, kd, vd)
    b.run(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(a.o, b.o)
    assert torch.equal(a.lse, b.lse)


def test_attention_unit_values():
    wl, q, k, v, sel = _case("ragged")
    plan = _plan(wl)
    ones = np.full_like(v, 0x3F80)
    plan.run(to_dev(q), to_dev(k), to_dev(ones))
    torch.cuda.synchronize()
    o = plan.o.float().cpu().numpy()
    assert np.max(np.abs(o - 1.0)) <= 1e-2


def test_attention_wide_score_range():
    """Keys of the later frames multiplied by 32 (exact in bf16): scores jump by
    far more than 32 in the log2 domain in the middle of rows and the early
    blocks' weights fall to nothing, so the online softmax raises its running
    max and rescales O mid-row; the result must still match the oracle."""
    wl = si.ALL["ragged"]
    q, k, v = si.make_qkv(wl)
    kf = si.bf16_bits_to_f32(k).reshape(wl.batch, wl.heads, wl.T, wl.H * wl.W, 128).copy()
    kf[:, :, wl.T // 2:] *= 32.0
    k2 = (np.ascontiguousarray(kf, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    k2 = k2.reshape(k.shape)
    assert np.array_equal(si.bf16_bits_to_f32(k2).reshape(kf.shape), kf)
    sel = oracle.select(wl, q, k2)
    plan = _plan(wl)
    plan.run(to_dev(q), to_dev(k2), to_dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(plan.kv_idx.cpu().numpy(), sel["kv_idx"])
    rows = sample_rows(wl, 48, seed=3)
    _check_attention(wl, q, k2, v, sel, plan, rows)


def test_dense_equals_all_kept():
    wl, q, k, v, sel = _case("wide-k")            # top-k clamps to every block
    assert np.all(sel["kv_cnt"] == wl.n_tiles)
    sparse = _plan(wl)
    dense = _plan(wl, dense=True)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sparse.run(qd, kd, vd)
    dense.run(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(sparse.o, dense.o)
    assert torch.equal(sparse.lse, dense.lse)


def test_t64_dense_equals_all_kept():
    """64-token blocks with top-k covering every block: the sparse run over
    full kept lists, the dense run (no lists) and the oracle's dense attention
    agree -- bit for bit between the two runs, within the bars against the
    oracle on every row."""
    base = si.ALL["t64-grid"]
    wl = base.with_(name="t64-grid-all", topk=base.n_tiles)
    q, k, v = si.make_qkv(wl)
    sel = oracle.select(wl, q, k)
    assert np.all(sel["kv_cnt"] == wl.n_tiles)
    sparse = _plan(wl)
    dense = _plan(wl, dense=True)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sparse.run(qd, kd, vd)
    dense.run(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(sparse.o, dense.o)
    assert torch.equal(sparse.lse, dense.lse)
    rows = np.arange(wl.batch * wl.heads * wl.n_rows, dtype=np.int64)
    _check_attention(wl, q, k, v, sel, dense, rows)


def test_deterministic():
    wl, q, k, v, sel = _case("dup-ties")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    a = _plan(wl)
    b = _plan(wl)
    a.run(qd, kd, vd)
    b.run(qd, kd, vd)
    torch.cuda.synchronize()
    for x, y in ((a.o, b.o), (a.lse, b.lse), (a.kv_idx, b.kv_idx), (a.topk_idx, b.topk_idx)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["grid32-w1-k2", "t64-grid"])
@pytest.mark.parametrize("flags", [oracle.COMBINE_AND, oracle.TOPK_EXCLUDE_WINDOW,
                                   oracle.COMBINE_AND | oracle.TOPK_EXCLUDE_WINDOW])
def test_flag_variants(name, flags):
    wl, q, k, v, sel = _case(name, flags)
    plan = _plan(wl, flags)
    plan.run(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(plan.topk_idx.cpu().numpy(), sel["topk"])
    assert np.array_equal(plan.kv_cnt.cpu().numpy(), sel["kv_cnt"])
    assert np.array_equal(plan.kv_idx.cpu().numpy(), sel["kv_idx"])
    rows = np.arange(wl.batch * wl.heads * wl.n_tiles)
    o_ref, lse_ref = oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"], rows)
    o_t = o_rows(wl, plan.o, rows)
    mx, mean = compare_o(o_t, o_ref)
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS
    lse = plan.lse.cpu().numpy().reshape(-1, wl.tile_tokens)
    check_lse(wl, q, k, rows, lse, lse_ref)
    if flags == oracle.COMBINE_AND | oracle.TOPK_EXCLUDE_WINDOW:
        # selection outside the window intersected with the window: nothing is kept
        assert np.all(sel["kv_cnt"] == 0) and np.all(o_t == 0)


def test_joint_text_with_nothing_kept():
    """AND of the window with a selection outside it keeps no clip block; clip
    rows still attend to the text, and text rows to everything."""
    flags = oracle.COMBINE_AND | oracle.TOPK_EXCLUDE_WINDOW
    wl, q, k, v, sel = _case("joint-grid32", flags)
    assert np.all(sel["kv_cnt"] == 0)
    plan = _plan(wl, flags)
    plan.run(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(plan.kv_cnt.cpu().numpy(), sel["kv_cnt"])
    rows = np.arange(wl.batch * wl.heads * wl.n_rows)
    _check_attention(wl, q, k, v, sel, plan, rows)
    assert np.all(np.isfinite(plan.lse.cpu().numpy()[..., :wl.n_tiles, :]))


def test_device_argument_errors():
    import video_dit_block_tile_amd as m
    wl = si.ALL["tiny"]
    g = geom_of(wl)
    x = torch.zeros(wl.batch, wl.heads, wl.n_tokens, 128, dtype=torch.bfloat16, device="cuda")
    pooled = torch.empty(wl.batch * wl.heads * wl.n_tiles * 128 + 1, dtype=torch.float32,
                         device="cuda")
    lib = m.load()
    import ctypes
    rc = lib.ssta_tile_pool(ctypes.byref(g), x.data_ptr(), None, 0, pooled.data_ptr() + 4, None)
    assert rc == -3                                   # SSTA_ERR_ALIGN, nothing launched
    rc = lib.ssta_tile_pool(ctypes.byref(g), x.data_ptr(), None, 0, None, None)
    assert rc == -1                                   # no output requested
    torch.cuda.synchronize()


def test_calibrate_mfma_runs():
    """The matrix-core calibration loop computes what it claims: with all
    operands 1.0 every product adds 16 to each accumulator element, so each
    thread's sink value is 4 chains x 16 elements x 16 x iters."""
    import video_dit_block_tile_amd as m
    grid, iters = 8, 100
    ops = torch.ones(256, 8, dtype=torch.bfloat16, device="cuda")
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    m.ssta_calibrate_mfma(ops, sink, grid, iters)
    torch.cuda.synchronize()
    assert torch.all(sink == 4 * 16 * 16 * iters)


@pytest.mark.parametrize("name", ["grid32-w1-k2", "ragged", "partial"])
def test_similarity_only_variant(name):
    """lambda = 1, beta = 0 through every GPU step: scores, ids and lists bit-exact."""
    import video_dit_block_tile_amd as m
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    sel = oracle.select(wl, q, k, lambda_=1.0, beta=0.0)
    plan = m.SstaPlan(geom_of(wl), params_of(wl, lambda_=1.0, beta=0.0), bitmask=True)
    plan.run(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(plan.topk_idx.cpu().numpy(), sel["topk"])
    assert np.array_equal(plan.kv_idx.cpu().numpy(), sel["kv_idx"])
    assert np.array_equal(plan.kv_cnt.cpu().numpy(), sel["kv_cnt"])
    rows = sample_rows(wl, 24, seed=4)
    _check_attention(wl, q, k, v, sel, plan, rows)


@pytest.mark.parametrize("text_len", [0, 70])
def test_t64_half_units_without_keys(text_len):
    """With 64-token blocks two waves share each query group, one 32-key half
    of every unit each.  Here every query block keeps only blocks of the last
    block row in t, which holds 2 of its 4 frames: the second half of each
    such unit has no key at all, so one wave of each pair sees no real key in
    its first unit (or, without text, in any); every third query block keeps
    nothing.  O and LSE of every row against the oracle."""
    import video_dit_block_tile_amd as m
    wl = si.ALL["t64-partial"].with_(text_len=text_len)
    q, k, v = si.make_qkv(wl)
    nt, ny, nx = wl.tile_grid
    n = wl.n_tiles
    last = np.arange((nt - 1) * ny * nx, n, dtype=np.int32)
    assert len(last) >= 3
    for j in last:     # positions 32..63 of these blocks lie past the clip
        assert all(oracle.tile_to_token(wl, int(j), r) < 0 for r in range(32, 64))
    kv_idx = np.full((wl.batch, wl.heads, n, len(last)), -1, np.int32)
    kv_cnt = np.zeros((wl.batch, wl.heads, n), np.int32)
    for bh in range(wl.batch * wl.heads):
        b, h = divmod(bh, wl.heads)
        for i in range(n):
            if i % 3 == 2:
                continue
            keep = np.sort(np.roll(last, i + bh)[: 1 + (i + bh) % len(last)])
            kv_idx[b, h, i, :len(keep)] = keep
            kv_cnt[b, h, i] = len(keep)
    g, p = geom_of(wl), params_of(wl)
    o = torch.zeros(wl.batch, wl.heads, wl.seq_len, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.batch, wl.heads, wl.n_rows, wl.tile_tokens, dtype=torch.float32,
                      device="cuda")
    m.ssta_attention_fwd_tokens(g, p, to_dev(q), to_dev(k), to_dev(v),
                                torch.from_numpy(kv_idx).cuda(), torch.from_numpy(kv_cnt).cuda(),
                                o, lse)
    torch.cuda.synchronize()
    rows = np.arange(wl.batch * wl.heads * wl.n_rows)
    o_ref, lse_ref = oracle.attention(wl, q, k, v, kv_idx, kv_cnt, rows)
    mx, mean = compare_o(o_rows(wl, o, rows), o_ref)
    ratio = check_lse(wl, q, k, rows, lse.cpu().numpy().reshape(-1, wl.tile_tokens)[rows],
                      lse_ref)
    print("[t64 half units, text %d] O max-abs %.3e mean-abs %.3e, LSE error / bound %.3f"
          % (text_len, mx, mean, ratio), flush=True)
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, (mx, mean)

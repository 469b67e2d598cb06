"""Oracle pins for Topk (Step 2), the sliding-tile window (Step 3) and the
mask combination into kept-block lists (Step 4).

Pinned against Python brute force (full sorts, set algebra over all block
pairs) and the closed-form window size.
"""
import itertools

import numpy as np
import pytest

import oracle
import synthetic_inputs as si


def _brute_topk(row, k, exclude=()):
    cand = [j for j in range(len(row)) if j not in exclude]
    return sorted(sorted(cand, key=lambda j: (-float(row[j]), j))[:k])


@pytest.mark.parametrize("name", ["grid32-w1-k2", "ragged", "dup-ties", "wide-k"])
def test_topk_brute_force(name):
    wl = si.ALL[name]
    out = oracle.select(wl, si.generate(wl, 0), si.generate(wl, 1))
    sc, tk = out["scores"], out["topk"]
    k = min(wl.topk, wl.n_tiles)
    assert tk.shape[-1] == k
    for b, h, i in itertools.product(range(wl.batch), range(wl.heads), range(wl.n_tiles)):
        assert tk[b, h, i].tolist() == _brute_topk(sc[b, h, i], k)


def test_topk_ties_take_lower_index():
    wl = si.Workload("t", 1, 1, 2, 16, 32, tile=(2, 8, 8), win=(0, 0, 0))
    rng = np.random.default_rng(3)
    sc = rng.integers(0, 4, size=(1, 1, 8, 8)).astype(np.float32) / 4
    sc[0, 0, 0, :] = 0.5
    sc[0, 0, 1, :] = [0.0, -0.0, 0.0, -0.0, 0.0, -0.0, 0.0, -0.0]  # -0 == +0
    tk = oracle.topk(wl, sc, 3)
    assert tk[0, 0, 0].tolist() == [0, 1, 2]
    assert tk[0, 0, 1].tolist() == [0, 1, 2]
    for i in range(8):
        assert tk[0, 0, i].tolist() == _brute_topk(sc[0, 0, i], 3)


def test_topk_clamp():
    wl = si.ALL["wide-k"]
    assert oracle.k_eff(wl) == wl.n_tiles
    sc = np.random.default_rng(4).standard_normal((1, 2, 45, 45)).astype(np.float32)
    tk = oracle.topk(wl, sc)
    assert np.array_equal(tk, np.broadcast_to(np.arange(45, dtype=np.int32), tk.shape))
    assert oracle.topk(wl, sc, 0).shape[-1] == 0


def test_topk_exclude_window():
    wl = si.ALL["grid32-w1-k2"]
    sc = np.random.default_rng(5).standard_normal((1, 2, 32, 32)).astype(np.float32)
    tk = oracle.topk(wl, sc, 4, flags=oracle.TOPK_EXCLUDE_WINDOW)
    for h, i in itertools.product(range(2), range(32)):
        w = set(oracle.window(wl, i).tolist())
        assert tk[0, h, i].tolist() == _brute_topk(sc[0, h, i], 4, w)


def _closed_form_size(c, w, n):
    return min(c + w, n - 1) - max(c - w, 0) + 1


@pytest.mark.parametrize("name,win", [("720p-5s", (1, 1, 1)), ("ragged", (1, 0, 2)),
                                      ("tiny", (1, 1, 1)), ("480p-short", (0, 2, 3))])
def test_window_closed_form_and_brute_force(name, win):
    wl = si.ALL[name]
    nt, ny, nx = wl.tile_grid
    coords = np.array([(t, y, x) for t in range(nt) for y in range(ny) for x in range(nx)])
    sizes = []
    for i in range(wl.n_tiles):
        w = oracle.window(wl, i, win)
        ti, yi, xi = coords[i]
        size = (_closed_form_size(ti, win[0], nt) * _closed_form_size(yi, win[1], ny) *
                _closed_form_size(xi, win[2], nx))
        assert len(w) == size
        brute = np.nonzero(np.all(np.abs(coords - coords[i]) <= np.array(win), axis=1))[0]
        assert w.tolist() == brute.tolist()
        sizes.append(size)
    if name == "720p-5s":
        assert max(sizes) == 27 and min(sizes) == 8     # interior 3x3x3, corner 2x2x2


@pytest.mark.parametrize("name", ["grid32-w1-k2", "grid32-w0-k3", "grid32-w0-k0", "ragged",
                                  "dup-ties", "tiny"])
def test_union_lists(name):
    wl = si.ALL[name]
    out = oracle.select(wl, si.generate(wl, 0), si.generate(wl, 1))
    kv_idx, kv_cnt, bm, tk = out["kv_idx"], out["kv_cnt"], out["bitmask"], out["topk"]
    mk = oracle.max_kept(wl)
    assert kv_idx.shape[-1] == mk
    n = wl.n_tiles
    for b, h, i in itertools.product(range(wl.batch), range(wl.heads), range(n)):
        want = sorted(set(oracle.window(wl, i).tolist()) | set(tk[b, h, i].tolist()))
        c = kv_cnt[b, h, i]
        assert kv_idx[b, h, i, :c].tolist() == want
        assert np.all(kv_idx[b, h, i, c:] == -1)
        bits = [j for j in range(n) if (bm[b, h, i, j // 32] >> (j % 32)) & 1]
        assert bits == want
        if wl.topk == 0:
            assert want == oracle.window(wl, i).tolist()


def test_and_lists():
    wl = si.ALL["grid32-w1-k2"]
    q, k = si.generate(wl, 0), si.generate(wl, 1)
    out = oracle.select(wl, q, k, flags=oracle.COMBINE_AND)
    tk = out["topk"]
    for h, i in itertools.product(range(wl.heads), range(wl.n_tiles)):
        want = sorted(set(oracle.window(wl, i).tolist()) & set(tk[0, h, i].tolist()))
        c = out["kv_cnt"][0, h, i]
        assert out["kv_idx"][0, h, i, :c].tolist() == want


@pytest.mark.parametrize("name", ["grid32-w1-k2", "ragged"])
def test_similarity_only_sampling(name):
    """lambda = 1, beta = 0 (the similarity-only variant): Score_i equals Score_s
    exactly, and the kept ids are the k most query-similar key blocks, checked
    against cosines recomputed in fp64 wherever the k-th gap is not a near tie."""
    wl = si.ALL[name]
    q, k = si.generate(wl, 0), si.generate(wl, 1)
    out = oracle.select(wl, q, k, lambda_=1.0, beta=0.0)
    qh, kh = out["q_hat"], out["k_hat"]
    gs = oracle.scores(qh, kh, out["red"] * 0.0, 1.0, 0.0)
    assert np.array_equal(out["scores"].view(np.uint32), gs.view(np.uint32))
    qp = oracle.pool(wl, q).astype(np.float64)
    kp = oracle.pool(wl, k).astype(np.float64)
    cos = np.einsum("bhid,bhjd->bhij", qp / np.linalg.norm(qp, axis=-1, keepdims=True),
                    kp / np.linalg.norm(kp, axis=-1, keepdims=True))
    kk = min(wl.topk, wl.n_tiles)
    checked = 0
    for b, h, i in itertools.product(range(wl.batch), range(wl.heads), range(wl.n_tiles)):
        row = cos[b, h, i]
        order = np.argsort(-row, kind="stable")
        if kk < wl.n_tiles and row[order[kk - 1]] - row[order[kk]] < 1e-5:
            continue
        assert out["topk"][b, h, i].tolist() == sorted(order[:kk].tolist())
        checked += 1
    assert checked > 0.9 * wl.batch * wl.heads * wl.n_tiles

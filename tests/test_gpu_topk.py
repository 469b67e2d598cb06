"""GPU parity of the per-row top-k on long rows, through the C ABI.

Step 2 of SSTA keeps, for each query block, the k key blocks of highest
importance Score_i ("HunyuanVideo 1.5 Technical Report" summary page, section
"SSTA: Selective and Sliding Tile Attention", Step 2; ties go to the lowest
block id, the oracle's reading).  The kernel finds each row's k-th largest
score bit by bit and, once few keys can still be selected, continues on a
compact copy of them.  The rows here hold 900 key blocks, so that every branch
runs: k below 64, between 64 and 192 and above 192, k at and beyond the row
length, the window excluded, and exact ties at the k-th score, both where the
compact copy is taken and where it is not.

Inputs are seeded synthetic block means (the pooled q and k the scoring takes);
the expected ids are the oracle's top-k of the oracle's Score_i on the same
means.  Bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from _helpers import geom_of

pytestmark = pytest.mark.gpu

# 15 x 6 x 10 = 900 blocks of 2 x 8 x 8 tokens
WL = si.Workload("topk-long", 1, 2, 30, 48, 80, topk=48, seed=41)
N = 900


def _random_means(seed):
    rng = np.random.default_rng(seed)
    qp = rng.standard_normal((1, 2, N, 128)).astype(np.float32)
    kp = rng.standard_normal((1, 2, N, 128)).astype(np.float32)
    return qp, kp


def _tied_means(seed):
    """30 key blocks aligned with every query, 40 zero key blocks and the rest
    opposed: in every row the zero blocks score exactly alike (their cosine is
    0 and their redundancy the exact mean of (n - 1) halves), between the
    aligned and the opposed ones."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal(128).astype(np.float32)
    qp = (base + 0.3 * rng.standard_normal((1, 2, N, 128))).astype(np.float32)
    kp = (-base + 0.3 * rng.standard_normal((1, 2, N, 128))).astype(np.float32)
    ids = rng.permutation(N)
    aligned, zero = ids[:30], ids[30:70]
    kp[:, :, aligned] = (base + 0.3 * rng.standard_normal((1, 2, 30, 128))).astype(np.float32)
    kp[:, :, zero] = 0.0
    return qp, kp, aligned, zero


def _oracle_topk(qp, kp, k, flags):
    qh, kh = oracle.normalize(qp), oracle.normalize(kp)
    red = oracle.redundancy(kh)
    sc = oracle.scores(qh, kh, red)
    return sc, oracle.topk(WL, sc, topk=k, flags=flags)


def _gpu_topk(qp, kp, k, flags):
    import video_dit_block_tile_amd as m
    g = geom_of(WL)
    p = m.make_params(win=WL.win, topk=k, flags=flags)
    width = m.ssta_topk_width(g, p)
    out = torch.full((1, 2, N, width), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.ssta_workspace_bytes(g, p), dtype=torch.uint8, device="cuda")
    m.ssta_score_select(g, p, torch.from_numpy(qp).cuda(), torch.from_numpy(kp).cuda(), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("flags", [0, oracle.TOPK_EXCLUDE_WINDOW])
@pytest.mark.parametrize("k", [1, 48, 64, 65, 100, 192, 193, 400, 899, 900, 1000])
def test_topk_long_rows(k, flags):
    qp, kp = _random_means(7)
    _, want = _oracle_topk(qp, kp, k, flags)
    got = _gpu_topk(qp, kp, k, flags)
    assert got.shape == want.shape
    bad = np.count_nonzero(got != want)
    assert bad == 0, "%d of %d ids differ (k=%d, flags=%d)" % (bad, got.size, k, flags)


@pytest.mark.parametrize("k", [20, 30, 48, 70, 71, 100, 300])
def test_topk_exact_ties(k):
    qp, kp, aligned, zero = _tied_means(11)
    sc, want = _oracle_topk(qp, kp, k, 0)
    # the zero blocks do tie in every row, below every aligned block
    z = sc[..., zero]
    assert (z == z[..., :1]).all()
    assert (sc[..., aligned].min(axis=-1) > z[..., 0]).all()
    got = _gpu_topk(qp, kp, k, 0)
    bad = np.count_nonzero(got != want)
    assert bad == 0, "%d of %d ids differ (k=%d)" % (bad, got.size, k)
    if 30 < k < 70:
        # the k-th score is the tied one: the lowest-id zero blocks fill the rest
        kept = np.sort(zero)[: k - 30]
        row = got[0, 0, 0]
        assert set(kept) <= set(row.tolist()) and not set(np.sort(zero)[k - 30:]) & set(row)


def test_topk_all_equal():
    """Every key block the same unit vector: all the key-key products are
    exactly 1, so every Score_r and, in each row, every Score_i are equal and
    every row keeps the k lowest ids."""
    rng = np.random.default_rng(5)
    qp = rng.standard_normal((1, 2, N, 128)).astype(np.float32)
    kp = np.zeros((1, 2, N, 128), np.float32)
    kp[..., 3] = 2.0
    for k in (48, 300):
        _, want = _oracle_topk(qp, kp, k, 0)
        got = _gpu_topk(qp, kp, k, 0)
        assert np.array_equal(got, want)
        assert (got[..., :k] == np.arange(k)).all()


@pytest.mark.parametrize("shape", [(30, 48, 80), (60, 48, 80), (8, 128, 136)])
def test_scores_long_rows(shape):
    """Score_r and Score_i bit-exact on rows of 900, 1800 and 1088 key blocks:
    several groups of 128 key blocks, the last one partial (the key-key tiles
    that hold it are computed transposed, and the waves past the last block
    skip their products)."""
    import video_dit_block_tile_amd as m
    T, H, W = shape
    wl = si.Workload("scores-long", 1, 2, T, H, W, topk=48, seed=43)
    n = wl.n_tiles
    rng = np.random.default_rng(n)
    qp = rng.standard_normal((1, 2, n, 128)).astype(np.float32)
    kp = (0.5 + rng.standard_normal((1, 2, n, 128))).astype(np.float32)
    kp[0, 1, 5] = 0.0                      # a zero mean stays zero after normalising
    qh, kh = oracle.normalize(qp), oracle.normalize(kp)
    red_want = oracle.redundancy(kh)
    sc_want = oracle.scores(qh, kh, red_want)
    g = geom_of(wl)
    p = m.make_params(win=wl.win, topk=48)
    sc = torch.empty(1, 2, n, n, dtype=torch.float32, device="cuda")
    red = torch.empty(1, 2, n, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.ssta_workspace_bytes(g, p), dtype=torch.uint8, device="cuda")
    m.ssta_scores(g, p, torch.from_numpy(qp).cuda(), torch.from_numpy(kp).cuda(), sc, red, ws)
    torch.cuda.synchronize()
    assert np.array_equal(red.cpu().numpy().view(np.uint32), red_want.view(np.uint32))
    bad = np.count_nonzero(sc.cpu().numpy().view(np.uint32) != sc_want.view(np.uint32))
    assert bad == 0, "%d of %d scores differ" % (bad, sc_want.size)

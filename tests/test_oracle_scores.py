"""Oracle pins for Step 2 scoring: normalisation, Score_s, Score_r, Score_i.

Pinned against hand-derived exact cases (orthonormal and duplicated block
vectors, whose cosines are exactly 0 or 1), an algebraic identity for the
redundancy evaluated in fp64, and an fp64 evaluation of the score formula.
"""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si

F = np.float32
LAM, BETA = oracle.DEFAULT_LAMBDA, oracle.DEFAULT_BETA


def test_default_weights():
    # lambda_ = 0.9 and the redundancy weight 1 - lambda_, as fp32 values.
    assert LAM == F(0.9) and BETA == F(0.1)


def test_normalize_exact_cases():
    p = np.zeros((3, 8), F)
    p[0, :2] = [3, 4]                 # norm 5: 3/5 and 4/5 correctly rounded
    p[1, :4] = 1                      # norm 2: every entry exactly 0.5
    out = oracle.normalize(p)
    assert out[0, 0] == F(3) / F(5) and out[0, 1] == F(4) / F(5)
    assert np.all(out[0, 2:] == 0)
    assert np.array_equal(out[1, :4], np.full(4, 0.5, F)) and np.all(out[1, 4:] == 0)
    assert np.all(out[2] == 0)        # a zero vector stays zero (no NaN)


def test_normalize_unit_norm():
    rng = np.random.default_rng(1)
    p = rng.standard_normal((50, 128)).astype(F)
    out = oracle.normalize(p).astype(np.float64)
    assert np.allclose(np.linalg.norm(out, axis=1), 1.0, atol=1e-6)
    assert np.allclose(out, p / np.linalg.norm(p.astype(np.float64), axis=1, keepdims=True),
                       atol=1e-6)


def _redundancy_case():
    """Key blocks 0..4 all equal e0, blocks 5, 6, 7 are e1, e2, e3."""
    k = np.zeros((1, 1, 8, 16), F)
    k[0, 0, :5, 0] = 1
    k[0, 0, 5, 1] = k[0, 0, 6, 2] = k[0, 0, 7, 3] = 1
    return k


def test_redundancy_worked_case():
    kh = oracle.normalize(_redundancy_case())
    red = oracle.redundancy(kh)[0, 0]
    # copies: four other copies (cos 1 -> 1.0) and three orthogonal blocks (-> 0.5)
    assert np.all(red[:5] == F(5.5) / F(7))
    # unique blocks: seven orthogonal blocks -> 3.5 / 7
    assert np.all(red[5:] == F(0.5))


def test_score_worked_case_prefers_unique_blocks():
    kh = oracle.normalize(_redundancy_case())
    q = np.zeros((1, 1, 8, 16), F)
    q[..., :4] = 1                    # cosine 0.5 with every key block
    qh = oracle.normalize(q)
    red = oracle.redundancy(kh)
    sc = oracle.scores(qh, kh, red)[0, 0]
    g = F(0.75)                       # (0.5 + 1) / 2
    want_copy = F(LAM * g) - F(BETA * (F(5.5) / F(7)))
    want_unique = F(LAM * g) - F(BETA * F(0.5))
    assert np.all(sc[:, :5] == want_copy) and np.all(sc[:, 5:] == want_unique)
    wl = si.Workload("w", 1, 1, 2, 16, 32, tile=(2, 8, 8), win=(0, 0, 0), topk=3)
    assert wl.n_tiles == 8
    assert oracle.topk(wl, sc[None, None], 3)[0, 0, 0].tolist() == [5, 6, 7]
    # fourth pick: the five tied copies, lowest block id wins
    assert oracle.topk(wl, sc[None, None], 4)[0, 0, 0].tolist() == [0, 5, 6, 7]


def test_similarity_orientation_and_ties():
    n, D = 12, 16
    sigma = [(i + 3) % n for i in range(n)]         # not an involution
    k = np.eye(n, D, dtype=F)[None, None]
    q = np.eye(n, D, dtype=F)[sigma][None, None]
    qh, kh = oracle.normalize(q), oracle.normalize(k)
    red = oracle.redundancy(kh)
    assert np.all(red == F(0.5))
    sc = oracle.scores(qh, kh, red)[0, 0]
    for i in range(n):
        for j in range(n):
            g = F(1.0) if j == sigma[i] else F(0.5)
            assert sc[i, j] == F(LAM * g) - F(BETA * F(0.5))
    wl = si.Workload("w", 1, 1, 2, 8, 96, tile=(2, 8, 8), win=(0, 0, 0))
    assert wl.n_tiles == n
    t1 = oracle.topk(wl, sc[None, None], 1)[0, 0]
    assert t1[:, 0].tolist() == sigma
    t2 = oracle.topk(wl, sc[None, None], 2)[0, 0]
    for i in range(n):
        low = 0 if sigma[i] != 0 else 1
        assert sorted(t2[i].tolist()) == sorted({sigma[i], low})


def test_redundancy_identity_fp64():
    wl = si.ALL["ragged"]
    kp = oracle.pool(wl, si.generate(wl, 1))
    kh = oracle.normalize(kp)
    red = oracle.redundancy(kh).astype(np.float64)
    k64 = kh.astype(np.float64)
    n = k64.shape[-2]
    tot = k64.sum(axis=-2, keepdims=True)
    off = (k64 * tot).sum(-1) - (k64 * k64).sum(-1)       # sum over i != j of khat_i . khat_j
    want = (off + (n - 1)) / 2.0 / (n - 1)
    assert np.max(np.abs(red - want)) < 2e-6


def test_redundancy_many_blocks():
    """280 key blocks (three groups of the two-level sum): the value still meets
    the fp64 identity, and the order is the stated one: group partials from 0
    in ascending i, added in ascending group order (replayed in float32; the
    plain ascending sum differs from it in the last bits somewhere)."""
    wl = si.ALL["480p-5s"].with_(heads=2)
    kh = oracle.normalize(oracle.pool(wl, si.generate(wl, 1)))
    red = oracle.redundancy(kh)
    k64 = kh.astype(np.float64)
    n = k64.shape[-2]
    assert n == 280
    tot = k64.sum(axis=-2, keepdims=True)
    off = (k64 * tot).sum(-1) - (k64 * k64).sum(-1)
    assert np.max(np.abs(red - (off + (n - 1)) / 2.0 / (n - 1))) < 2e-6
    u = ((np.einsum("hid,hjd->hij", kh[0].astype(np.float32), kh[0].astype(np.float32))
          + np.float32(1)) * np.float32(0.5)).astype(np.float32)
    grouped = np.empty((2, n), np.float32)
    plain = np.empty((2, n), np.float32)
    for h in range(2):
        for j in range(n):
            col = u[h, :, j].copy()
            col[j] = 0.0                                   # +0 in place of the diagonal
            s = np.float32(0)
            for g0 in range(0, n, 128):
                part = np.float32(0)
                for x in col[g0:g0 + 128]:
                    part = np.float32(part + x)
                s = np.float32(s + part)
            grouped[h, j] = s / np.float32(n - 1)
            t = np.float32(0)
            for x in col:
                t = np.float32(t + x)
            plain[h, j] = t / np.float32(n - 1)
    # the dot products here come from numpy, not the oracle's fmaf chain, so
    # compare the sum orders through their rounding, not bit for bit
    assert np.max(np.abs(grouped - red[0])) < 1e-6
    assert not np.array_equal(grouped, plain)


def test_scores_fp64_formula():
    wl = si.ALL["ragged"]
    q, k = si.generate(wl, 0), si.generate(wl, 1)
    qh = oracle.normalize(oracle.pool(wl, q))
    kh = oracle.normalize(oracle.pool(wl, k))
    red = oracle.redundancy(kh)
    sc = oracle.scores(qh, kh, red).astype(np.float64)
    g = (np.einsum("bhid,bhjd->bhij", qh.astype(np.float64), kh.astype(np.float64)) + 1) / 2
    want = float(LAM) * g - float(BETA) * red.astype(np.float64)[:, :, None, :]
    assert np.max(np.abs(sc - want)) < 2e-6


def test_similarity_only_weights():
    """lambda = 1, beta = 0: the ranking is the ranking of the cosines."""
    wl = si.ALL["grid32-w1-k2"]
    q, k = si.generate(wl, 0), si.generate(wl, 1)
    qh = oracle.normalize(oracle.pool(wl, q))
    kh = oracle.normalize(oracle.pool(wl, k))
    red = oracle.redundancy(kh)
    sc = oracle.scores(qh, kh, red, F(1.0), F(0.0))
    cos = np.einsum("bhid,bhjd->bhij", qh.astype(np.float64), kh.astype(np.float64))
    top = oracle.topk(wl, sc, 3)
    for b in range(wl.batch):
        for h in range(wl.heads):
            for i in range(wl.n_tiles):
                c = cos[b, h, i]
                order = np.argsort(-c, kind="stable")
                if c[order[2]] - c[order[3]] > 1e-5:
                    assert sorted(order[:3].tolist()) == top[b, h, i].tolist()


@pytest.mark.parametrize("name", ["grid32-w1-k2", "ragged"])
def test_score_ranges(name):
    wl = si.ALL[name]
    out = oracle.select(wl, si.generate(wl, 0), si.generate(wl, 1))
    assert np.all(out["red"] >= 0) and np.all(out["red"] <= 1)
    # g in [0, 1] and red in [0, 1]: score in [-beta, lambda] up to rounding
    assert np.all(out["scores"] >= -BETA - 1e-6) and np.all(out["scores"] <= LAM + 1e-6)

"""Oracle pins for Step 1 (3D block partition) and the block means of Step 2.

Pinned against: the pages' worked token count, a numpy reshape/transpose
formulation of the same partition (an independent construction), brute-force
bijection checks, fp64 means, and closed-form special inputs.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _reshape_tiles(wl, x):
    """Tile-major view built with reshape/transpose only."""
    B, h, D = wl.batch, wl.heads, wl.head_dim
    tt, th, tw = wl.tile
    nt, ny, nx = wl.tile_grid
    g = x.reshape(B, h, nt, tt, ny, th, nx, tw, D)
    g = g.transpose(0, 1, 2, 4, 6, 3, 5, 7, 8)
    return g.reshape(B, h, nt * ny * nx, tt * th * tw, D)


def test_pages_worked_example():
    with open(os.path.join(GOLDEN, "pages_worked_numbers.json")) as f:
        ex = json.load(f)
    wl = si.Workload("pages", 1, 1, ex["latent_frames"], ex["latent_height"], ex["latent_width"],
                     tile=(1, 1, 1), head_dim=4)
    assert wl.n_tokens == ex["tokens"]
    assert oracle.n_tiles(wl) == ex["tokens"]           # 1x1x1 blocks: one per token
    assert abs(ex["tokens"] ** 2 / ex["attention_matrix_entries_approx"] - 1) < 0.005
    wl4 = si.Workload("pages4", 1, 1, 8, 8, 8, tile=tuple(ex["example_block"]), head_dim=4)
    assert oracle.tile_tokens(wl4) == ex["example_block_tokens"]
    assert oracle.n_tiles(wl4) == 8


@pytest.mark.parametrize("name", ["tiny", "grid32-w1-k2", "ragged"])
def test_permute_matches_reshape(name):
    wl = si.ALL[name]
    x = si.generate(wl, 0)
    assert np.array_equal(oracle.permute(wl, x), _reshape_tiles(wl, x))


@pytest.mark.parametrize("shape,tile", [((4, 6, 10), (2, 3, 5)), ((3, 4, 4), (1, 2, 4)),
                                        ((2, 16, 16), (2, 8, 8))])
def test_token_tile_bijection(shape, tile):
    wl = si.Workload("bij", 1, 1, *shape, tile=tile, head_dim=4)
    N = wl.n_tokens
    seen = set()
    for n in range(N):
        t, r = oracle.token_to_tile(wl, n)
        assert 0 <= t < oracle.n_tiles(wl) and 0 <= r < oracle.tile_tokens(wl)
        assert oracle.tile_to_token(wl, t, r) == n
        seen.add((t, r))
    assert len(seen) == N
    # Block ids are row-major over the block grid: the block of token (t,y,x).
    T, H, W = shape
    for n in range(0, N, 7):
        t, y, x = n // (H * W), (n // W) % H, n % W
        want = ((t // tile[0]) * (H // tile[1]) + y // tile[1]) * (W // tile[2]) + x // tile[2]
        assert oracle.token_to_tile(wl, n)[0] == want


def test_pool_against_fp64_mean():
    wl = si.ALL["ragged"]
    x = si.generate(wl, 1)
    got = oracle.pool(wl, x).astype(np.float64)
    want = _reshape_tiles(wl, si.bf16_bits_to_f32(x)).astype(np.float64).mean(axis=3)
    scale = np.abs(si.bf16_bits_to_f32(x)).max()
    assert np.max(np.abs(got - want)) <= 128 * 2.0 ** -24 * scale * 4


def test_pool_exact_cases():
    wl = si.ALL["grid32-w1-k2"]
    rng = np.random.default_rng(0)
    # Small integers are exact in bf16 and their fp32 sums are exact, so the mean is too.
    vals = rng.integers(-8, 9, size=(wl.batch, wl.heads, wl.n_tokens, wl.head_dim))
    x = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = oracle.pool(wl, x)
    want = _reshape_tiles(wl, vals.astype(np.float64)).sum(axis=3) / 128.0
    assert np.array_equal(got.astype(np.float64), want)
    # A block whose rows are all equal pools to that row exactly.
    row = si.generate(wl, 2)[0, 0, 0]
    xc = np.broadcast_to(row, x.shape).copy()
    got = oracle.pool(wl, xc)
    assert np.array_equal(got[0, 0, 5], si.bf16_bits_to_f32(row))

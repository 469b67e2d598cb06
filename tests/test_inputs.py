"""The seeded input generator: Philox known answers, determinism, distributions."""
import json
import os

import numpy as np

import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        c = [int(x, 16) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["out"]]
        assert list(si.philox4x32_10(c, k)) == want


def test_deterministic_and_distinct_streams():
    wl = si.ALL["grid32-w1-k2"]
    a = si.generate(wl, 0)
    b = si.generate(wl, 0)
    c = si.generate(wl, 1)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    d = si.generate(wl.with_(seed=wl.seed + 1), 0)
    assert not np.array_equal(a, d)


def test_iid_moments():
    wl = si.CONFIGS["tiny"]
    x = si.bf16_bits_to_f32(si.generate(wl, 0)).astype(np.float64)
    assert abs(x.mean()) < 0.02
    assert abs(x.std() - 1.0) < 0.02


def test_field_moments():
    # sin(.) has variance 1/2; noise std 0.5 adds 1/4.
    wl = si.CONFIGS["480p-short"]
    x = si.bf16_bits_to_f32(si.generate(wl, 2)).astype(np.float64)
    assert abs(x.mean()) < 0.02
    assert abs(x.var() - 0.75) < 0.02


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x3E00], dtype=np.uint16)
    f = si.bf16_bits_to_f32(bits)
    assert f.tolist()[:4] == [1.0, -1.0, 0.0, -0.0]
    assert np.isinf(f[4]) and f[5] == 0.125


def test_duplicated_tiles_are_copies():
    wl = si.ALL["dup-ties"]
    x = si.generate(wl, 1)
    tt, th, tw = wl.tile
    _, ny, nx = wl.tile_grid
    xg = x.reshape(wl.batch, wl.heads, wl.T, wl.H, wl.W, wl.head_dim)

    def tile(t):
        a, b, c = t // (ny * nx), (t // nx) % ny, t % nx
        return xg[:, :, a * tt:(a + 1) * tt, b * th:(b + 1) * th, c * tw:(c + 1) * tw]

    for src, dst in wl.dup_tiles:
        assert np.array_equal(tile(src), tile(dst))

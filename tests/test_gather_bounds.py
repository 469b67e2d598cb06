"""Address model of the attention kernels' token-row gathers (CPU).

The forward and backward kernels gather each key unit's token rows straight
into LDS with buffer loads whose address is a scalar base (the unit's block
origin) plus a per-lane offset.  The hardware range check covers only the
per-lane offset, so every scalar base must itself stay inside the head's
tokens.  This test restates the kernels' address arithmetic (block origins,
the bit-field in-block offsets, the chunk swizzle, the redirect of rows whose
position does not exist) and checks, for the ragged, joint and 64-token
shapes, that

  * every address of every lane of every unit lies inside the head's
    S * 256 bytes,
  * a row whose position exists is read from that position's own token, and
  * a row whose position does not exist is read from the block's first token.

Block geometry follows the pages' Step 1 (3D blocks of tile_t x tile_h x
tile_w tokens, numbered row-major; "HunyuanVideo 1.5 Technical Report"
summary page, section "SSTA: Selective and Sliding Tile Attention").
"""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si

SHAPES = ["partial", "partial-x", "ragged", "joint-tiny", "joint-partial", "joint-grid32",
          "t64-partial", "t64-grid", "720p-10s-latent", "720p-10s-text"]


class Model:
    """The kernels' gather arithmetic for one workload."""

    def __init__(self, wl):
        self.wl = wl
        self.tt, self.th, self.tw = wl.tile
        self.R = wl.tile_tokens
        self.nt, self.ny, self.nx = wl.tile_grid
        self.N, self.S, self.L = wl.n_tokens, wl.seq_len, wl.text_len
        self.n = wl.n_tiles
        self.ltw = int(np.log2(self.tw))
        self.lth = int(np.log2(self.th))

    def origin(self, j):
        """First token of clip block j (block_origin32)."""
        bt, rem = divmod(j, self.ny * self.nx)
        by, bx = divmod(rem, self.nx)
        return ((bt * self.tt) * self.wl.H + by * self.th) * self.wl.W + bx * self.tw

    def ibo(self, r):
        """Token offset of in-block position r (in_block_offset)."""
        r = np.asarray(r)
        it = r >> (self.ltw + self.lth)
        iy = (r >> self.ltw) & (self.th - 1)
        ix = r & (self.tw - 1)
        return (it * self.wl.H + iy) * self.wl.W + ix

    def token(self, j, pos):
        """Token of position pos of block j, -1 where none exists (the oracle's map)."""
        return np.array([oracle.tile_to_token(self.wl, j, int(p)) for p in pos])


def forward_addresses(m, j, p):
    """Byte addresses (within one head) and destination rows of the forward's
    K and V gathers of unit p (64 keys) of block j; 64 rows, per lane chunk."""
    R = m.R
    waves, loads = R // 32, 16 // (R // 32)
    lanes = np.arange(64)
    pos = 64 * p + np.arange(64)
    tok = m.token(j, pos)
    valid = tok >= 0
    text = j >= m.n
    part = not valid.all()
    origin = (m.N + (j - m.n) * R) if text else m.origin(j)
    half = (64 if text else int(m.ibo(64))) * 256 if p else 0
    so = origin * 256 + (0 if part else half)
    out = {}
    for kv, swz in (("k", lambda r: r & 15), ("v", lambda r: 4 * (r & 3))):
        addr = np.zeros((64, 16), dtype=np.int64)   # row -> the 16 chunk addresses
        for w in range(waves):
            for mm in range(loads):
                b = loads * w + mm
                row = 4 * b + (lanes >> 4)
                chunk = (lanes & 15) ^ swz(row)
                vo = m.ibo(row) * 256 + (chunk << 4)
                if text:
                    vo = row * 256 + (chunk << 4)
                if part:
                    vo = np.where(valid[row], vo + half, vo & 255)
                addr[row, lanes & 15] = so + vo
        out[kv] = addr
    return out, tok


def backward_addresses(m, j, p):
    """The same for the backward's 32-row units (unit p of block j)."""
    R = m.R
    waves, loads = R // 32, 8 // (R // 32)
    lanes = np.arange(64)
    pos = 32 * p + np.arange(32)
    tok = m.token(j, pos)
    valid = tok >= 0
    text = j >= m.n
    part = not valid.all()
    origin = (m.N + (j - m.n) * R) if text else m.origin(j)
    half = (32 * p if text else int(m.ibo(32 * p))) * 256
    so = origin * 256 + (0 if part else half)
    addr = np.zeros((32, 16), dtype=np.int64)
    swz = lambda r: ((r & 3) << 2) | ((r >> 2) & 3)
    for w in range(waves):
        for mm in range(loads):
            b = loads * w + mm
            row = 4 * b + (lanes >> 4)
            chunk = (lanes & 15) ^ swz(row)
            vo = m.ibo(row) * 256 + (chunk << 4)
            if text:
                vo = row * 256 + (chunk << 4)
            if part:
                vo = np.where(valid[row], vo + half, vo & 255)
            addr[row, lanes & 15] = so + vo
    return addr, tok


def check_unit(m, addr, tok, first):
    rows = addr >> 8
    assert addr.min() >= 0 and addr.max() + 16 <= m.S * 256, (addr.min(), addr.max())
    # each row's 16 chunks come from one token row, and cover its 256 bytes once
    assert (rows == rows[:, :1]).all()
    assert (np.sort(addr & 255, axis=1) == np.arange(0, 256, 16)).all()
    want = np.where(tok >= 0, tok, first)
    assert np.array_equal(rows[:, 0], want)


@pytest.mark.parametrize("name", SHAPES)
def test_gather_addresses(name):
    wl = si.ALL[name]
    m = Model(wl)
    # every partial block (ragged edge, text tail) and a sample of full ones
    blocks = [j for j in range(m.n) if (m.token(j, np.arange(m.R)) < 0).any()]
    blocks += list(range(0, m.n, max(1, m.n // 16))) + list(range(m.n, wl.n_rows))
    checked = 0
    for j in sorted(set(blocks)):
        first = m.N + (j - m.n) * m.R if j >= m.n else m.origin(j)
        for p in range(m.R // 64):
            out, tok = forward_addresses(m, j, p)
            check_unit(m, out["k"], tok, first)
            check_unit(m, out["v"], tok, first)
        for p in range(m.R // 32):
            addr, tok = backward_addresses(m, j, p)
            check_unit(m, addr, tok, first)
        checked += 1
    assert checked > 0


def test_unit_past_the_grid_exists():
    """The case the redirect is for: at 61 latent frames the last block row holds
    one frame, so its second 64-key unit has no position at all, and the first
    token of that unit would lie past the clip."""
    wl = si.ALL["720p-10s-latent"]
    m = Model(wl)
    j = m.n - 1
    assert (m.token(j, 64 + np.arange(64)) < 0).all()
    assert m.origin(j) + m.ibo(64) >= m.N
    out, tok = forward_addresses(m, j, 1)
    assert (out["k"] >> 8 == m.origin(j)).all() and (out["v"] >> 8 == m.origin(j)).all()

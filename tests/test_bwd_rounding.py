"""The backward's rounding model against the fp64 oracle (CPU).

tests/_bwd_emulation.py repeats the roundings of the GPU backward (bf16 P and
dS entering the products, D from the bf16 output, fp32 sums, bf16 outputs).
Its distance to the fp64 oracle (the gradient of the attention equation of
the "HunyuanVideo 1.5 Technical Report" summary page, section "SSTA:
Selective and Sliding Tile Attention", with the kept lists fixed) is what a
correct kernel shows.  These tests check that

  * every emulated element lies inside the per-element bound the GPU tests
    assert (tests/_helpers.py, bwd_bounds), so the bound's derivation covers
    the roundings the kernels make, and
  * the emulated mean error is the small, rounding-sized fraction of the
    gradients' mean magnitude that the GPU tests' mean-error bar is scaled
    from (the bar there is a multiple of the emulation on the same rows).
"""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from _bwd_emulation import bf16, emulate
from _helpers import bwd_bounds, token_rows

CASES = ["grid32-w1-k2", "partial", "joint-tiny", "t64-grid"]


def forward_outputs(wl, q, k, v, sel):
    """The forward's outputs as the GPU stores them: O as bf16 bits in token
    order, LSE in fp32 (both rounded from the oracle's fp64)."""
    rows = np.arange(wl.batch * wl.heads * wl.n_rows)
    o, lse = oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"], rows)
    ob = np.zeros((wl.batch * wl.heads, wl.seq_len, 128), np.float32)
    tok = token_rows(wl, rows)
    bh = rows // wl.n_rows
    there = tok >= 0
    ob[np.broadcast_to(bh[:, None], tok.shape)[there], tok[there]] = \
        bf16(o.astype(np.float32))[there]
    bits = (ob.view(np.uint32) >> 16).astype(np.uint16)
    return bits.reshape(wl.batch, wl.heads, wl.seq_len, 128), lse.astype(np.float32)


@pytest.mark.parametrize("name", CASES)
def test_emulated_roundings_within_bounds(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    sel = oracle.select(wl, q, k)
    o_bits, lse = forward_outputs(wl, q, k, v, sel)
    rows = np.arange(wl.batch * wl.heads * wl.n_rows)
    ref = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    em = emulate(wl, q, k, v, do, o_bits, lse, sel["kv_idx"], sel["kv_cnt"], rows, rows)
    bounds = bwd_bounds(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"], rows, rows)
    for label, e, r, b in zip(("dq", "dk", "dv"), em, ref, bounds):
        err = np.abs(e - r)
        there = b > 0
        assert not err[~there].any(), label      # rows that must be exactly zero
        ratio = float((err[there] / b[there]).max())
        rel = float(err.mean() / np.abs(r).mean())
        print("[%s] %s: emulated error / bound %.3f, mean error %.4f%% of mean |ref|"
              % (name, label, ratio, 100 * rel))
        assert ratio <= 1.0, label
        # rounding-sized: above zero (the model rounds) and far below a percent
        assert 0.0 < rel < 5e-3, label


def test_emulation_detects_a_dropped_term():
    """The model is sensitive: dropping D (the dO.O term) moves the gradients
    far outside the bounds."""
    import _bwd_emulation as em_mod
    wl = si.ALL["grid32-w1-k2"]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    sel = oracle.select(wl, q, k)
    o_bits, lse = forward_outputs(wl, q, k, v, sel)
    zero_o = np.zeros_like(o_bits)           # D = 0
    rows = np.arange(wl.batch * wl.heads * wl.n_rows)
    ref = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    dq, _, _ = em_mod.emulate(wl, q, k, v, do, zero_o, lse, sel["kv_idx"], sel["kv_cnt"], rows,
                              rows[:1])
    bq, _, _ = bwd_bounds(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"], rows, rows[:1])
    there = bq > 0
    assert (np.abs(dq - ref[0])[there] / bq[there]).max() > 1.0

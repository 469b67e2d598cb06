"""GPU parity of the attention backward (dq, dk, dv with the kept lists held
fixed) against the fp64 oracle, through the C ABI.

Bars (bf16 inputs and outputs; probabilities and dS enter the products as
bf16, D = dO . O uses the bf16 O, accumulation in fp32): every element within
the per-element bound that _helpers.bwd_bounds derives from that arithmetic
(worst case, all rounding errors of one sign), and per tensor max-abs error
<= 2e-2 * max|ref|.  Where the rounding model of tests/_bwd_emulation.py is
run on the same rows (fed the GPU forward's own O and LSE), the mean error
must also stay within 1.5 times the model's mean error: the kernels make the
model's roundings, and only add fp32 summation-order and exp2 differences
that are far smaller.  Empty rows give exactly zero dq.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from _helpers import bwd_bounds, geom_of, params_of, sample_rows, to_dev, token_rows

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2


def _rows_of(wl, t, rows):
    """fp32 [len(rows), R, 128] block rows of a token-major device tensor."""
    x = t.float().cpu().numpy().reshape(wl.batch * wl.heads, wl.seq_len, 128)
    tok = token_rows(wl, rows)
    bh = np.asarray(rows) // wl.n_rows
    out = x[bh[:, None], np.maximum(tok, 0)].astype(np.float64)
    out[tok < 0] = 0.0
    return out


MEAN_VS_MODEL = 1.5


def _check(name, got, ref, bound, model=None):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    rmx, rmean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    there = bound > 0
    ratio = float((err[there] / bound[there]).max()) if there.any() else 0.0
    extra = ""
    if model is not None:
        model_mean = float(np.abs(model - ref).mean())
        extra = ", model mean-abs %.3e (GPU / model %.3f)" % (
            model_mean, mean / model_mean if model_mean > 0 else 0.0)
    print("  %s: max-abs %.3e (ref max %.3e), mean-abs %.3e (ref mean %.3e), "
          "largest error / bound %.3f%s" % (name, mx, rmx, mean, rmean, ratio, extra), flush=True)
    assert mx <= MAX_REL * rmx, name
    assert ratio <= 1.0 and not err[~there].any(), name
    if model is not None:
        assert mean <= MEAN_VS_MODEL * model_mean + 1e-6 * rmean, name


def _model(wl, q, k, v, do, plan, kv_idx, kv_cnt, q_rows, k_rows):
    """The rounding model on these rows, fed the GPU forward's O and LSE."""
    from _bwd_emulation import emulate
    o_bits = plan.o.view(torch.int16).cpu().numpy().view(np.uint16)
    return emulate(wl, q, k, v, do, o_bits, plan.lse.cpu().numpy(), kv_idx, kv_cnt, q_rows,
                   k_rows)


def _run(wl, q, k, v, do, flags=0, dense=False):
    import video_dit_block_tile_amd as m
    g, p = geom_of(wl), params_of(wl, flags)
    plan = m.SstaPlan(g, p, dense=dense)
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    plan.run(qd, kd, vd)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(m.ssta_attention_bwd_workspace_bytes(g), dtype=torch.uint8, device="cuda")
    idx, cnt = (None, None) if dense else (plan.kv_idx, plan.kv_cnt)
    m.ssta_attention_bwd(g, p, qd, kd, vd, plan.o, dod, plan.lse, idx, cnt, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return plan, dq, dk, dv


# small cases that also run the rounding model (it costs seconds per case on the CPU)
MODELLED = ("grid32-w1-k2", "partial", "joint-partial", "t64-partial")


@pytest.mark.parametrize("name", ["tiny", "grid32-w1-k2", "ragged", "dup-ties", "partial",
                                  "partial-x", "joint-tiny", "joint-grid32", "joint-partial",
                                  "t64-grid", "t64-partial"])
def test_backward_vs_oracle(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    print("[%s]" % name, flush=True)
    plan, dq, dk, dv = _run(wl, q, k, v, do)
    sel = oracle.select(wl, q, k)
    assert np.array_equal(plan.kv_idx.cpu().numpy(), sel["kv_idx"])
    rows = np.arange(wl.batch * wl.heads * wl.n_rows)
    rq, rk, rv = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    bq, bk, bv = bwd_bounds(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"], rows, rows)
    mq = mk = mv = None
    if name in MODELLED:
        mq, mk, mv = _model(wl, q, k, v, do, plan, sel["kv_idx"], sel["kv_cnt"], rows, rows)
    _check("dq", _rows_of(wl, dq, rows), rq, bq, mq)
    _check("dk", _rows_of(wl, dk, rows), rk, bk, mk)
    _check("dv", _rows_of(wl, dv, rows), rv, bv, mv)


@pytest.mark.parametrize("name", ["grid32-w1-k2", "t64-grid"])
def test_backward_partial_lists(name):
    """Window AND top-k: some rows and key blocks keep nothing, the rest few
    blocks, so the key-block lists are short, uneven or empty."""
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    flags = oracle.COMBINE_AND
    print("[%s AND]" % name, flush=True)
    plan, dq, dk, dv = _run(wl, q, k, v, do, flags)
    sel = oracle.select(wl, q, k, flags)
    assert np.array_equal(plan.kv_cnt.cpu().numpy(), sel["kv_cnt"])
    assert np.array_equal(plan.kv_idx.cpu().numpy(), sel["kv_idx"])
    cnt = sel["kv_cnt"].reshape(-1)
    assert (cnt == 0).any() and (cnt > 0).any()
    rows = np.arange(wl.batch * wl.heads * wl.n_rows)
    rq, rk, rv = oracle.attention_bwd(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"])
    bq, bk, bv = bwd_bounds(wl, q, k, v, do, sel["kv_idx"], sel["kv_cnt"], rows, rows)
    _check("dq", _rows_of(wl, dq, rows), rq, bq)
    _check("dk", _rows_of(wl, dk, rows), rk, bk)
    _check("dv", _rows_of(wl, dv, rows), rv, bv)


def test_backward_dense_equals_all_kept():
    wl = si.ALL["wide-k"]                          # every block kept
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    _, dq1, dk1, dv1 = _run(wl, q, k, v, do)
    _, dq2, dk2, dv2 = _run(wl, q, k, v, do, dense=True)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)


def test_backward_empty_rows():
    wl = si.ALL["grid32-w1-k2"]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    flags = oracle.COMBINE_AND | oracle.TOPK_EXCLUDE_WINDOW   # nothing kept anywhere
    plan, dq, dk, dv = _run(wl, q, k, v, do, flags)
    assert int(plan.kv_cnt.sum()) == 0
    assert not dq.any() and not dk.any() and not dv.any()


@pytest.mark.parametrize("name", ["720p-10s", "720p-10s-latent", "720p-10s-text",
                                  "720p-10s-t64"])
def test_backward_full_size_sampled(name):
    wl = si.ALL[name]
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    print("[%s] inputs ready" % name, flush=True)
    plan, dq, dk, dv = _run(wl, q, k, v, do)
    print("[%s] gpu done" % name, flush=True)
    kv_idx, kv_cnt = plan.kv_idx.cpu().numpy(), plan.kv_cnt.cpu().numpy()
    rows = sample_rows(wl, 2, seed=5)[:10]
    krows = rows[:4]
    if wl.text_len:
        # dq of one text query block (it attends to every token) beside clip
        # rows; dk, dv of a joint sequence are checked in full on the small
        # joint cases (here each key block would need every text query's
        # dense row in fp64)
        rows = np.concatenate([rows[:6], [wl.n_tiles]])
        krows = rows[:0]
    rq, rk, rv = oracle.attention_bwd(wl, q, k, v, do, kv_idx, kv_cnt, rows, krows)
    print("[%s] oracle done" % name, flush=True)
    bq, bk, bv = bwd_bounds(wl, q, k, v, do, kv_idx, kv_cnt, rows, krows)
    mq, mk, mv = _model(wl, q, k, v, do, plan, kv_idx, kv_cnt, rows, krows)
    print("[%s] bounds and model done" % name, flush=True)
    _check("dq", _rows_of(wl, dq, rows), rq, bq, mq)
    if len(krows):
        _check("dk", _rows_of(wl, dk, krows), rk, bk, mk)
        _check("dv", _rows_of(wl, dv, krows), rv, bv, mv)


@pytest.mark.parametrize("name", ["ragged", "joint-partial", "t64-partial", "720p-5s"])
def test_same_head_in_two_launch_configurations(name):
    """Every step is per (batch, head), so a head's results must not depend
    on the launch it runs in.  Each head of a multi-head batch is run again
    alone, as a one-head batch: the grids differ (other workgroup counts,
    XCD slices, and dK/dV order of key blocks), the block means, ids, kept
    lists, O, LSE, dq, dk and dv of that head must be bit-identical."""
    import video_dit_block_tile_amd as m
    wl = si.ALL[name]
    if name == "720p-5s":
        wl = wl.with_(heads=2)
    q, k, v = si.make_qkv(wl)
    do = si.generate(wl, 3)
    print("[%s] %d heads" % (name, wl.batch * wl.heads), flush=True)
    plan, dq, dk, dv = _run(wl, q, k, v, do)
    one = wl.with_(batch=1, heads=1)
    for bh in range(wl.batch * wl.heads):
        b, h = divmod(bh, wl.heads)
        pick = lambda x: np.ascontiguousarray(x[b:b + 1, h:h + 1])
        p1, dq1, dk1, dv1 = _run(one, pick(q), pick(k), pick(v), pick(do))
        for label, x_all, x_one in (("topk", plan.topk_idx, p1.topk_idx),
                                    ("kv_idx", plan.kv_idx, p1.kv_idx),
                                    ("kv_cnt", plan.kv_cnt, p1.kv_cnt),
                                    ("o", plan.o, p1.o), ("lse", plan.lse, p1.lse),
                                    ("dq", dq, dq1), ("dk", dk, dk1), ("dv", dv, dv1)):
            assert torch.equal(x_all[b:b + 1, h:h + 1], x_one), (label, b, h)

"""CPU emulation of the roundings of the attention backward (test helper).

The backward of the block-sparse attention ("HunyuanVideo 1.5 Technical
Report" summary page, section "SSTA: Selective and Sliding Tile Attention":
the attention equation; the distillation paragraph applies SSTA while the
model is trained) computes, for a query a and a kept key b,

  p_ab = exp2(fma(s_ab, scale*log2 e, -lse_a*log2 e)),   s_ab = q_a . k_b,
  D_a = dO_a . O_a            (O the forward's bf16 output),
  dS_ab = p_ab * (dP_ab - D_a),   dP_ab = dO_a . v_b,
  dq_a = scale * sum_b bf16(dS_ab) k_b,  dk_b = scale * sum_a bf16(dS_ab) q_a,
  dv_b = sum_a bf16(p_ab) dO_a,

with bf16 inputs, fp32 sums and bf16 outputs.  This module repeats exactly
those roundings in numpy (float32 sums in numpy's order, which differs from
the matrix cores' only in the order of exact fp32 terms), so its distance to
the fp64 oracle is the error a correct kernel is expected to show.  The GPU
tests compare the kernels' mean error with it; the CPU tests check that its
errors lie inside the per-element bounds the GPU tests assert.
"""
from __future__ import annotations

import numpy as np

import oracle
import synthetic_inputs as si
from _helpers import _row_keys, _token_map

LOG2E = np.float32(1.44269504088896340736)


def bf16(x):
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _f32_dot(a, b):
    return np.matmul(a.astype(np.float32), b.astype(np.float32), dtype=np.float32)


def _probs(Q, K, lse, scale):
    """p = exp2(fma(s, c, -lse2)) in fp32 (the fma as one rounding of the exact
    fp64 value, which holds s*c exactly)."""
    s = _f32_dot(Q, K.T)
    c = np.float32(np.float32(scale) * LOG2E)
    lse2 = (lse.astype(np.float32) * LOG2E).astype(np.float32)
    arg = (s.astype(np.float64) * np.float64(c) - lse2.astype(np.float64)[:, None])
    return np.exp2(arg.astype(np.float32)).astype(np.float32)


def emulate(wl, q, k, v, do, o_bf16, lse, kv_idx, kv_cnt, q_rows, k_rows):
    """Emulated (dq [len(q_rows), R, 128], dk, dv [len(k_rows), R, 128]) in
    float64 holding the emulated bf16 values; o_bf16 is the forward's output
    (bf16 bits, token-major) and lse its fp32 LSE [B, h, n_rows, R]."""
    R = wl.tile_tokens
    scale = np.float32(oracle.default_scale(wl))
    tmap = _token_map(wl)
    sh = (wl.batch, wl.heads, wl.seq_len, 128)
    qf, kf, vf, dof, of = (si.bf16_bits_to_f32(x).reshape(sh) for x in (q, k, v, do, o_bf16))
    lse = np.asarray(lse, dtype=np.float32).reshape(wl.batch, wl.heads, wl.n_rows, R)

    def row_state(b, h, i, keys):
        qt = tmap[i]
        qt = qt[qt >= 0]
        Q, dO, O = qf[b, h, qt], dof[b, h, qt], of[b, h, qt]
        K, V = kf[b, h, keys], vf[b, h, keys]
        pos = np.nonzero(tmap[i] >= 0)[0]
        P = _probs(Q, K, lse[b, h, i, pos], scale)
        D = (dO * O).sum(axis=1, dtype=np.float32)
        dS = (P * (_f32_dot(dO, V.T) - D[:, None])).astype(np.float32)
        return Q, dO, K, P, dS

    dq = np.zeros((len(q_rows), R, 128))
    for a, row in enumerate(q_rows):
        bh, i = divmod(int(row), wl.n_rows)
        b, h = divmod(bh, wl.heads)
        keys = _row_keys(wl, tmap, kv_idx, kv_cnt, b, h, i)
        if keys.size == 0:
            continue
        Q, dO, K, P, dS = row_state(b, h, i, keys)
        there = tmap[i] >= 0
        dq[a, there] = bf16(scale * _f32_dot(bf16(dS), K))
    dk = np.zeros((len(k_rows), R, 128))
    dv = np.zeros((len(k_rows), R, 128))
    for a, row in enumerate(k_rows):
        bh, j = divmod(int(row), wl.n_rows)
        b, h = divmod(bh, wl.heads)
        kt = tmap[j]
        there = kt >= 0
        if j >= wl.n_tiles:
            users = np.arange(wl.n_rows)
        else:
            lists = kv_idx[b, h]
            listed = (lists == j) & (np.arange(lists.shape[1])[None, :] < kv_cnt[b, h][:, None])
            users = np.concatenate([np.nonzero(listed.any(axis=1))[0],
                                    np.arange(wl.n_tiles, wl.n_rows)])
        acc_k = np.zeros((int(there.sum()), 128), np.float32)
        acc_v = np.zeros_like(acc_k)
        for i in users:
            keys = _row_keys(wl, tmap, kv_idx, kv_cnt, b, h, int(i))
            col = {int(t): c for c, t in enumerate(keys)}
            cols = np.array([col[int(t)] for t in kt[there]])
            Q, dO, K, P, dS = row_state(b, h, int(i), keys)
            acc_k += _f32_dot(bf16(dS[:, cols]).T, Q)
            acc_v += _f32_dot(bf16(P[:, cols]).T, dO)
        dk[a, there] = bf16(scale * acc_k)
        dv[a, there] = bf16(acc_v)
    return dq, dk, dv

"""The whole SSTA forward as one sequence of C-ABI calls on one stream.

``SstaPlan`` allocates every buffer once for a geometry (PyTorch is only the
allocator here) and ``run`` enqueues the steps.  Default (``fused_io=True``):

  1. ssta_tile_pool            Q -> block means; K -> block means
                               (Step 1 + Step 2 pooling)
  2. ssta_score_select         block means -> top-k key blocks per query block  (Step 2)
  3. ssta_build_mask           top-k + sliding-tile window -> kept lists  (Steps 3-4)
  4. ssta_attention_fwd_tokens block-sparse attention, gathering each query block
                               and each kept key block (K and V) from token
                               order and writing O in token order  (Step 4)

With ``fused_io=False`` the block gathers are materialised instead: step 1
also writes tile-major Q_t and K_t and dim-major V_t, step 4 is
ssta_attention_fwd, and ssta_tile_unpermute brings O_t back to token order.
Both give bit-identical O.

A geometry with text_len > 0 describes a joint sequence (the clip's tokens,
then the text's): the text is kept out of steps 2-3, and step 4 adds every
text block to each clip row and runs text rows over every block.

(Steps as numbered in the "HunyuanVideo 1.5 Technical Report" summary page,
section "SSTA: Selective and Sliding Tile Attention".)
"""
from __future__ import annotations

import torch

from . import _lib as L


class SstaPlan:
    def __init__(self, geom: L.SstaGeom, params: L.SstaParams, device="cuda",
                 bitmask: bool = False, dense: bool = False, fused_io: bool = True):
        self.geom, self.params, self.dense, self.fused_io = geom, params, dense, fused_io
        g = geom
        dev = torch.device(device)
        n, nr, R, D = g.n_tiles, g.n_rows, g.tile_tokens, g.head_dim
        bh = (g.batch, g.heads)
        if fused_io:
            self.q_t = self.k_t = self.v_t = self.o_t = None
        else:
            self.q_t = torch.empty(bh + (nr, R, D), dtype=torch.bfloat16, device=dev)
            self.k_t = torch.empty_like(self.q_t)
            self.o_t = torch.empty_like(self.q_t)
            self.v_t = torch.empty(bh + (nr, D, R), dtype=torch.bfloat16, device=dev)
        self.o = torch.empty(bh + (g.seq_len, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(bh + (nr, R), dtype=torch.float32, device=dev)
        self.q_pooled = torch.empty(bh + (n, D), dtype=torch.float32, device=dev)
        self.k_pooled = torch.empty_like(self.q_pooled)
        self.width = L.ssta_topk_width(g, params)
        self.max_kept = L.ssta_max_kept(g, params)
        self.topk_idx = torch.empty(bh + (n, self.width), dtype=torch.int32, device=dev)
        self.kv_idx = torch.empty(bh + (n, self.max_kept), dtype=torch.int32, device=dev)
        self.kv_cnt = torch.empty(bh + (n,), dtype=torch.int32, device=dev)
        self.bitmask = (torch.empty(bh + (n, (n + 31) // 32), dtype=torch.int32, device=dev)
                        if bitmask else None)
        self.workspace = torch.empty(L.ssta_workspace_bytes(g, params), dtype=torch.uint8,
                                     device=dev)

    # individual steps -----------------------------------------------------
    def tile_pool(self, q, k, v, stream=None):
        g = self.geom
        self._q, self._k, self._v = q, k, v
        L.ssta_tile_pool(g, q, self.q_t, L.LAYOUT_TOKEN_MAJOR, self.q_pooled, stream)
        L.ssta_tile_pool(g, k, self.k_t, L.LAYOUT_TOKEN_MAJOR, self.k_pooled, stream)
        if not self.fused_io:
            L.ssta_tile_pool(g, v, self.v_t, L.LAYOUT_DIM_MAJOR, None, stream)

    def score_select(self, stream=None):
        """Block scores and per-query-block top-k (Step 2)."""
        if self.width > 0:
            L.ssta_score_select(self.geom, self.params, self.q_pooled, self.k_pooled,
                                self.topk_idx, self.workspace, stream)

    def build_mask(self, stream=None):
        """Window union top-k -> ascending kept lists (Steps 3-4)."""
        L.ssta_build_mask(self.geom, self.params, self.topk_idx, self.kv_idx, self.kv_cnt,
                          self.bitmask, stream)

    def select(self, stream=None):
        self.score_select(stream)
        self.build_mask(stream)

    def attend(self, stream=None, dense=None):
        """Attention for the inputs of the last tile_pool call."""
        dense = self.dense if dense is None else dense
        g, p = self.geom, self.params
        idx, cnt = (None, None) if dense else (self.kv_idx, self.kv_cnt)
        if self.fused_io:
            L.ssta_attention_fwd_tokens(g, p, self._q, self._k, self._v, idx, cnt, self.o,
                                        self.lse, stream)
        else:
            L.ssta_attention_fwd(g, p, self.q_t, self.k_t, self.v_t, idx, cnt, self.o_t,
                                 self.lse, stream)

    def unpermute(self, stream=None):
        """Token-order O (a no-op for the fused path, which writes it directly)."""
        if not self.fused_io:
            L.ssta_tile_unpermute(self.geom, self.o_t, self.o, stream)

    # whole forward --------------------------------------------------------
    def run(self, q, k, v, stream=None):
        """Enqueue the whole forward; returns (o [B,h,S,D] bf16, lse [B,h,n_rows,R] fp32)."""
        self.tile_pool(q, k, v, stream)
        if not self.dense:
            self.select(stream)
        self.attend(stream)
        self.unpermute(stream)
        return self.o, self.lse


def ssta_forward(q, k, v, geom: L.SstaGeom, params: L.SstaParams, dense: bool = False,
                 fused_io: bool = True):
    """One-shot SSTA forward on bf16 [B, h, T*H*W + text_len, 128] device tensors."""
    plan = SstaPlan(geom, params, device=q.device, dense=dense, fused_io=fused_io)
    o, lse = plan.run(q, k, v)
    return o, lse, plan

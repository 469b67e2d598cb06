"""ssta_score_select_noalloc, the scoring entry point that allocates nothing,
against ssta_score_select on the same inputs (GPU, through the C ABI).

Two calls in a row share the library's one scratch array: the first scores a
16-head, 1,800-block batch (several passes of heads through the array), the
second a smaller 2-head, 900-block batch with the window excluded from the
candidates.  Each call's ids must equal, bit for bit, what the workspace entry
point gives on the same means.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from _helpers import geom_of

pytestmark = pytest.mark.gpu

CALLS = [
    (si.Workload("noalloc-large", 1, 16, 60, 48, 80, topk=48, seed=51), 0),     # 1,800 blocks
    (si.Workload("noalloc-small", 1, 2, 30, 48, 80, topk=100, seed=52),
     oracle.TOPK_EXCLUDE_WINDOW),                                             # 900 blocks
]


def _means(wl):
    rng = np.random.default_rng(wl.seed)
    shape = (wl.batch, wl.heads, wl.n_tiles, 128)
    return (torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).cuda(),
            torch.from_numpy((0.3 + rng.standard_normal(shape)).astype(np.float32)).cuda())


def test_noalloc_matches_workspace_entry():
    import video_dit_block_tile_amd as m
    for wl, flags in CALLS:
        print("[noalloc] %s: %d heads x %d blocks, k=%d, flags=%d"
              % (wl.name, wl.batch * wl.heads, wl.n_tiles, wl.topk, flags), flush=True)
        g = geom_of(wl)
        p = m.make_params(win=wl.win, topk=wl.topk, flags=flags)
        qp, kp = _means(wl)
        width = m.ssta_topk_width(g, p)
        shape = (wl.batch, wl.heads, wl.n_tiles, width)
        want = torch.full(shape, -7, dtype=torch.int32, device="cuda")
        ws = torch.empty(m.ssta_workspace_bytes(g, p), dtype=torch.uint8, device="cuda")
        m.ssta_score_select(g, p, qp, kp, want, ws)
        got = torch.full(shape, -7, dtype=torch.int32, device="cuda")
        m.ssta_score_select_noalloc(g, p, qp, kp, got)
        torch.cuda.synchronize()
        w, o = want.cpu().numpy(), got.cpu().numpy()
        assert (w >= -1).all() and (w[..., 0] >= 0).all()
        bad = np.count_nonzero(o != w)
        assert bad == 0, "%s: %d of %d ids differ" % (wl.name, bad, w.size)

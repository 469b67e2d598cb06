"""The whole forward step, and the backward, captured in a HIP graph (through
torch.cuda.graph) and replayed: the library enqueues only kernels on the
caller's stream (no allocation, memset or synchronisation), so a captured
step must reproduce the eager results bit for bit.  Each graph is replayed
several times with eager work and synchronisations in between, then again
after new inputs are copied into the captured buffers."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from _helpers import geom_of, params_of, to_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("name", ["grid32-w1-k2", "joint-partial", "t64-partial"])
def test_forward_step_replays(name):
    import video_dit_block_tile_amd as m
    wl = si.ALL[name]
    q, k, v = (to_dev(x) for x in si.make_qkv(wl))
    g, p = geom_of(wl), params_of(wl)
    plan = m.SstaPlan(g, p)
    eager = m.SstaPlan(g, p)
    graph = _capture(lambda: plan.run(q, k, v))

    def check(ref):
        for a, b in ((plan.o, ref.o), (plan.lse, ref.lse), (plan.kv_idx, ref.kv_idx),
                     (plan.kv_cnt, ref.kv_cnt), (plan.topk_idx, ref.topk_idx)):
            assert torch.equal(a, b)

    eager.run(q, k, v)
    torch.cuda.synchronize()
    for _ in range(3):
        plan.o.zero_()                         # eager work between replays
        plan.kv_cnt.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(eager)
    # new inputs in the captured buffers
    q2, k2, v2 = (to_dev(x) for x in si.make_qkv(wl.with_(seed=wl.seed + 100)))
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    graph.replay()
    eager.run(q2, k2, v2)
    torch.cuda.synchronize()
    check(eager)


def test_backward_replays():
    import video_dit_block_tile_amd as m
    wl = si.ALL["partial"]
    q, k, v = (to_dev(x) for x in si.make_qkv(wl))
    do = to_dev(si.generate(wl, 3))
    g, p = geom_of(wl), params_of(wl)
    plan = m.SstaPlan(g, p)
    plan.run(q, k, v)
    ws = torch.empty(m.ssta_attention_bwd_workspace_bytes(g), dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(q) for _ in range(3)]
    ref = [torch.empty_like(q) for _ in range(3)]

    def bwd(out):
        m.ssta_attention_bwd(g, p, q, k, v, plan.o, do, plan.lse, plan.kv_idx, plan.kv_cnt,
                             out[0], out[1], out[2], ws)

    bwd(ref)
    torch.cuda.synchronize()
    graph = _capture(lambda: bwd(grads))
    for _ in range(3):
        for t in grads:
            t.zero_()
        ws.fill_(0xAB)                         # the workspace holds nothing across calls
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(grads, ref):
            assert torch.equal(a, b)

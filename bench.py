#!/usr/bin/env python3
"""SSTA forward benchmark on one MI355X.

One step = the whole SSTA forward on one batch of synthetic inputs already
resident in HBM: tile/pool Q, K, V -> block scores + top-k -> window/union
lists -> block-sparse attention (-> unpermute O when the block I/O is
materialised).  W untimed warm-up steps, then K timed steps between device
synchronisations.  Prints one JSON line.

  value        effective TFLOP/s on kept blocks over the whole step
               (kept (query block, key block) pairs x 4*128^3 FLOP / step time)
  phase_ms     per phase (tile_pool, score_select, build_mask, attention,
               unpermute): mean, median, p10, p90 over the K steps, from HIP
               events recorded on the launch stream
  phase_rates  algorithmic bytes, GB/s and % of HBM peak per phase (attention:
               the logical K/V block bytes it requests, most served by L2/MALL,
               as a rate only); VALU FLOP and % of the usable (unpacked) fp32
               vector peak for the block scoring
  per_config   the five workload shapes: step and attention time, attention
               TFLOP/s, kept fraction and speedup over the dense path
  materialised_io  the block gather with tile writes and the output
               unpermute (the non-fused path) timed once, with their HBM rate
  cold_cache   steps timed right after overwriting a 512 MB buffer
  roofline     the attention kernel (the dominant kernel): kept FLOP / its
               mean launch time vs the dense bf16 MFMA peak of 2.5 PFLOP/s;
               traffic = HBM bytes per launch from rocprofv3 counters, if they
               were taken on this version of the kernel
  backward     the attention backward (dq, dk, dv) on the same kept lists:
               time, algorithmic TFLOP/s (5 products per kept pair) and
               executed TFLOP/s (7: the dq kernel and the dk/dv kernel each compute S and dP)
  mfma_sustained  the chip's sustained bf16 matrix-core rate on random and on
               constant operands (ssta_calibrate_mfma): under random data the
               power limit holds the clock well below its peak
  speedup vs dense: the same pipeline with every block kept (dense attention)
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSTA fwd effective TFLOP/s on kept blocks (% bf16 MFMA peak) + speedup vs dense"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_VECTOR_TFLOPS = 157.3    # MI355X published fp32 vector peak (packed FMA)
# the fp32 vector rate this build can reach: packed fp32 instructions are
# disabled, so one FMA per lane per cycle: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz
PEAK_FP32_UNPACKED_TFLOPS = 78.6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p-10s")
    ap.add_argument("--dense-steps", type=int, default=2)
    ap.add_argument("--cold-steps", type=int, default=3,
                    help="extra steps, each after overwriting a 512 MB buffer (cold caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=3,
                    help="timed runs of the attention backward (dq, dk, dv) after the forward")
    ap.add_argument("--variant-steps", type=int, default=5,
                    help="timed forward steps of each variant workload (64-token blocks, "
                         "joint text, ragged latent grid); 0 to skip")
    ap.add_argument("--config-steps", type=int, default=5,
                    help="timed forward steps of each of the five workload shapes (per_config; "
                         "dense on the same inputs for the speedup); 0 to skip")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the sustained bf16 matrix-core rate measurement")
    ap.add_argument("--materialised", action="store_true",
                    help="permute Q/K to tile-major and unpermute O in separate kernels "
                         "instead of gathering blocks inside the attention kernel")
    ap.add_argument("--cpu-rows", type=int, default=1800,
                    help="query-block rows of head 0 in the CPU oracle sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 5 times (calibrates "
                         "the HBM byte counters) and exit")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per attention launch measured with rocprofv3 counters")
    return ap.parse_args()


def load_traffic(path, workload, kernel_hash):
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(workload)
    if not ent or ent.get("kernel_source_sha256") != kernel_hash:
        return None           # counters taken on another version of the kernel
    return ent.get("attn_bytes_per_launch")


def kernel_hash():
    import hashlib
    p = os.path.join(ROOT, "video_dit_block_tile_amd", "csrc", "k_attn.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


_SINGLE_CORE = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
import numpy as np
import oracle
import synthetic_inputs as si
wl = si.ALL[sys.argv[2]].with_(heads=1, batch=1)
q, k, v = (np.load(sys.argv[3] + "/%s.npy" % n) for n in "qkv")
rows = np.linspace(0, wl.n_tiles - 1, num=int(sys.argv[4])).astype(np.int64)
t0 = time.perf_counter()
sel = oracle.select(wl, q, k)
t_sel = time.perf_counter() - t0
t0 = time.perf_counter()
oracle.attention(wl, q, k, v, sel["kv_idx"], sel["kv_cnt"], rows)
t_att = time.perf_counter() - t0
print(json.dumps({"t_sel": t_sel, "t_att": t_att,
                  "pairs": int(sel["kv_cnt"].reshape(-1)[rows].sum()), "rows": int(rows.size)}))
"""


def cpu_single_core(wl, q1, k1, v1, rows):
    """The same oracle with one thread (OMP_NUM_THREADS=1 in a child process),
    on head 0's selection and `rows` query blocks."""
    import tempfile
    import subprocess
    import numpy as np
    with tempfile.TemporaryDirectory() as d:
        for name, x in zip("qkv", (q1, k1, v1)):
            np.save(os.path.join(d, name + ".npy"), x)
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-c", _SINGLE_CORE, ROOT, wl.name, d, str(rows)],
                           env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-400:]}
    res = json.loads(r.stdout.strip().splitlines()[-1])
    n = wl.n_tiles
    t = res["t_att"] + res["t_sel"] * res["rows"] / n
    return {"value": res["pairs"] * 4 * wl.tile_tokens ** 2 * 128 / t / 1e12, "unit": "TFLOP/s",
            "cores": 1, "selection_head0_s": round(res["t_sel"], 3),
            "attention_s_per_query_block": round(res["t_att"] / res["rows"], 4),
            "sample": "head 0: full selection (prorated) + fp64 attention of %d query blocks"
                      % res["rows"]}


def cpu_baseline(wl, q, k, v, rows_wanted, single_rows=24):
    """Oracle (as is) on a bounded sample: the selection for head 0 and the
    attention of `rows_wanted` query blocks of head 0, on every host thread,
    then a smaller sample of the same on one thread."""
    import numpy as np
    import oracle

    wl1 = wl.with_(heads=1, batch=1)
    q1, k1, v1 = (np.ascontiguousarray(x[:1, :1]) for x in (q, k, v))
    t0 = time.perf_counter()
    sel = oracle.select(wl1, q1, k1)
    t_sel = time.perf_counter() - t0
    n = wl1.n_tiles
    rows = np.linspace(0, n - 1, num=min(rows_wanted, n)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attention(wl1, q1, k1, v1, sel["kv_idx"], sel["kv_cnt"], rows)
    t_att = time.perf_counter() - t0
    pairs = int(sel["kv_cnt"].reshape(-1)[rows].sum())
    t = t_att + t_sel * len(rows) / n            # selection prorated to the sampled rows
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": pairs * 4 * wl.tile_tokens ** 2 * 128 / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("%s head 0: full selection (%.1f s, prorated to the sampled rows) + fp64 "
                   "attention of %d of %d query blocks (%d kept pairs, %.1f s)"
                   % (wl.name, t_sel, len(rows), n, pairs, t_att)),
        "selection_head0_s": round(t_sel, 3),
        "attention_s_per_query_block": round(t_att / len(rows), 4),
        "single_core": cpu_single_core(wl, q1, k1, v1, single_rows),
    }


def backward_bench(torch, m, si, wl, plan, g, p, qd, kd, vd, pairs, steps):
    """The attention backward (dq, dk, dv for a seeded synthetic dO, kept lists
    of the timed forward) timed with HIP events on the launch stream."""
    import numpy as np
    do = si.generate(wl, 3)
    dod = torch.from_numpy(do.view(np.int16)).view(torch.bfloat16).cuda()
    plan.run(qd, kd, vd)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(m.ssta_attention_bwd_workspace_bytes(g), dtype=torch.uint8, device="cuda")

    def run():
        m.ssta_attention_bwd(g, p, qd, kd, vd, plan.o, dod, plan.lse, plan.kv_idx, plan.kv_cnt,
                             dq, dk, dv, ws)

    run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    # five 128^3 products per kept pair (S, dP, dQ, dK, dV); the kernels also
    # recompute S twice and dP once more
    alg = pairs * 5 * 2 * 128 ** 3
    exe = pairs * 7 * 2 * 128 ** 3
    mean = float(ms.mean())
    return {"ms": {"mean": round(mean, 4), "median": round(float(np.median(ms)), 4),
                   "min": round(float(ms.min()), 4), "max": round(float(ms.max()), 4)},
            "steps": steps,
            "algorithmic_flop": alg, "executed_flop": exe,
            "algorithmic_tflops": round(alg / (mean * 1e-3) / 1e12, 2),
            "executed_tflops": round(exe / (mean * 1e-3) / 1e12, 2),
            "pct_bf16_peak_executed": round(100 * exe / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "dout": "seeded synthetic, same field + noise recipe as Q/K/V"}


VARIANTS = ("720p-10s-t64", "720p-10s-text", "720p-10s-latent")


def block_pairs(wl, plan):
    """(query block, key block) pairs the attention computes, text pairs
    included (text blocks are kept by every clip row; text rows keep all)."""
    n, nt = wl.n_tiles, wl.n_text_blocks
    return (int(plan.kv_cnt.sum().item()) + wl.batch * wl.heads * (n * nt + nt * (n + nt)))


def variant_runs(torch, m, si, steps):
    """Forward step and attention time of the variant workloads (each in
    turn: inputs generated, timed, freed).  TFLOP/s counts whole block pairs,
    4 * R * R * 128 FLOP each (partial edge and text blocks as full)."""
    import numpy as np
    out = {}
    for name in VARIANTS:
        wl = si.ALL[name]
        q, k, v = si.make_qkv(wl)
        dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        qd, kd, vd = dev(q), dev(k), dev(v)
        g = m.make_geom(wl.batch, wl.heads, wl.T, wl.H, wl.W, tile=wl.tile,
                        text_len=wl.text_len)
        p = m.make_params(win=wl.win, topk=wl.topk)
        plan = m.SstaPlan(g, p)
        for _ in range(2):
            plan.run(qd, kd, vd)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in ev:
            e[0].record()
            plan.tile_pool(qd, kd, vd)
            plan.select()
            e[1].record()
            plan.attend()
            e[2].record()
        torch.cuda.synchronize()
        step = float(np.mean([e[0].elapsed_time(e[2]) for e in ev]))
        attn = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        R = wl.tile_tokens
        pairs = block_pairs(wl, plan)
        flop = pairs * 4 * R * R * 128
        out[name] = {"tile": list(wl.tile), "grid": [wl.T, wl.H, wl.W], "text_len": wl.text_len,
                     "topk": wl.topk, "block_pairs": pairs, "step_ms": round(step, 4),
                     "attention_ms": round(attn, 4),
                     "attention_tflops": round(flop / (attn * 1e-3) / 1e12, 2)}
        print("[bench] variant %s: step %.3f ms, attention %.3f ms (%.1f TFLOP/s)"
              % (name, step, attn, out[name]["attention_tflops"]), file=sys.stderr, flush=True)
        del plan, qd, kd, vd
        torch.cuda.empty_cache()
    return out


def per_config_runs(torch, m, si, steps, dense_steps):
    """The five workload shapes in turn (inputs generated, timed, freed): step,
    phase and attention times from HIP events on the launch stream (medians),
    the block means' HBM rate, the scoring's fp32 rate, attention TFLOP/s on
    kept blocks, kept fraction, and the same pipeline with every block kept
    (dense) on the same inputs for the speedup."""
    import numpy as np
    out = {}
    for name, wl in si.CONFIGS.items():
        q, k, v = si.make_qkv(wl)
        dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        qd, kd, vd = dev(q), dev(k), dev(v)
        g = m.make_geom(wl.batch, wl.heads, wl.T, wl.H, wl.W, tile=wl.tile,
                        text_len=wl.text_len)
        p = m.make_params(win=wl.win, topk=wl.topk)
        res = {}
        for mode in ("sparse", "dense"):
            plan = m.SstaPlan(g, p, dense=(mode == "dense"))
            n_steps = steps if mode == "sparse" else dense_steps
            for _ in range(2):
                plan.run(qd, kd, vd)
            torch.cuda.synchronize()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_steps)]
            for e in ev:
                e[0].record()
                plan.tile_pool(qd, kd, vd)
                e[1].record()
                if mode == "sparse":
                    plan.score_select()
                e[2].record()
                if mode == "sparse":
                    plan.build_mask()
                e[3].record()
                plan.attend()
                e[4].record()
            torch.cuda.synchronize()
            med = lambda a, b: float(np.median([e[a].elapsed_time(e[b]) for e in ev]))
            res[mode] = (med(0, 4), med(3, 4),
                         block_pairs(wl, plan) if mode == "sparse" else
                         wl.batch * wl.heads * wl.n_rows * wl.n_rows,
                         (med(0, 1), med(1, 2), med(2, 3)), plan.width)
            del plan
        step, attn, pairs, (t_pool, t_score, t_mask), width = res["sparse"]
        dstep, dattn, dpairs, _, _ = res["dense"]
        flop = pairs * 4 * wl.tile_tokens ** 2 * 128
        tf = flop / (attn * 1e-3) / 1e12
        bh = wl.batch * wl.heads
        # block means: read Q and K, write both fp32 mean arrays
        pool_bytes = 2 * bh * wl.seq_len * 128 * 2 + 2 * bh * wl.n_tiles * 128 * 4
        pool_gbs = pool_bytes / (t_pool * 1e-3) / 1e9
        score_flop = 2 * bh * wl.n_tiles ** 2 * 128 * 2 if width > 0 else 0
        score_tf = score_flop / (t_score * 1e-3) / 1e12 if t_score > 0 else 0.0
        out[name] = {"grid": [wl.T, wl.H, wl.W], "n_tiles": wl.n_tiles, "topk": wl.topk,
                     "kept_pairs": pairs, "kept_fraction": round(pairs / dpairs, 5),
                     "step_ms": round(step, 4),
                     "tile_pool_ms": round(t_pool, 4), "tile_pool_gbs": round(pool_gbs, 1),
                     "tile_pool_pct_hbm": round(100 * pool_gbs / PEAK_HBM_GBS, 1),
                     "score_select_ms": round(t_score, 4),
                     "score_valu_tflops": round(score_tf, 2),
                     "score_pct_fp32_unpacked": round(100 * score_tf / PEAK_FP32_UNPACKED_TFLOPS, 1),
                     "build_mask_ms": round(t_mask, 4),
                     "attention_ms": round(attn, 4),
                     "attention_tflops": round(tf, 2),
                     "pct_bf16_peak_attention": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                     "dense_step_ms": round(dstep, 3), "dense_attention_ms": round(dattn, 3),
                     "speedup_vs_dense_step": round(dstep / step, 3),
                     "speedup_vs_dense_attention": round(dattn / attn, 3)}
        print("[bench] config %s: step %.3f ms, attention %.3f ms (%.1f TFLOP/s), kept %.4f, "
              "dense step %.2f ms" % (name, step, attn, tf, pairs / dpairs, dstep),
              file=sys.stderr, flush=True)
        del qd, kd, vd
        torch.cuda.empty_cache()
    return out


def materialised_io(torch, m, wl, g, qd, reps=5):
    """The block gather that writes tile-major copies (token-major for Q and
    K, dim-major for V; plus the block means) and the unpermute of a
    tile-major output back to token order, each timed with HIP events.
    Algorithmic bytes: one tensor read + one written (+ the fp32 means)."""
    import numpy as np
    bh = wl.batch * wl.heads
    tiled = torch.empty(wl.batch, wl.heads, wl.n_rows, wl.tile_tokens, 128,
                        dtype=torch.bfloat16, device="cuda")
    tiled_d = torch.empty(wl.batch, wl.heads, wl.n_rows, 128, wl.tile_tokens,
                          dtype=torch.bfloat16, device="cuda")
    pooled = torch.empty(wl.batch, wl.heads, wl.n_tiles, 128, dtype=torch.float32,
                         device="cuda")
    out = torch.empty_like(qd)
    calls = {
        "tile_pool_token_major": lambda: m.ssta_tile_pool(g, qd, tiled, m.LAYOUT_TOKEN_MAJOR,
                                                          pooled),
        "tile_pool_dim_major": lambda: m.ssta_tile_pool(g, qd, tiled_d, m.LAYOUT_DIM_MAJOR,
                                                        None),
        "unpermute": lambda: m.ssta_tile_unpermute(g, tiled, out),
    }
    tensor = bh * wl.seq_len * 128 * 2
    nbytes = {"tile_pool_token_major": 2 * tensor + bh * wl.n_tiles * 128 * 4,
              "tile_pool_dim_major": 2 * tensor, "unpermute": 2 * tensor}
    res = {}
    for name, call in calls.items():
        call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        gbs = nbytes[name] / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "bytes": nbytes[name], "gbs": round(gbs, 1),
                     "pct_hbm": round(100 * gbs / PEAK_HBM_GBS, 1)}
    del tiled, tiled_d, pooled, out
    torch.cuda.empty_cache()
    return res


def mfma_ceiling(torch, m, iters=160000, reps=3):
    """Sustained bf16 matrix-core rate with the chip fully loaded (2 workgroups
    of 4 waves per CU, as the attention kernel runs), for random and for
    constant operands; about 20 ms per launch so the clock settles."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = 2 * cus
    gen = torch.Generator().manual_seed(7)
    tables = {"random_operands_tflops": torch.randn(256, 8, generator=gen).to(torch.bfloat16),
              "constant_operands_tflops": torch.full((256, 8), 0.5, dtype=torch.bfloat16)}
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    flop = grid * 4 * iters * 4 * 32768.0
    out = {"grid": grid, "iters": iters, "flop_per_launch": flop}
    for name, tab in tables.items():
        tab = tab.cuda()
        m.ssta_calibrate_mfma(tab, sink, grid, iters)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            m.ssta_calibrate_mfma(tab, sink, grid, iters)
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(flop * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SSTA forward shards by heads with no "
              "communication inside it, so a multi-GPU figure is N independent copies; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 19, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2, "launches": 5}))
        return

    import synthetic_inputs as si
    import video_dit_block_tile_amd as m

    wl = si.ALL[args.workload]
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    q, k, v = si.make_qkv(wl)
    gen_s = time.perf_counter() - t0
    print("[bench] %s inputs generated in %.1f s" % (wl.name, gen_s), file=sys.stderr, flush=True)

    def dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()

    qd, kd, vd = dev(q), dev(k), dev(v)
    g = m.make_geom(wl.batch, wl.heads, wl.T, wl.H, wl.W, tile=wl.tile, text_len=wl.text_len)
    p = m.make_params(win=wl.win, topk=wl.topk)
    fused = not args.materialised
    plan = m.SstaPlan(g, p, fused_io=fused)
    stream = torch.cuda.current_stream()

    phases = ("tile_pool", "score_select", "build_mask", "attention", "unpermute")
    calls = (lambda: plan.tile_pool(qd, kd, vd), plan.score_select, plan.build_mask,
             plan.attend, plan.unpermute)

    def step(ev=None):
        for j, call in enumerate(calls):
            if ev is not None:
                ev[j].record(stream)
            call()
        if ev is not None:
            ev[len(calls)].record(stream)

    def new_events(count):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
                for _ in range(count)]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = new_events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    def stats(xs):
        xs = np.asarray(xs, dtype=np.float64)
        return {"mean": round(float(xs.mean()), 4), "median": round(float(np.median(xs)), 4),
                "p10": round(float(np.percentile(xs, 10)), 4),
                "p90": round(float(np.percentile(xs, 90)), 4)}

    phase_stats = {ph: stats([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)])
                   for j, ph in enumerate(phases)}
    phase_ms = {ph: st["mean"] for ph, st in phase_stats.items()}
    step_event_stats = stats([evs[i][0].elapsed_time(evs[i][-1]) for i in range(args.steps)])

    # Cold L2/MALL: a 512 MB buffer is overwritten before each of these steps.
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ce = new_events(args.cold_steps)
        for i in range(args.cold_steps):
            flush.fill_(i & 0xFF)
            step(ce[i])
        torch.cuda.synchronize()
        cold = {"step_ms": stats([e[0].elapsed_time(e[-1]) for e in ce]),
                "attention_ms": stats([e[3].elapsed_time(e[4]) for e in ce])}
        del flush

    # block pairs computed (for a joint sequence the text pairs too); each is
    # 4 * R * R * 128 FLOP (R = tokens per block: 4 * 128^3 at the default block)
    pairs = block_pairs(wl, plan)
    n = wl.n_tiles
    R = wl.tile_tokens
    total_pairs = wl.batch * wl.heads * wl.n_rows * wl.n_rows
    flop = pairs * 4 * R * R * 128
    value = flop / (ms_step * 1e-3) / 1e12
    attn_tflops = flop / (phase_ms["attention"] * 1e-3) / 1e12
    print("[bench] sparse step %.3f ms, attention %.3f ms (%.1f TFLOP/s)"
          % (ms_step, phase_ms["attention"], attn_tflops), file=sys.stderr, flush=True)

    # Dense reference: the same pipeline with every block kept.
    dense_ms = dense_attn_ms = None
    if args.dense_steps > 0:
        dplan = m.SstaPlan(g, p, dense=True, fused_io=fused)
        dplan.run(qd, kd, vd)
        torch.cuda.synchronize()
        de = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for _ in range(args.dense_steps)]
        t0 = time.perf_counter()
        for i in range(args.dense_steps):
            dplan.tile_pool(qd, kd, vd)
            de[i][0].record(stream)
            dplan.attend()
            de[i][1].record(stream)
            dplan.unpermute()
        torch.cuda.synchronize()
        dense_ms = (time.perf_counter() - t0) * 1e3 / args.dense_steps
        dense_attn_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in de]))
        print("[bench] dense step %.1f ms, attention %.1f ms" % (dense_ms, dense_attn_ms),
              file=sys.stderr, flush=True)

    backward = None
    if args.backward_steps > 0:
        backward = backward_bench(torch, m, si, wl, plan, g, p, qd, kd, vd, pairs,
                                  args.backward_steps)
        print("[bench] backward %.3f ms (%.1f algorithmic TFLOP/s)"
              % (backward["ms"]["mean"], backward["algorithmic_tflops"]), file=sys.stderr,
              flush=True)

    variants = variant_runs(torch, m, si, args.variant_steps) if args.variant_steps > 0 else None
    mat_io = materialised_io(torch, m, wl, g, qd) if args.variant_steps > 0 else None
    configs = (per_config_runs(torch, m, si, args.config_steps, 1)
               if args.config_steps > 0 else None)

    ceiling = None if args.no_mfma_ceiling else mfma_ceiling(torch, m)
    if ceiling is not None:
        print("[bench] sustained bf16 MFMA: %.0f TFLOP/s random operands, %.0f constant"
              % (ceiling["random_operands_tflops"], ceiling["constant_operands_tflops"]),
              file=sys.stderr, flush=True)

    traffic = load_traffic(args.traffic_json, wl.name, kernel_hash())
    roof = {
        "kernel": "k_attn_fwd",
        "bound": "mfma",
        "achieved": round(attn_tflops, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "algorithmic_flop_per_launch": flop,
        "avg_launch_ms": round(phase_ms["attention"], 4),
        "frac_of_sustained_random": (None if ceiling is None else
                                     round(attn_tflops / ceiling["random_operands_tflops"], 4)),
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, q, k, v, args.cpu_rows)

    # Algorithmic bytes and VALU work of each phase (what the step must move or
    # compute at minimum).
    bh = wl.batch * wl.heads
    tensor = bh * wl.seq_len * 128 * 2                  # one of Q, K, V, O in bf16
    pooled = bh * n * 128 * 4
    phase_bytes = {
        # read Q and K, write both pooled arrays (materialised blocks: also read V and
        # write Q_t, K_t and V_t)
        "tile_pool": (2 if fused else 6) * tensor + 2 * pooled,
        # read both pooled arrays, write the top-k ids
        "score_select": 2 * pooled + bh * n * plan.width * 4,
        # read the top-k ids, write the kept lists and counts
        "build_mask": bh * n * (plan.width + plan.max_kept + 1) * 4,
        # each kept pair reads one K block and one V block (32 KB each at 128 tokens);
        # Q read, O written once
        "attention": pairs * 2 * R * 128 * 2 + 2 * tensor,
        "unpermute": 0 if fused else 2 * tensor,
    }
    phase_rates = {}
    for ph in phases:
        ms = phase_stats[ph]["median"]
        gbs = phase_bytes[ph] / (ms * 1e-3) / 1e9 if ms > 0 and phase_bytes[ph] else None
        if ph == "attention":
            # requested K/V block bytes: served mostly by L2 and the MALL, so no
            # fraction of HBM is claimed (the HBM-side bytes are roofline.traffic)
            phase_rates[ph] = {"logical_bytes": phase_bytes[ph],
                               "logical_gbs": None if gbs is None else round(gbs, 1)}
            continue
        phase_rates[ph] = {"bytes": phase_bytes[ph],
                           "gbs": None if gbs is None else round(gbs, 1),
                           "pct_hbm": None if gbs is None else round(100 * gbs / PEAK_HBM_GBS, 1)}
    # tile-score GEMV (q.k for every block pair) and key redundancy (k.k for every
    # pair): one fp32 FMA (2 FLOP) per channel each
    score_flop = 2 * bh * n * n * 128 * 2 if plan.width > 0 else 0
    ss_ms = phase_stats["score_select"]["median"]
    score_tflops = score_flop / (ss_ms * 1e-3) / 1e12 if ss_ms > 0 else 0.0
    phase_rates["score_select"].update({
        "valu_flop": score_flop, "valu_tflops": round(score_tflops, 2),
        "pct_fp32_unpacked_peak": round(100 * score_tflops / PEAK_FP32_UNPACKED_TFLOPS, 1),
        "pct_fp32_vector_peak_packed": round(100 * score_tflops / PEAK_FP32_VECTOR_TFLOPS, 1)})
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": wl.batch, "heads": wl.heads, "head_dim": wl.head_dim,
            "grid": [wl.T, wl.H, wl.W], "tile": list(wl.tile), "window_half": list(wl.win),
            "topk": wl.topk, "n_tiles": n, "seq_len": wl.n_tokens,
            "block_io": ("query blocks gathered / output scattered in the attention kernel"
                         if fused else "query blocks and output materialised tile-major"),
            "input": "smooth 3D sinusoid field + N(0, 0.5^2) noise, bf16, seed %d" % wl.seed,
        },
        "pct_bf16_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "attention_tflops": round(attn_tflops, 2),
        "pct_bf16_peak_attention": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "kept_pairs": pairs,
        "kept_fraction": round(pairs / total_pairs, 5),
        "phase_ms": phase_stats,
        "step_ms_events": step_event_stats,
        "phase_rates": phase_rates,
        "cold_cache": cold,
        "dense_ms_per_step": None if dense_ms is None else round(dense_ms, 3),
        "dense_attention_ms": None if dense_attn_ms is None else round(dense_attn_ms, 3),
        "speedup_vs_dense_step": None if dense_ms is None else round(dense_ms / ms_step, 3),
        "speedup_vs_dense_attention": (None if dense_attn_ms is None
                                       else round(dense_attn_ms / phase_ms["attention"], 3)),
        "roofline": roof,
        "mfma_sustained": ceiling,
        "backward": backward,
        "variants": variants,
        "per_config": configs,
        "materialised_io": mat_io,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

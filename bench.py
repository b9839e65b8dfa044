"""Benchmark of the block-sparse spatio-temporal attention path on one MI355X.

One step = the whole path over one synthetic batch at 75,600 tokens
(21 x 45 x 80), 10 heads, head dim 128, bf16: route the heads on 64 sampled
queries -> build the tile map on the GPU -> permute Q, K, V of temporal heads
-> block-sparse attention (full/boundary tile map, 256 x 128 tiles) ->
unpermute O. Inputs are resident in HBM before timing starts.

Prints one JSON line. Besides the step latency it reports, for the attention
kernel (the dominant one), its average duration measured with HIP events on
the stream it runs on, the algorithmic FLOP rate (4 * head_dim per kept
query-key pair) against the MI355X dense bf16 MFMA peak, the executed-tile
FLOP rate, the dense-map and in-kernel-gather variants, a query-tile sweep,
balanced rounding, and the oracle timed on the host cores.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attention fwd latency (ms) + effective TFLOP/s vs MFMA peak @75.6K tok"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PAGES_TPU_V6E_MS = {"B0 dense": 78.70, "B1 naive": 96.37, "B2 full/boundary": 54.12, "B3 rounded": 32.76}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--bq", type=int, default=256)
    ap.add_argument("--bkv", type=int, default=128)
    ap.add_argument("--mode", default="exact")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the variant and sweep timings")
    ap.add_argument("--layer-1440p", action="store_true",
                    help="only time the 302,400-token layer (routing, tile map, permutations, attention, "
                         "unpermutation) and print its figures as one JSON line (for kernel traces)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on whole heads and the whole tile map, routing and permutations "
                         "(a few minutes) instead of the bounded sample")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this path has no multi-GPU variant; "
              "see DESIGN.md for how it would shard by head.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_spatio_amd as B
    from synth import HEADLINE, P1440, planted_qkv, sample_indices

    w = HEADLINE
    dev = torch.device("cuda:0")
    if args.layer_1440p:
        aws = torch.empty(B.svga_attn_split_workspace_bytes(P1440.d, 512), dtype=torch.uint8, device=dev)
        print(json.dumps(layer_1440p(B, torch, dev, P1440, aws)), flush=True)
        return
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    mode = B.MODES[args.mode]
    bq, bkv = args.bq, args.bkv

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    log("bench: generating inputs")
    q, k, v = planted_qkv(1, w.F, w.H, w.W, w.d, w.kinds, seed=0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    idx = sample_indices(w.N, w.n_samples, seed=0).to(dev)
    ws = torch.empty(B.svga_route_workspace_bytes(1, w.heads, geom, w.d, w.n_samples), dtype=torch.uint8, device=dev)
    flags = torch.empty(1, w.heads, dtype=torch.uint8, device=dev)
    err = torch.empty(1, w.heads, 2, dtype=torch.float32, device=dev)
    off = B.svga_tilemap_layout(geom, bq, bkv)
    tmap = torch.empty(off.total, dtype=torch.uint8, device=dev)
    qp, kp, vp, op, o = (torch.empty_like(qd) for _ in range(5))
    # persistent workgroups with the split tail (the size for 256-row workgroups covers every bq)
    aws = torch.empty(B.svga_attn_split_workspace_bytes(w.d, 512), dtype=torch.uint8, device=dev)

    def step():
        B.svga_route_heads(qd, kd, vd, geom, mask, idx, workspace=ws, flags_out=flags, err_out=err)
        B.svga_build_tilemap(geom, mask, bq, bkv, mode, out=tmap)
        B.svga_permute(qd, flags, geom, mask, out=qp)
        B.svga_permute(kd, flags, geom, mask, out=kp)
        B.svga_permute(vd, flags, geom, mask, out=vp)
        B.svga_sparse_attn_fwd(qp, kp, vp, flags, tmap, geom, mask, bq, bkv, mode, out=op, workspace=aws)
        B.svga_unpermute(op, flags, geom, mask, out=o)

    log("bench: warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    routed = flags.cpu().numpy()[0].tolist()

    log("bench: timed steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-kernel times: HIP events on torch's current stream, which is the stream the library launches on
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(5, args.steps)
    t_route = timed(lambda: B.svga_route_heads(qd, kd, vd, geom, mask, idx, workspace=ws, flags_out=flags,
                                               err_out=err), reps)
    t_map = timed(lambda: B.svga_build_tilemap(geom, mask, bq, bkv, mode, out=tmap), reps)
    t_perm = timed(lambda: B.svga_permute(kd, flags, geom, mask, out=kp), reps)
    t_unperm = timed(lambda: B.svga_unpermute(op, flags, geom, mask, out=o), reps)
    t_attn = timed(lambda: B.svga_sparse_attn_fwd(qp, kp, vp, flags, tmap, geom, mask, bq, bkv, mode, out=op, workspace=aws), reps)
    # latency: median of 20 individually event-timed calls after 5 warm-ups
    for _ in range(5):
        B.svga_sparse_attn_fwd(qp, kp, vp, flags, tmap, geom, mask, bq, bkv, mode, out=op, workspace=aws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a_, b_ in ev:
        a_.record()
        B.svga_sparse_attn_fwd(qp, kp, vp, flags, tmap, geom, mask, bq, bkv, mode, out=op, workspace=aws)
        b_.record()
    torch.cuda.synchronize()
    t_attn_median = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev]))

    # work accounting from the tile map (read once, outside timing)
    host_map = B.tilemap_views(tmap.cpu().numpy(), geom, bq, bkv)
    fl = np.asarray(routed)
    n_exec = int(sum(host_map["n_full"][kk].sum() + host_map["n_bnd"][kk].sum() for kk in fl))
    n_bnd = int(sum(host_map["n_bnd"][kk].sum() for kk in fl))
    S, F, N, d = w.S, w.F, w.N, w.d
    sp_pairs = S * S * sum((min(F - 1, f + w.spatial_band) - max(0, f - w.spatial_band) + 1)
                           + (1 if f - w.spatial_band > 0 else 0) for f in range(F))
    wb = w.temporal_band
    tp_pairs = F * ((F - 1) * (S * (2 * wb + 1) - wb * (wb + 1)) + S * S)
    kept_pairs = int(sum(tp_pairs if kk else sp_pairs for kk in fl))
    flop_alg = 4.0 * d * kept_pairs
    flop_exec = 4.0 * d * bq * bkv * n_exec
    tflops_alg = flop_alg / (t_attn * 1e-3) / 1e12
    tflops_exec = flop_exec / (t_attn * 1e-3) / 1e12
    perm_bytes = 2.0 * w.heads * N * d * 2        # one tensor read + written
    route_bytes = 2.0 * w.heads * N * d * 2       # K and V read once

    extras = {}
    if not args.no_extras:
        log("bench: variants")
        def attn_with(mode_x, bq_x, gather=False):
            m = B.svga_build_tilemap(geom, mask, bq_x, bkv, mode_x)
            if gather:
                return timed(lambda: B.svga_sparse_attn_fwd(qd, kd, vd, flags, m, geom, mask, bq_x, bkv, mode_x,
                                                            gather_temporal=True, out=op, workspace=aws), reps)
            return timed(lambda: B.svga_sparse_attn_fwd(qp, kp, vp, flags, m, geom, mask, bq_x, bkv, mode_x, out=op,
                                                        workspace=aws), reps)
        t_dense = attn_with(B.MAP_DENSE, bq)
        extras["dense_map_ms (B0)"] = round(t_dense, 4)
        extras["dense_map_tflops"] = round(4.0 * d * N * N * w.heads / (t_dense * 1e-3) / 1e12, 1)
        extras["naive_map_ms (B1)"] = round(attn_with(B.MAP_NAIVE, bq), 4)
        extras["exact_map_ms (B2)"] = round(t_attn, 4)
        extras["rounded_map_ms (B3)"] = round(attn_with(B.MAP_ROUNDED, bq), 4)
        extras["speedup_exact_vs_dense"] = round(t_dense / t_attn, 3)
        extras["gather_temporal_ms"] = round(attn_with(mode, bq, gather=True), 4)
        extras["permute_path_ms (3 permutes + attention + unpermute)"] = round(3 * t_perm + t_attn + t_unperm, 4)
        for bq_x in (128, 256, 512):
            extras[f"exact_bq{bq_x}_ms"] = round(attn_with(B.MAP_EXACT, bq_x), 4)
        # balanced rounding (B3): temporal heads through the permutations or read in place by the kernel
        for bq_x in (128, 256):
            t_r = attn_with(B.MAP_ROUNDED, bq_x)
            extras[f"rounded_{bq_x}x{bkv}"] = {
                "attn_ms": round(t_r, 4),
                "permute_path_ms (3 permutes + attention + unpermute)": round(3 * t_perm + t_r + t_unperm, 4),
                "gather_ms (attention reading temporal heads in place)": round(
                    attn_with(B.MAP_ROUNDED, bq_x, gather=True), 4)}
        extras["small_3456"] = small_dense_vs_sparse(B, torch, dev, aws, timed, reps)
        extras["layer_1440p"] = layer_1440p(B, torch, dev, P1440, aws)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: oracle cpu baseline")
        cpu = cpu_baseline(w, q, k, v, routed, bq, bkv, args.cpu_seconds, full=args.cpu_full)

    out = {
        "metric": METRIC,
        "value": round(ms_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) entries with planted per-frame / per-position structure so routing "
                "selects 5 spatial + 5 temporal heads)",
        "config": {
            "workload": "75,600 tokens (21x45x80 latent), 10 heads, head_dim 128, bf16; 5 spatial heads (band 4 "
                        "frames) + 5 temporal heads (window 644), first-frame sink; step = route(64 samples) + "
                        f"tile map + permute QKV + {args.mode} attention + unpermute",
            "tiles": f"{bq}x{bkv}",
            "launch": "persistent workgroups taking query tiles from a counter, the last 256 query tiles split "
                      "in 4 pieces merged by log-sum-exp (svga_sparse_attn_fwd_ws, split-tail workspace)",
            "mode": args.mode,
        },
        "roofline": {
            "kernel": "attn_fwd_kernel + merge_kernel (one svga_sparse_attn_fwd_ws call)",
            "bound": "mfma",
            "achieved": round(tflops_alg, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops_alg / PEAK_BF16_TFLOPS, 4),
            "traffic": counted_traffic(args.mode, bq, bkv),
            "mfma_busy_pct": counted_mfma_busy(args.mode, bq, bkv),
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE, calibrated on a copy kernel)",
            "avg_ms": round(t_attn, 4),
            "latency_median_ms": round(t_attn_median, 4),
            "algorithmic_flop": flop_alg,
            "executed_tile_tflops": round(tflops_exec, 2),
            "executed_tile_frac": round(tflops_exec / PEAK_BF16_TFLOPS, 4),
        },
        "cpu_baseline": cpu,
        "breakdown_ms": {
            "route_heads": round(t_route, 4),
            "build_tilemap": round(t_map, 4),
            "permute_one_tensor": round(t_perm, 4),
            "sparse_attn_fwd": round(t_attn, 4),
            "unpermute": round(t_unperm, 4),
        },
        "hbm": {
            "permute_GBps": round(perm_bytes / (t_perm * 1e-3) / 1e9, 1),
            "permute_frac": round(perm_bytes / (t_perm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "route_GBps": round(route_bytes / (t_route * 1e-3) / 1e9, 1),
        },
        "work": {
            "kept_pairs": kept_pairs,
            "kept_frac": round(kept_pairs / (w.heads * N * N), 5),
            "executed_tiles": n_exec,
            "visited_frac": round(n_exec / (w.heads * off.tq * off.tk), 5),
            "boundary_of_executed": round(n_bnd / max(1, n_exec), 5),
            "routed_flags": routed,
        },
        "extras": extras,
        "context_tpu_v6e_ms (pages, isolated kernel, other hardware)": PAGES_TPU_V6E_MS,
    }
    print(json.dumps(out), flush=True)


def small_dense_vs_sparse(B, torch, dev, aws, timed, reps):
    """The 3,456-token case (9x16x24, 4 heads: 2 spatial, 2 temporal, d=128, 128x128 tiles): exact sparse
    attention against the dense map on the same permuted inputs (attention call only)."""
    from synth import SMALL, normal_qkv
    w = SMALL
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    q, k, v = (x.to(dev) for x in normal_qkv(1, w.heads, w.N, w.d, seed=1))
    flags = torch.tensor([list(w.kinds)], dtype=torch.uint8, device=dev)
    qp, kp, vp = (B.svga_permute(x, flags, geom, mask) for x in (q, k, v))
    op = torch.empty_like(qp)
    res = {"workload": "3,456 tokens (9x16x24), 4 heads (2 spatial band 1, 2 temporal window 24), d=128, 128x128"}
    for name, mode in (("exact", B.MAP_EXACT), ("dense", B.MAP_DENSE)):
        m = B.svga_build_tilemap(geom, mask, w.bq, w.bkv, mode, device=dev)
        t = timed(lambda: B.svga_sparse_attn_fwd(qp, kp, vp, flags, m, geom, mask, w.bq, w.bkv, mode, out=op,
                                                 workspace=aws), reps)
        hm = B.tilemap_views(m.cpu().numpy(), geom, w.bq, w.bkv)
        n_exec = int(sum(hm["n_full"][kk].sum() + hm["n_bnd"][kk].sum() for kk in w.kinds))
        res[f"{name}_ms"] = round(t, 4)
        res[f"{name}_executed_tile_tflops"] = round(4.0 * w.d * w.bq * w.bkv * n_exec / (t * 1e-3) / 1e12, 1)
    res["speedup_exact_vs_dense"] = round(res["dense_ms"] / res["exact_ms"], 3)
    return res


def layer_1440p(B, torch, dev, w, aws):
    """The 302,400-token layer end to end: routing on 64 samples, tile map, permutation of Q, K, V,
    exact sparse attention, unpermutation (HIP events; a few calls, inputs resident)."""
    from synth import planted_qkv, sample_indices
    geom = (w.F, w.H, w.W)
    mask = (w.sink_frames, w.spatial_band, w.temporal_band, w.temporal_layout)
    q, k, v = planted_qkv(1, w.F, w.H, w.W, w.d, w.kinds, seed=0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    idx = sample_indices(w.N, w.n_samples, seed=0).to(dev)
    ws = torch.empty(B.svga_route_workspace_bytes(1, w.heads, geom, w.d, w.n_samples), dtype=torch.uint8, device=dev)
    flags = torch.empty(1, w.heads, dtype=torch.uint8, device=dev)
    err = torch.empty(1, w.heads, 2, dtype=torch.float32, device=dev)
    off = B.svga_tilemap_layout(geom, w.bq, w.bkv)
    tmap = torch.empty(off.total, dtype=torch.uint8, device=dev)
    qp, kp, vp, op, o = (torch.empty_like(qd) for _ in range(5))
    mode = B.MAP_EXACT

    def parts():
        return [lambda: B.svga_route_heads(qd, kd, vd, geom, mask, idx, workspace=ws, flags_out=flags, err_out=err),
                lambda: B.svga_build_tilemap(geom, mask, w.bq, w.bkv, mode, out=tmap),
                lambda: (B.svga_permute(qd, flags, geom, mask, out=qp), B.svga_permute(kd, flags, geom, mask, out=kp),
                         B.svga_permute(vd, flags, geom, mask, out=vp)),
                lambda: B.svga_sparse_attn_fwd(qp, kp, vp, flags, tmap, geom, mask, w.bq, w.bkv, mode, out=op,
                                               workspace=aws),
                lambda: B.svga_unpermute(op, flags, geom, mask, out=o)]

    for f in parts():
        f()
    torch.cuda.synchronize()
    reps = 3
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
          for _ in range(reps)]
    for r in range(reps):
        for (a, b), f in zip(ev[r], parts()):
            a.record()
            f()
            b.record()
    torch.cuda.synchronize()
    ms = [sum(a.elapsed_time(b) for a, b in ev[r]) for r in range(reps)]
    each = [sum(ev[r][i][0].elapsed_time(ev[r][i][1]) for r in range(reps)) / reps for i in range(5)]
    host_map = B.tilemap_views(tmap.cpu().numpy(), geom, w.bq, w.bkv)
    fl = flags.cpu().numpy()[0]
    n_exec = int(sum(host_map["n_full"][kk].sum() + host_map["n_bnd"][kk].sum() for kk in fl))
    return {"workload": "302,400 tokens (21x90x160), 10 heads, d=128, routed on 64 samples, EXACT 256x128",
            "step_ms": round(sorted(ms)[reps // 2], 3), "route_ms": round(each[0], 4), "tilemap_ms": round(each[1], 4),
            "permute_qkv_ms": round(each[2], 4), "attn_ms": round(each[3], 3), "unpermute_ms": round(each[4], 4),
            "routed_flags": fl.tolist(),
            "attn_executed_tile_tflops": round(4.0 * w.d * w.bq * w.bkv * n_exec / (each[3] * 1e-3) / 1e12, 1)}


def counter_record(name, key, mode, bq, bkv):
    """A figure from a committed rocprofv3 counter summary under profiles/, or None when the record is for
    another configuration or the kernel sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", name)
    try:
        rec = json.loads(re.search(r"```json\n(.*?)\n```", open(path).read(), re.S).group(1))
    except (OSError, AttributeError, ValueError):
        return None
    if (rec["mode"], rec["bq"], rec["bkv"]) != (mode, bq, bkv):
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec[key] if h.hexdigest() == rec["sources_sha256"] else None


def counted_traffic(mode, bq, bkv):
    """HBM bytes per attention launch (calibrated FETCH_SIZE / WRITE_SIZE)."""
    return counter_record("attn_fwd_headline_exact_256x128_hbm_counters.md", "traffic_bytes", mode, bq, bkv)


def counted_mfma_busy(mode, bq, bkv):
    """MFMA-busy % of the attention kernel (rocprofv3 MfmaUtil formula)."""
    return counter_record("attn_fwd_headline_exact_256x128_mfma_counters.md", "mfma_busy_pct", mode, bq, bkv)


def cpu_baseline(w, q, k, v, flags, bq, bkv, target_s, full=False):
    """The oracle, unchanged, on a bounded sample of the step; extrapolated to the whole step. With `full`,
    every query row of one spatial and one temporal head (the other heads of each kind cost the same: the
    oracle's work depends on the mask, not on the values), the whole tile map, routing of every head on all
    its samples, and every permutation of the step."""
    import numpy as np

    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    except Exception:
        blas = cores
    scale = 1 / math.sqrt(w.d)
    N = w.N
    mask = (w.sink_frames, w.spatial_band, w.temporal_band)
    # attention: rows of head 0 (spatial) and head 5 (temporal), grown until the target time
    t_begin = time.perf_counter()
    rows_done, t_attn = 0, 0.0
    rng = np.random.default_rng(0)
    q0 = {h: (q[0, h].double().numpy(), k[0, h].double().numpy(), v[0, h].double().numpy()) for h in (0, 5)}
    n_rows = 64
    if full:
        for h in (0, 5):
            t0 = time.perf_counter()
            O.attention_head(*q0[h], flags[h], w.F, w.H, w.W, *mask, w.temporal_layout, O.MODE_EXACT, bq, bkv,
                             scale)
            t_attn += (time.perf_counter() - t0) * sum(1 for f in flags if f == flags[h])
        rows_done = N * w.heads
    while not full and t_attn < 0.6 * target_s and rows_done < N:
        for h in (0, 5):
            rows = rng.choice(N, n_rows, replace=False)
            t0 = time.perf_counter()
            O.attention_head(*q0[h], flags[h], w.F, w.H, w.W, *mask, w.temporal_layout, O.MODE_EXACT, bq, bkv,
                             scale, rows=rows)
            t_attn += time.perf_counter() - t0
            rows_done += n_rows
        n_rows *= 2
    attn_full = t_attn if full else t_attn / rows_done * N * w.heads
    # tile map: the element scan of a few query tiles per kind
    t0 = time.perf_counter()
    tq = -(-N // bq)
    nq = tq if full else 4
    for kind in (0, 1):
        O.tile_counts(w.F, w.H, w.W, kind, *mask, w.temporal_layout, bq, bkv, q_tiles=range(nq))
    map_full = (time.perf_counter() - t0) / nq * tq
    # routing: 8 of the 64 sampled queries of one head
    t0 = time.perf_counter()
    if full:
        from synth import sample_indices
        O.route_heads(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.F, w.H, w.W, *mask,
                      sample_indices(N, w.n_samples, seed=0).numpy(), scale)
        route_full = time.perf_counter() - t0
    else:
        O.route_heads(q[:, :1].double().numpy()[:, :, :], k[:, :1].double().numpy(), v[:, :1].double().numpy(),
                      w.F, w.H, w.W, *mask, np.arange(8) * 997, scale)
        route_full = (time.perf_counter() - t0) / 8 * w.n_samples * w.heads
    # permutation of one head of one tensor
    t0 = time.perf_counter()
    order = O.executed_order(w.F, w.H, w.W, 1, w.sink_frames, w.temporal_layout)
    if full:
        for h in range(w.heads):
            if flags[h]:
                for x in (q, k, v):
                    O.permute(x[0, h].float().numpy(), order)
                O.unpermute(q[0, h].float().numpy(), order)
        perm_full = time.perf_counter() - t0
    else:
        O.permute(q[0, 5].float().numpy(), order)
        perm_full = (time.perf_counter() - t0) * 4 * sum(flags)
    total_s = attn_full + map_full + route_full + perm_full
    return {
        "value": round(total_s * 1e3, 1),
        "unit": "ms",
        "cores": blas,
        "host_cpus": cores,
        "kind": "oracle",
        "sample": ("whole step: every query row of head 0 (spatial) and head 5 (temporal), each counted once "
                   "per head of its kind; the whole tile map; routing of all heads on all samples; every "
                   "permutation" if full else
                   f"attention: {rows_done} query rows of heads 0 and 5 (of {N * w.heads}); tile map: {nq} of {tq} "
                   f"query tiles per kind; routing: 8 of {w.n_samples} samples of 1 of {w.heads} heads; permute: "
                   "1 head of 1 tensor; each scaled linearly to the full step"),
        "measured_s": round(time.perf_counter() - t_begin, 2),
        "parts_ms": {"attention": round(attn_full * 1e3, 1), "tilemap": round(map_full * 1e3, 1),
                     "routing": round(route_full * 1e3, 1), "permute": round(perm_full * 1e3, 1)},
    }


if __name__ == "__main__":
    main()

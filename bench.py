"""Benchmark of the routed-expert MoE layer (prompt ingestion) on one MI355X.

Workload: 2,048 tokens x 512 experts x top-10, hidden 2048, expert intermediate 512, T1
experts (~1.78 bits/weight), bf16 activations, seeded synthetic inputs (the reference pages
measure one layer of a real model file, which is not available here; the synthetic layer has
the same shapes and ~40 pairs per expert).

A step is one rl_moe_prefill call (grouping with the split of x, fused dequant + gate/up +
SwiGLU, split of h, fused dequant + down, ordered combine) over the resident inputs.  Weight sets rotate over several arena
copies at different addresses so that every step reads its weights from HBM rather than from
the 256 MB Infinity Cache.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Useful-FLOP ceiling of the gate/up kernel: it multiplies on the fp8 MFMA (5.03 PFLOP/s dense)
# but every useful multiply-add takes two fp8 products (activation = hi + lo), so the ceiling is
# half the fp8 peak, which equals the dense bf16/fp16 MFMA peak (256 CU x 4 SIMD x 1024 FLOP/clk
# x 2.4 GHz).
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS  # the fp8 MFMA rate the T1 kernels issue at (AMD: 5.0 PFLOP/s dense)
PEAK_HBM_GBS = 8000.0
STAGES = ("group", "gate_up", "hsplit", "down", "combine")  # group includes the split of x
KERNEL_SOURCES = ("routed_experts_bit_amd/csrc/rl_kernels.h", "routed_experts_bit_amd/csrc/rl_decode.h")


def kernel_digest():
    """sha256 over the kernel sources (a traffic measurement is valid only for these)."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each calibrated against a device copy of known size), or None
    when there is none for this workload or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_digest") != kernel_digest():
        return None
    return rec.get("gate_up_bytes_per_launch")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed layer steps before the timed ones (the 1-2 row and router measurements run "
                         "first, so the GPU is already under load)")
    ap.add_argument("--config", default="t1_2048")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--rotate", type=int, default=0,
                    help="distinct arena copies cycled through (0: at least 3 and at least 1 GiB in all, so that "
                         "the weights come from HBM, not the memory-side cache)")
    ap.add_argument("--no-oracle", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--oracle-threads", type=int, default=0)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size reference for HBM byte "
                         "counters under a profiler)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the single-GPU hot path only: run it with --gpus 1 (one process, one GPU).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import routed_experts_bit_amd as rl
    from workload import make_workload, matrix_bytes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t0 = time.time()
    wl = make_workload(args.config, seed=args.seed)
    ex0 = wl.experts
    T, k, E, H, I = wl.T, wl.k, ex0.E, ex0.H, ex0.I
    counts = np.bincount(wl.ids.ravel(), minlength=E)
    log(f"[bench] workload {args.config}: T={T} k={k} E={E} H={H} I={I} arena={ex0.arena.nbytes / 2**20:.1f} MiB "
        f"pairs/expert min={counts.min()} mean={counts.mean():.1f} max={counts.max()} (gen {time.time() - t0:.1f}s)")

    dev = rl.DeviceExperts.from_workload(ex0)
    if args.rotate <= 0:
        args.rotate = max(3, -(-(1 << 30) // ex0.arena.nbytes))
    sets = [dev] + [dev.with_arena(dev.arena.clone()) for _ in range(max(args.rotate, 1) - 1)]
    x = torch.from_numpy(wl.x.view(np.int16).copy()).cuda()
    ids = torch.from_numpy(wl.ids).cuda()
    w = torch.from_numpy(wl.w).cuda()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    # a layer of T tokens is taken as consecutive calls of at most `chunk` tokens (one call unless
    # the workload names a chunk size), all on one stream and one workspace
    chunk = int(wl.meta.get("chunk") or T)
    spans = [(c0, min(T, c0 + chunk)) for c0 in range(0, T, chunk)]
    ws = rl.alloc_workspace(min(T, chunk), k, dev)

    def layer(exps):
        for c0, c1 in spans:
            rl.prefill(x[c0:c1], ids[c0:c1], w[c0:c1], exps, out=out[c0:c1], ws=ws)

    flops = 6.0 * H * I * T * k
    qts = ex0.qtypes
    touched = np.unique(wl.ids)
    layer_bytes = int(sum(3 * matrix_bytes(I, H, int(qts[e])) for e in touched) + T * H * 2 + T * k * 8 + T * H * 4)
    flops_gateup = 4.0 * H * I * T * k
    flops_down = 2.0 * H * I * T * k

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the 1-2 row path (decode and 2-row verify) on the same experts: each step its own seeded
    # routing and x, weight sets rotating as above; weight bytes = the distinct experts' 3 matrices
    from workload.gen import _routing, gen_x, matrix_bytes

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    qt = ex0.qtypes

    dec = {}
    nd = 1000  # steps per row count, each with its own seeded routing and x
    for R in (1, 2):
        xs_d, ids_d, w_d, wb = [], [], [], []
        for s in range(nd):
            i_np, w_np = _routing(R, E, k, args.seed + 100 + s)
            # weight bytes of the step: each distinct expert's gate, up and down matrices once
            wb.append(sum(3 * matrix_bytes(I, H, int(qt[e])) for e in set(i_np.ravel().tolist())))
            ids_d.append(torch.from_numpy(i_np).cuda())
            w_d.append(torch.from_numpy(w_np).cuda())
            xs_d.append(torch.from_numpy(gen_x(R, H, args.seed + 300 + s).view(np.int16).copy()).cuda())
        out_d = torch.empty((R, H), dtype=torch.float32, device="cuda")
        ws_d = rl.alloc_workspace(R, k, dev)
        for s in range(5):
            rl.decode(xs_d[s], ids_d[s], w_d[s], sets[s % len(sets)], out=out_d, ws=ws_d)
        torch.cuda.synchronize()
        # eager: one Python call per step (argument checks, ctypes, two launches): host-bound
        e0.record(stream)
        for s in range(nd):
            rl.decode(xs_d[s], ids_d[s], w_d[s], sets[s % len(sets)], out=out_d, ws=ws_d)
        e1.record(stream)
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) / nd * 1e3
        # the same steps captured once in a graph and replayed: the GPU time per step, as a serving
        # loop that replays its decode step sees it
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(nd):
                rl.decode(xs_d[s], ids_d[s], w_d[s], sets[s % len(sets)], out=out_d, ws=ws_d)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / nd * 1e3
        del g
        wbytes = float(np.mean(wb))
        dec[f"rows_{R}"] = {"us_per_step": round(us, 2), "timing": "graph replay of the steps",
                            "us_per_call_eager": round(us_eager, 2), "weight_bytes": round(wbytes),
                            "GB_s": round(wbytes / us / 1e3, 1), "pct_hbm_peak": round(100 * wbytes / us / 1e3 / PEAK_HBM_GBS, 2)}
    log("[bench] 1-2 row path: " + "; ".join(f"{k_}: {v['us_per_step']} us/step ({v['us_per_call_eager']} per eager call), "
                                              f"{v['GB_s']} GB/s" for k_, v in dec.items()))

    # the router (the step before the layer): fp32 logits [T][E] -> ids and weights [T][k], on
    # seeded logits of the workload's shape (with its per-expert bias, if any)
    from workload import gen_logits, zipf_bias

    bias = zipf_bias(E, args.seed + 3) if wl.meta.get("bias") == "zipf" else None
    lg_np = gen_logits(T, E, args.seed + 2, bias)
    lg = torch.from_numpy(lg_np).cuda()
    r_ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    r_w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    for _ in range(5):
        rl.route(lg, k, r_ids, r_w)
    nr = 10 * args.steps
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(nr):
        rl.route(lg, k, r_ids, r_w)
    e1.record(stream)
    torch.cuda.synchronize()
    r_us = e0.elapsed_time(e1) / nr * 1e3
    # the same calls replayed from a captured HIP graph: the GPU's own time per call, without
    # the host's launch pacing (one small kernel per call)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(nr):
            rl.route(lg, k, r_ids, r_w)
    graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    r_us_g = e0.elapsed_time(e1) / nr * 1e3
    r_bytes = T * E * 4 + T * k * 8
    router = {"us_per_call": round(r_us, 2), "us_per_call_graph": round(r_us_g, 2), "bytes": r_bytes,
              "GB_s_graph": round(r_bytes / r_us_g / 1e3, 1),
              "pct_hbm_peak_graph": round(100 * r_bytes / r_us_g / 1e3 / PEAK_HBM_GBS, 2)}
    log(f"[bench] router: {r_us:.2f} us per call, {r_us_g:.2f} us per call from a graph ({router['GB_s_graph']} GB/s)")
    # the MoE block (shared expert + residual, rl_moe_prefill_block) and the router fused with the
    # grouping (rl_moe_prefill_from_logits) against the router and the layer as two calls, on the
    # same workload with one more (shared) expert of the same block type (run before the layer's
    # warm-up and timed steps, which then start on a GPU under load)
    from workload import make_block_workload

    bw = make_block_workload(args.config, seed=args.seed)
    bdev = rl.DeviceExperts.from_workload(bw.wl.experts)
    bsets = [bdev] + [bdev.with_arena(bdev.arena.clone()) for _ in range(max(args.rotate, 1) - 1)]
    gate = torch.from_numpy(bw.gate).cuda()
    resid = torch.from_numpy(bw.residual).cuda()
    lg_b = torch.from_numpy(gen_logits(T, E, args.seed + 2, zipf_bias(E, args.seed + 3) if wl.meta.get("bias") == "zipf"
                                       else None)).cuda()
    ws_b = torch.empty(rl.workspace_bytes(min(T, chunk), k + 1, E + 1, H, I), dtype=torch.uint8, device="cuda")
    ids_r = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_r = torch.empty((T, k), dtype=torch.float32, device="cuda")

    def block_layer(exps):
        for c0, c1 in spans:
            rl.prefill_block(x[c0:c1], ids[c0:c1], w[c0:c1], exps, bw.shared, gate[c0:c1], resid[c0:c1],
                             out=out[c0:c1], ws=ws_b)

    def fused_route_layer(exps):
        for c0, c1 in spans:
            rl.prefill_from_logits(x[c0:c1], lg_b[c0:c1], k, exps, out=out[c0:c1], ids=ids_r[c0:c1],
                                   w=w_r[c0:c1], ws=ws)

    def split_route_layer(exps):
        for c0, c1 in spans:
            rl.route(lg_b[c0:c1], k, ids_r[c0:c1], w_r[c0:c1])
            rl.prefill(x[c0:c1], ids_r[c0:c1], w_r[c0:c1], exps, out=out[c0:c1], ws=ws)

    def time_layer(fn, sets_):
        # 40 untimed calls first: after the short 1-2 row kernels the clocks need tens of ms of
        # load to settle (5 calls left the MoE block ~40 us slower than on a warm GPU)
        for i in range(40):
            fn(sets_[i % len(sets_)])
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(sets_[i % len(sets_)])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_block = time_layer(block_layer, bsets)
    ms_fused = time_layer(fused_route_layer, sets)
    ms_split = time_layer(split_route_layer, sets)
    del bsets, bdev
    log(f"[bench] MoE block (shared expert + residual): {ms_block * 1e3:.1f} us/layer; router + layer: fused "
        f"{ms_fused * 1e3:.1f} us, two calls {ms_split * 1e3:.1f} us")
    # warm-up
    for i in range(args.warmup):
        layer(sets[i % len(sets)])
    torch.cuda.synchronize()
    assert rl.status(ws)[0] == 0

    # timed region: K steps, rotating weight sets
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        layer(sets[i % len(sets)])
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-step times (one event pair around each step's calls; each interval also holds one
    # event's overhead) for the median and the minimum
    ev_steps = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev_steps[i][0].record(stream)
        layer(sets[i % len(sets)])
        ev_steps[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([a_.elapsed_time(b_) for a_, b_ in ev_steps])

    # same number of steps with events between the kernels (on the stream the kernels run on)
    # (per chunk; a step's stage time is the sum over its chunks)
    ne = rl.TIMED_EVENTS
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(ne)] for _ in spans] for _ in range(args.steps)]
    for step_evs in evs:  # torch creates the HIP event on its first record
        for row in step_evs:
            for e in row:
                e.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        for (c0, c1), row in zip(spans, evs[i]):
            rl.prefill_timed(x[c0:c1], ids[c0:c1], w[c0:c1], sets[i % len(sets)], out[c0:c1], ws, row)
    torch.cuda.synchronize()
    stage = np.array([[sum(row[j].elapsed_time(row[j + 1]) for row in evs[i]) for j in range(ne - 1)]
                      for i in range(args.steps)])
    st_ms = dict(zip(STAGES, stage.mean(axis=0)))

    # warm (same weights every step) for context
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        layer(dev)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / args.steps

    gpu_out = out.cpu().numpy().astype(np.float64)


    tflops = flops / (ms_step * 1e-3) / 1e12
    gu_tflops = flops_gateup / (st_ms["gate_up"] * 1e-3) / 1e12
    log(f"[bench] {ms_step * 1e3:.1f} us/layer = {tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.2f}% of bf16 "
        f"peak); kernels us: " + " ".join(f"{k} {v * 1e3:.1f}" for k, v in st_ms.items()) +
        f"; warm {ms_warm * 1e3:.1f} us")

    result = {
        "metric": "routed-expert layer ms & TFLOPS (% bf16 MFMA peak), 2048 tok, 512 exp, top-10",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # T1 experts on the fp8 MFMA: weights s*t exact in e4m3, bf16 x carried exactly as hi + lo e4m3
        # pairs (h with 8 significant bits), fp32 accumulation: bf16-class arithmetic
        "dtype": "bf16-equivalent (fp8 e4m3 hi+lo operands, fp32 accumulation)",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {T} tokens x {E} experts x top-{k}, hidden {H}, intermediate {I}, "
                        f"{'T1' if args.config.startswith('t1') else wl.meta['types']} experts, bf16 activations"
                        + (f", as {len(spans)} calls of {chunk} tokens" if len(spans) > 1 else ""),
            "tokens": T, "experts": E, "top_k": k, "hidden": H, "intermediate": I, "pairs": T * k,
            "seed": args.seed, "weight_sets_rotated": len(sets),
        },
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 3),
        "ms_per_layer_median": round(float(np.median(per_step)), 5),
        "ms_per_layer_min": round(float(per_step.min()), 5),
        # algorithmic bytes of the layer: every touched expert's three matrices once, x read,
        # ids and weights read, out written; at 8 TB/s
        "layer_bytes": layer_bytes,
        "pct_hbm_roofline": round(100 * layer_bytes / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9), 3),
        "ms_per_layer_warm": round(ms_warm, 5),
        "stage_ms": {k_: round(v, 5) for k_, v in st_ms.items()},
        "decode_path": dec,
        "router": router,
        "roofline": {
            "kernel": {"t1": "k_t1_f8<gate/up> (fused T1 decode + gate/up grouped GEMM on fp8 MFMA + SwiGLU + split of h "
                             "into hi/lo fp8 for the down kernel)",
                       "q2b": "k_q2_mm<gate/up> (fused Q2B decode + gate/up grouped GEMM on bf16 MFMA + SwiGLU)",
                       "mixed": "k_q2_mm<gate/up> + k_t1_f8<gate/up> (both gate/up stage kernels, one per block "
                                "type)"}[wl.meta["types"]],
            "bound": "mfma",
            "achieved": round(gu_tflops, 3),
            # the kernel issues fp8 MFMAs (T1; Q2B: bf16 at the same time per product), two per useful
            # product (activation hi and lo): frac against the fp8 peak, and against half of it
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gu_tflops / PEAK_FP8_TFLOPS, 5),
            "frac_of_hi_lo_ceiling": round(gu_tflops / PEAK_BF16_TFLOPS, 5),
            "traffic": measured_traffic(args.config),
        },
        "moe_block_ms_per_layer": round(ms_block, 5),
        "router_fused_ms_per_layer": round(ms_fused, 5),
        "router_then_layer_ms": round(ms_split, 5),
    }

    if not args.no_oracle:
        import oracle

        nthr = args.oracle_threads or oracle.default_threads()
        t1 = time.time()
        ref = oracle.moe_workload(wl, threads=nthr)
        cpu_s = time.time() - t1
        err = float(np.linalg.norm(gpu_out - ref) / np.linalg.norm(ref))
        try:
            affinity = len(os.sched_getaffinity(0))
        except (AttributeError, OSError):
            affinity = None
        result["cpu_baseline"] = {"value": round(flops / cpu_s / 1e12, 6), "unit": "TFLOP/s", "cores": nthr,
                                  "kind": "oracle", "ms_per_layer": round(cpu_s * 1e3, 1),
                                  "host_cpus": os.cpu_count(), "cpus_available": affinity,
                                  "sample": f"the whole {args.config} layer once (all {T * k} pairs; same inputs), "
                                            f"C, float64, {nthr} threads (the cores this process may use, capped "
                                            f"by OMP_NUM_THREADS)"}
        result["parity_rel_l2_vs_oracle"] = err
        log(f"[bench] oracle {cpu_s:.1f}s on {nthr} threads; GPU vs oracle rel_l2 {err:.3e}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of one sliding-tile attention layer training step on one MI355X.

Workload (the 720P-shaped training step): batch 1, 24 heads, head dim 128,
token grid (T,H,W) = (30,48,80) = 115200 tokens, tile (6,8,8) = 384 tokens,
5x6x10 tile grid, window 3x3x5 tiles, bf16 with fp32 accumulation; inputs
are seeded synthetic N(0,1) values (see tests/inputs.py) already resident in
HBM when timing starts.

One step is the whole hot path:
  raster -> tile order of Q, K, V;  block-sparse index build;  forward;
  tile -> raster of O;  raster -> tile of dO;  backward (Delta, dK/dV, dQ);
  tile -> raster of dQ, dK, dV.
Throughput counts only unmasked tile pairs: forward 4*L^2*D flop per pair,
backward 2.5x that, as the operator's "linear in sequence length" work.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints ONE JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective attention TFLOP/s (unmasked tile pairs) + ms/layer, 115200-tok grid"
PEAK_BF16_TFLOPS = 2516.6        # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
WORKLOAD = 5                     # the training workload of tests/inputs.py
KEY_TILE_45 = 72                 # tile (1,1,2): exactly 45 query tiles attend it (the mean)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=320,
                    help="query rows and key rows of the oracle sample (CPU baseline)")
    return ap.parse_args()


def kernel_sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sliding_tile_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, per_launch_flop_digest):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != per_launch_flop_digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, rows):
    """The plain CPU oracle on a bounded sample of the same workload: forward
    and dQ for `rows` query rows plus dK/dV for `rows` key rows of head 0,
    counted as `rows` rows of the training step."""
    from oracle import oracle    # test infrastructure: only this leg of the benchmark uses it
    B, H, N, D = w["q"].shape
    L = int(np.prod(w["tile"]))
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))       # tile-order slot -> raster token
    g = np.random.default_rng(7)
    qrows = np.sort(inv[g.choice(L, rows, replace=False)])                      # query tile 0
    krows = np.sort(inv[KEY_TILE_45 * L + g.choice(L, rows, replace=False)])    # 45 query tiles attend it
    keys_per_row = 45 * L
    flop = rows * 3.5 * 4.0 * keys_per_row * D
    oracle.load()
    t0 = time.perf_counter()
    oracle.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"], rows=qrows)
    oracle.bwd(w["q"], w["k"], w["v"], w["dout"], w["grid"], w["tile"], w["windows"], qrows=qrows, krows=krows)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "head 0: forward + dQ for %d query rows of query tile 0 and dK/dV for %d key rows of key "
                      "tile %d (45 query tiles attend it), counted as %d training rows of 17280 keys each; "
                      "%.1f s wall" % (rows, rows, KEY_TILE_45, rows, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the sliding-tile attention path here has no multi-GPU "
              "mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_tile_attention_amd as sta
    from tests.inputs import workload

    w = workload(WORKLOAD)
    B, H, N, D = w["q"].shape
    geom = sta.Geometry(tuple(w["grid"]), tuple(w["tile"]))
    L, T = geom.tile_tokens, geom.num_tiles
    windows = [tuple(x) for x in w["windows"]]
    dev = torch.device("cuda", 0)
    bf = dict(dtype=torch.bfloat16, device=dev)
    # raster-order inputs resident in HBM
    q, k, v, do = (torch.from_numpy(x).to(**bf) for x in (w["q"], w["k"], w["v"], w["dout"]))
    # work buffers (tile order) and outputs (raster order)
    qt, kt, vt, ot, dot_, dqt, dkt, dvt = (torch.empty_like(q) for _ in range(8))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    idx = sta.StaIndex(geom, windows, None)
    scale = D ** -0.5
    row_bytes = D * 2
    stream = torch.cuda.current_stream()

    names = ["reorder_qkv", "index", "fwd", "reorder_o", "reorder_do", "bwd_delta", "bwd_dkdv", "bwd_dq",
             "reorder_grads"]

    def step(evs=None):
        def mark(i):
            if evs is not None:
                evs[i].record(stream)
        mark(0)
        for src, dst in ((q, qt), (k, kt), (v, vt)):
            sta.sta_tile_reorder(src, dst, B * H, row_bytes, geom, False, stream)
        mark(1)
        sta.sta_build_index(geom, windows, None, idx, stream)
        mark(2)
        sta.sta_fwd(qt, kt, vt, ot, lse, B, H, D, sta.STA_BF16, scale, geom, idx, stream)
        mark(3)
        sta.sta_tile_reorder(ot, o, B * H, row_bytes, geom, True, stream)
        mark(4)
        sta.sta_tile_reorder(do, dot_, B * H, row_bytes, geom, False, stream)
        mark(5)
        for i, part in enumerate((sta.STA_BWD_DELTA, sta.STA_BWD_DKDV, sta.STA_BWD_DQ)):
            sta.sta_bwd_parts(qt, kt, vt, ot, lse, dot_, dqt, dkt, dvt, delta, B, H, D, sta.STA_BF16, scale, geom,
                              idx, part, stream)
            mark(6 + i)
        for src, dst in ((dqt, dq), (dkt, dk), (dvt, dv)):
            sta.sta_tile_reorder(src, dst, B * H, row_bytes, geom, True, stream)
        mark(9)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(10)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}

    kv_cnt = idx.kv_cnt.cpu().numpy()
    fwd_flop = 4.0 * B * float(kv_cnt.sum()) * L * L * D          # counted: unmasked tile pairs
    step_flop = 3.5 * fwd_flop                                      # forward + backward (2.5x)
    value = step_flop / (ms_per_step * 1e-3) / 1e12

    # Algorithmic work of each attention kernel (flop per launch): the forward
    # does QK^T and PV (4 L^2 D per pair); dK/dV must form S, dP, dV and dK
    # (8 L^2 D); dQ adds only the dQ product (2 L^2 D; its S and dP are
    # recomputation).  Together the backward is 10 L^2 D = 2.5x the forward.
    alg = {"fwd": fwd_flop, "bwd_dkdv": 2.0 * fwd_flop, "bwd_dq": 0.5 * fwd_flop}
    dominant = max(alg, key=lambda n: per[n])
    achieved = alg[dominant] / (per[dominant] * 1e-3) / 1e12
    digest = kernel_sources_digest(["fwd_bf16.hip" if dominant == "fwd" else "bwd_bf16.hip", "mfma.h"])
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "kernel": dominant,
                "traffic": measured_traffic(dominant, digest)}

    tensor_bytes = B * H * N * D * 2
    reorder_gbs = 3 * 2 * tensor_bytes / (per["reorder_qkv"] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "720p training step: B=1 H=24 D=128, grid (30,48,80)=115200 tokens, tile (6,8,8), "
                        "window 3x3x5 tiles, forward+backward",
            "global_batch": B,
            "seq_len": N,
            "parallelism": "none (1 GPU)",
            "counted_flop_per_step": step_flop,
            "ms_per_layer_fwd_bwd": round(ms_per_step, 3),
            "ms_per_layer_fwd": round(per["reorder_qkv"] + per["index"] + per["fwd"] + per["reorder_o"], 3),
            "fwd_kernel_ms": round(per["fwd"], 3),
            "fwd_tflops": round(fwd_flop / (per["fwd"] * 1e-3) / 1e12, 1),
            "fwd_frac_of_peak": round(fwd_flop / (per["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_kernels_ms": round(per["bwd_delta"] + per["bwd_dkdv"] + per["bwd_dq"], 3),
            "reorder_qkv_gbs": round(reorder_gbs, 1),
            "per_call_ms": {n: round(t, 4) for n, t in per.items()},
        },
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

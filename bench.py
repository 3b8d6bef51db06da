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

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--text M]

--text M measures the joint text + video variant of the same step: M text
tokens follow the video tokens of every (b, h) slab (token-type-aware
masking: text rows and columns dense); the counted work adds the text pairs,
4*D*M*(2N + M) flop per (b, h) in the forward.

--forward-only times the inference layer instead (reorder Q,K,V; index;
forward; reorder O), counted as the forward's work; --precision fp8 runs that
forward with the quantized products (INT8 QK^T, FP8 e4m3 PV), whose roofline
peak is the MI355X dense fp8 / int8 rate.

--adaptive RT,RH,RW adds the window-shift producer to the step: after the
reorder, every query tile's window shift (|shift| <= R per axis) is chosen on
device from the tile means of Q and K (sta_window_shifts) and the index is
built from those shifts, one set per head.

--layout raster runs the step without any reorder pass: the attention
kernels read Q, K, V, dO and write O, LSE, dQ, dK, dV in raster token order
directly (index; forward; backward).

--grid T,H,W replaces the token grid, e.g. the 720p latent grid 30,45,80 that
the (6,8,8) tile does not divide (its last tile row along H is cut to 5
rows); counted work then sums len(q) * len(k) over the listed tile pairs.

--workload 720p-shifted-perhead runs the step on the deformable-window
workload of the same shape: every head draws its window from {3x3x3, 3x3x5,
5x5x5} tiles and every query tile a seeded window shift in
[-1,1]x[-2,2]x[-2,2] tiles (tests/inputs.py); the counted work sums the
tile pairs of the built lists (27, 45 or 125 key tiles per query tile).

Prints ONE JSON line.

HBM traffic of the attention kernels (roofline "traffic") comes from two
rocprofv3 counter passes over this benchmark (FETCH_SIZE, then WRITE_SIZE),
summarised into profiles/traffic.json by

    python bench.py --write-traffic FETCH_CSV WRITE_CSV

Each counter is scaled by what it reads for one launch of a plain streaming
copy probe (libsta_probe.so, copy_probe_kernel) of one attention input's bytes,
which every run of this benchmark makes once after the timed steps: its bytes
are known exactly (every source byte read once, every destination byte written
once), so the reorder kernel's traffic is measured like the others.  The
summary records a digest of the kernel sources; when they change, "traffic" is
reported as null.
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
PEAK_FP8_TFLOPS = 5033.2         # MI355X dense fp8 / int8 MFMA (twice the bf16 rate)
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
WORKLOAD = "720p-train"          # the training workload of tests/inputs.py


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="query rows and key rows of the oracle sample (CPU baseline)")
    ap.add_argument("--forward-only", action="store_true",
                    help="time the inference layer (reorder, index, forward, inverse reorder) only")
    ap.add_argument("--precision", choices=("default", "fp8"), default="default",
                    help="arithmetic of the forward (fp8: INT8 QK^T and FP8 PV; needs --forward-only)")
    ap.add_argument("--grid", type=str, default=None,
                    help="token grid T,H,W replacing the workload's (30,48,80)")
    ap.add_argument("--text", type=int, default=0,
                    help="text tokens appended to the video tokens (joint text + video step)")
    ap.add_argument("--layout", choices=("tile", "raster"), default="tile",
                    help="raster: the kernels address raster-order tensors, no reorder passes")
    ap.add_argument("--adaptive", type=str, default=None, metavar="RT,RH,RW",
                    help="choose the window shifts on device (search radius per axis) inside the step")
    ap.add_argument("--workload", choices=(WORKLOAD, "720p-shifted-perhead"), default=WORKLOAD,
                    help="720p-shifted-perhead: per-head windows and seeded window shifts (the deformable variant)")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the socket power and clock samples taken after the timed steps")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc counter_collection.csv files into profiles/traffic.json")
    return ap.parse_args()


# Kernel name fragments (as rocprofv3 reports them) -> benchmark names, and
# the sources each kernel is built from.
KERNELS = {"fwd_bf16_kernel": "fwd", "dkdv_kernel": "bwd_dkdv", "dq_kernel": "bwd_dq", "reorder_kernel": "reorder"}
KERNEL_SOURCES = {"fwd": ["fwd_bf16.hip", "tiles.h", "mfma.h", "common.h"],
                  "reorder": ["reorder.hip", "common.h"],
                  "bwd_dkdv": ["bwd_bf16.hip", "tiles.h", "mfma.h", "common.h"],
                  "bwd_dq": ["bwd_bf16.hip", "tiles.h", "mfma.h", "common.h"]}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sliding_tile_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != kernel_sources_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def write_traffic(fetch_csv, write_csv):
    """profiles/traffic.json from the FETCH_SIZE and WRITE_SIZE passes (KiB
    per dispatch), calibrated on the copy probe (a plain streaming copy)."""
    import csv
    import collections
    from tests.inputs import CONFIGS

    c = CONFIGS[WORKLOAD]
    n = int(np.prod(c["grid"]))
    copy_bytes = c["B"] * c["H"] * n * c["D"] * 2          # the copy probe reads and writes this
    means = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = collections.defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                key = "copy_probe" if "copy_probe_kernel" in name else next(
                    (v for k, v in KERNELS.items() if k in name), None)
                if key:
                    vals[key].append(float(row["Counter_Value"]) * 1024.0)
        means[counter] = {k: float(np.mean(v)) for k, v in vals.items()}
    cal = {ctr: copy_bytes / means[ctr]["copy_probe"] for ctr in means}
    out = {"_calibration": {"kernel": "copy_probe_kernel (plain streaming copy)", "bytes_per_launch": copy_bytes,
                            "FETCH_SIZE_bytes": means["FETCH_SIZE"]["copy_probe"],
                            "WRITE_SIZE_bytes": means["WRITE_SIZE"]["copy_probe"],
                            "fetch_factor": cal["FETCH_SIZE"], "write_factor": cal["WRITE_SIZE"]}}
    for key in KERNELS.values():
        fb = means["FETCH_SIZE"][key] * cal["FETCH_SIZE"]
        wb = means["WRITE_SIZE"][key] * cal["WRITE_SIZE"]
        out[key] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                    "source_digest": kernel_sources_digest(KERNEL_SOURCES[key])}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(w, rows, n_text=0):
    """The plain CPU oracle on a bounded sample of the same workload: forward
    and dQ for `rows` query rows plus dK/dV for `rows` key rows of head 0,
    counted as `rows` rows of the training step.  Query rows are the first
    rows (tile order) of the first query tiles; key rows those of the first
    key tiles that exactly 45 query tiles attend, so every sampled row meets
    45 tiles of keys (or queries), as the average row of the workload does
    (plus the n_text text keys or queries of a joint sequence)."""
    from oracle import oracle    # test infrastructure: only this leg of the benchmark uses it
    B, H, S, D = w["q"].shape
    N = S - n_text
    L = int(np.prod(w["tile"]))
    oracle.load()
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))       # tile-order slot -> raster token
    T = N // L
    _, _, _, q_cnt = oracle.index(w["grid"], w["tile"], w["windows"][:1], None, T, T)[:4]
    q_cnt = np.asarray(q_cnt)[0]
    ktiles = np.flatnonzero(q_cnt == 45)
    nt = -(-rows // L)
    qslots = (np.arange(nt)[:, None] * L + np.arange(L)[None, :]).ravel()[:rows]
    kslots = (ktiles[:nt, None] * L + np.arange(L)[None, :]).ravel()[:rows]
    qrows, krows = np.sort(inv[qslots]), np.sort(inv[kslots])
    keys_per_row = 45 * L + n_text
    flop = rows * 3.5 * 4.0 * keys_per_row * D
    t0 = time.perf_counter()
    oracle.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"], rows=qrows, n_text=n_text)
    oracle.bwd(w["q"], w["k"], w["v"], w["dout"], w["grid"], w["tile"], w["windows"], qrows=qrows, krows=krows,
               n_text=n_text)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "head 0: forward + dQ for %d query rows (query tiles 0..%d) and dK/dV for %d key rows (key "
                      "tiles attended by 45 query tiles), counted as %d training rows of %d keys each; %.1f s wall "
                      "on %s" % (rows, nt - 1, rows, rows, keys_per_row, dt, cpu_model())}


def gemm_ceiling(torch, dev, n=8192, reps=10):
    """Attainable dense bf16 rate on this GPU: a large square torch.matmul
    (hipBLASLt), as a measured ceiling beside the published peak."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return {"value": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
            "what": "bf16 %dx%dx%d torch.matmul (hipBLASLt), mean of %d" % (n, n, n, reps)}


def copy_ceiling(torch, x, reps=10):
    """Attainable HBM rate of a plain device copy of a tensor the size of one
    attention input (torch's copy_, read + write), beside the 8 TB/s peak."""
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del y
    return {"value": round(2.0 * x.numel() * x.element_size() / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "what": "torch copy_ of %d bytes (read + write), mean of %d" % (x.numel() * x.element_size(), reps)}


def probe_lib():
    """The measurement probes (libsta_probe.so, built beside libsta)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sliding_tile_attention_amd", "libsta_probe.so"))
    lib.sta_probe_exp.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sta_probe_exp.restype = ctypes.c_int
    lib.sta_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.sta_probe_copy.restype = ctypes.c_int
    lib.sta_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sta_probe_mfma.restype = ctypes.c_int
    lib.sta_probe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sta_probe_lds.restype = ctypes.c_int
    lib.sta_probe_block_copy.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.sta_probe_block_copy.restype = ctypes.c_int
    return lib


def calibration_copy(torch, x):
    """One launch of the copy probe over x's bytes (the traffic counters'
    calibration: it reads and writes exactly that many bytes)."""
    import ctypes
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    if probe_lib().sta_probe_copy(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                  x.numel() * x.element_size(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
        raise RuntimeError("copy probe failed to launch")
    torch.cuda.synchronize()
    del y


def mfma_launcher(torch, dev, blocks=4096, iters=1024):
    """One launch of the matrix-core rate probe (v_mfma_f32_32x32x16_bf16 with
    nothing else issued; 2 workgroups of 4 waves resident per CU, 8 rounds of
    them) and the flop it executes."""
    import ctypes
    lib = probe_lib()
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def launch():
        if lib.sta_probe_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters,
                              ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("matrix-core rate probe failed to launch")
    return launch, blocks * 4.0 * iters * 16 * 32 * 32 * 16 * 2


def mfma_rate(torch, dev, reps=5):
    """Sustained dense bf16 rate of the matrix instruction the attention
    kernels use, on this board and clock, timed with HIP events (TFLOP/s)."""
    launch, flop = mfma_launcher(torch, dev)
    for _ in range(2):
        launch()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    return flop / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12


def probe_launchers(torch, dev):
    """Launch functions of the single-unit probes, each with the units one
    launch issues: the matrix instruction (flop), 16-byte LDS reads (bytes),
    exponentials (count), and 16 KB key/value block copies into LDS (bytes)
    from a 2 MB region that stays in L2 and from a 1 GB region that streams
    from HBM (3072 workgroups of 4 waves, 512 blocks each)."""
    import ctypes
    lib = probe_lib()
    stream = torch.cuda.current_stream()
    sp = lambda: ctypes.c_void_p(stream.cuda_stream)
    out = torch.empty(3072 * 256, dtype=torch.int32, device=dev)
    bufs = {"l2_copy_probe": torch.zeros(128 * 16384, dtype=torch.uint8, device=dev),
            "hbm_copy_probe": torch.zeros(65536 * 16384, dtype=torch.uint8, device=dev)}

    def checked(name, rc):
        if rc != 0:
            raise RuntimeError("%s failed to launch" % name)

    mfma, mfma_flop = mfma_launcher(torch, dev)
    calls = {"mfma_probe": (mfma, mfma_flop, "flop"),
             "lds_probe": (lambda: checked("LDS-rate probe", lib.sta_probe_lds(ctypes.c_void_p(out.data_ptr()), 2048,
                                                                               1024, sp())),
                           2048 * 256.0 * 1024 * 16 * 16, "byte"),
             "exp_probe": (lambda: checked("exponential probe", lib.sta_probe_exp(ctypes.c_void_p(out.data_ptr()),
                                                                                  2048, 1024, sp())),
                           2048 * 256.0 * 1024 * 16, "exp")}
    for name, buf in bufs.items():
        calls[name] = (lambda buf=buf, name=name: checked(name, lib.sta_probe_block_copy(
            ctypes.c_void_p(buf.data_ptr()), buf.numel(), 3072, 512, ctypes.c_void_p(out.data_ptr()), sp())),
            3072 * 512 * 16384.0, "byte")
    return calls, (out, bufs)


def timed_rate(torch, fn, units, reps=5):
    """units per second of fn (HIP events over `reps` launches)."""
    for _ in range(2):
        fn()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return units / (e0.elapsed_time(e1) / reps * 1e-3)


def block_copy_bytes(lens, lists, counts, batch, row_bytes, rows_per_wg=128):
    """Bytes an attention kernel copies from global memory into LDS in one
    launch: each workgroup (4 waves of 32 rows) of a stationary tile copies
    every block of the tiles in that tile's list, `row_bytes` per listed row
    (K and V rows for the forward and dQ; Q, dO, and the two per-row floats
    for dK/dV); lens[t] = rows of tile t, list sets shared by `batch` items."""
    total = 0.0
    for h in range(counts.shape[0]):
        for t in range(counts.shape[1]):
            total += np.ceil(lens[t] / rows_per_wg) * lens[lists[h, t, :counts[h, t]]].sum()
    return total * batch * row_bytes


def energy_model(power, probes, rates, kernels, per):
    """Energy per unit of each probe above the idle board (J), and for each
    attention kernel the power its units would draw at those energies
    against the power measured under it.  Each probe's energy is taken at the
    clock the board ran it at."""
    idle = power["idle_socket_w"]
    e = {n: (power[n]["socket_w"] - idle) / rates[n] for n in probes if power.get(n) and power[n]["socket_w"]}
    if len(e) != len(probes):
        return None
    out = {"pj_per_unit_above_idle": {n: round(e[n] * 1e12, 3) for n in probes},
           "unit": {n: probes[n][2] for n in probes},
           "probe_rate_per_s": {n: float("%.4g" % rates[n]) for n in probes},
           "probe_clock_mhz": {n: power[n]["gfx_mhz"] for n in probes}, "kernels": {}}
    # HBM blocks also pass through L2 into LDS: their extra energy is the
    # HBM probe's less the L2 probe's
    price = {"mfma_flop": e["mfma_probe"], "lds_read_bytes": e["lds_probe"], "exps": e["exp_probe"],
             "l2_to_lds_bytes": e["l2_copy_probe"], "hbm_bytes": e["hbm_copy_probe"] - e["l2_copy_probe"]}
    for name, units in kernels.items():
        if name not in per or not power.get(name) or power[name]["socket_w"] is None:
            continue
        t = per[name] * 1e-3
        watts = {u: units[u] * price[u] / t for u in units if units[u] is not None}
        out["kernels"][name] = {"units_per_launch": {u: float("%.4g" % v) for u, v in units.items() if v is not None},
                                "model_w": {u: round(w, 1) for u, w in watts.items()},
                                "model_total_w": round(sum(watts.values()), 1),
                                "measured_w_above_idle": round(power[name]["socket_w"] - idle, 1)}
    return out


def lds_rate(torch, dev, blocks=2048, iters=1024, reps=5):
    """Rate of plain conflict-free 16-byte LDS reads on this GPU (TB/s), the
    row reads that feed the attention kernels' MFMAs."""
    import ctypes
    lib = probe_lib()
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    launch = lambda: lib.sta_probe_lds(ctypes.c_void_p(out.data_ptr()), blocks, iters,
                                       ctypes.c_void_p(stream.cuda_stream))
    for _ in range(2):
        if launch() != 0:
            raise RuntimeError("LDS-rate probe failed to launch")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    return blocks * 256.0 * iters * 16 * 16 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12


def exp_rate(torch, dev, blocks=2048, iters=1024, reps=5):
    """Measured rate of the hardware exponential (v_exp_f32) on this GPU: a
    probe launch of 2048 workgroups of 256 threads, each thread 1024 rounds of
    16 independent exponentials, timed with HIP events; exponentials per
    second."""
    import ctypes
    lib = probe_lib()
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    launch = lambda: lib.sta_probe_exp(ctypes.c_void_p(out.data_ptr()), blocks, iters,
                                       ctypes.c_void_p(stream.cuda_stream))
    for _ in range(2):
        if launch() != 0:
            raise RuntimeError("exponential-rate probe failed to launch")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return blocks * 256.0 * iters * 16 / (ms * 1e-3)


def power_samples(torch, calls, seconds=2.5, settle=1.0):
    """Socket power and GFX clock while each call in `calls` (name -> fn)
    runs back to back for `seconds`, read through amdsmi (the driver's
    sensors; no GPU setting is touched).  The calls are enqueued in chunks of
    ~50 ms with the next chunk always queued, and the sensors are read only
    while a chunk is still running, so every sample sees the GPU busy with
    that call.  The power reading trails the load by up to about a second,
    so each call's samples of its first `settle` seconds are dropped, and the
    idle reading is the mean over half a second taken 1.5 s after the GPU
    went idle.  Means, with the board's power limit; None where amdsmi is
    missing or fails."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        hd = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None

    def read():
        p = amdsmi.amdsmi_get_power_info(hd)
        c = amdsmi.amdsmi_get_clock_info(hd, amdsmi.AmdSmiClkType.GFX)
        return float(p["current_socket_power"]), float(c["clk"]), p.get("power_limit")

    try:
        torch.cuda.synchronize()
        time.sleep(1.5)
        idle = []
        for _ in range(10):
            idle.append(read())
            time.sleep(0.05)
        limit = idle[-1][2]
        out = {"idle_socket_w": round(float(np.mean([g[0] for g in idle])), 1),
               "power_limit_w": float(limit) / 1e6 if isinstance(limit, (int, float)) else None}
        for name, fn in calls.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            chunk = max(1, int(50.0 / max(e0.elapsed_time(e1), 1e-3)))
            t0, got, running = time.time(), [], None
            while time.time() - t0 < seconds:
                for _ in range(chunk):
                    fn()
                queued = torch.cuda.Event()
                queued.record()
                if running is not None:
                    while not running.query():
                        if time.time() - t0 >= settle:
                            got.append(read()[:2])
                        time.sleep(0.005)
                running = queued
            torch.cuda.synchronize()
            out[name] = {"socket_w": round(float(np.mean([g[0] for g in got])), 1) if got else None,
                         "gfx_mhz": round(float(np.mean([g[1] for g in got])), 1) if got else None,
                         "samples": len(got)}
        return out
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the sliding-tile attention path here has no multi-GPU "
              "mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_tile_attention_amd as sta
    from tests.inputs import workload

    nt = args.text
    if nt < 0:
        print("--text must be >= 0", file=sys.stderr)
        sys.exit(2)
    if args.precision == "fp8" and not args.forward_only:
        print("--precision fp8 measures the forward only: add --forward-only", file=sys.stderr)
        sys.exit(2)
    fwd_only = args.forward_only
    prec = sta.STA_PREC_FP8 if args.precision == "fp8" else sta.STA_PREC_DEFAULT
    grid = None if args.grid is None else tuple(int(x) for x in args.grid.split(","))
    shifted = args.workload != WORKLOAD
    if shifted and (nt or grid or args.adaptive or args.layout == "raster"):
        print("--workload %s takes none of --text, --grid, --adaptive, --layout raster" % args.workload,
              file=sys.stderr)
        sys.exit(2)
    w = workload(args.workload, n_text=nt, grid=grid, with_dout=True)
    B, H, S, D = w["q"].shape
    N = S - nt
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
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    radius = None if args.adaptive is None else tuple(int(x) for x in args.adaptive.split(","))
    off = None if radius is None else torch.zeros((H, T, 3), dtype=torch.int32, device=dev)
    if shifted:                                     # the workload's seeded shifts, shared by the heads
        off = torch.from_numpy(np.ascontiguousarray(w["offsets"], np.int32)).to(dev)
    idx = sta.StaIndex(geom, windows, off)          # with shifts: per-head capacity
    scale = D ** -0.5
    row_bytes = D * 2
    stream = torch.cuda.current_stream()

    raster = args.layout == "raster"
    if raster and (nt or radius):
        print("--layout raster takes video rows only and no --adaptive", file=sys.stderr)
        sys.exit(2)
    lay = sta.STA_LAYOUT_RASTER if raster else sta.STA_LAYOUT_TILE
    if raster:
        names = ["index", "fwd"] + ([] if fwd_only else ["bwd_delta", "bwd_dkdv", "bwd_dq"])
    else:
        names = ["reorder_qkv"] + (["shifts"] if radius else []) + ["index", "fwd", "reorder_o"]
        if not fwd_only:
            names += ["reorder_do", "bwd_delta", "bwd_dkdv", "bwd_dq", "reorder_grads"]

    def raster_step(evs=None):
        marks = iter(range(len(names) + 1))

        def mark():
            i = next(marks)
            if evs is not None:
                evs[i].record(stream)
        mark()
        sta.sta_build_index(geom, windows, None, idx, stream)
        mark()
        sta.sta_fwd_ex(q, k, v, o, lse, B, H, D, sta.STA_BF16, scale, geom, idx, 0, stream, prec, lay)
        mark()
        if fwd_only:
            return
        for part in (sta.STA_BWD_DELTA, sta.STA_BWD_DKDV, sta.STA_BWD_DQ):
            sta.sta_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, D, sta.STA_BF16, scale, geom, idx, part, 0,
                           stream, lay)
            mark()

    def step(evs=None):
        if raster:
            return raster_step(evs)
        marks = iter(range(len(names) + 1))

        def mark():
            i = next(marks)
            if evs is not None:
                evs[i].record(stream)
        mark()
        for src, dst in ((q, qt), (k, kt), (v, vt)):
            sta.sta_tile_reorder_ex(src, dst, B * H, row_bytes, geom, False, nt, stream)
        mark()
        if radius:
            sta.sta_window_shifts(qt, kt, B, H, D, sta.STA_BF16, scale, geom, windows, radius, off, "shift", False,
                                  nt, stream)
            mark()
            sta.sta_build_index_ex(geom, windows, off, idx, "shift", True, stream)
        else:
            sta.sta_build_index(geom, windows, off, idx, stream)
        mark()
        sta.sta_fwd_ex(qt, kt, vt, ot, lse, B, H, D, sta.STA_BF16, scale, geom, idx, nt, stream, prec)
        mark()
        sta.sta_tile_reorder_ex(ot, o, B * H, row_bytes, geom, True, nt, stream)
        mark()
        if fwd_only:
            return
        sta.sta_tile_reorder_ex(do, dot_, B * H, row_bytes, geom, False, nt, stream)
        mark()
        for part in (sta.STA_BWD_DELTA, sta.STA_BWD_DKDV, sta.STA_BWD_DQ):
            sta.sta_bwd_ex(qt, kt, vt, ot, lse, dot_, dqt, dkt, dvt, delta, B, H, D, sta.STA_BF16, scale, geom,
                           idx, part, nt, stream)
            mark()
        for src, dst in ((dqt, dq), (dkt, dk), (dvt, dv)):
            sta.sta_tile_reorder_ex(src, dst, B * H, row_bytes, geom, True, nt, stream)
        mark()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
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
    kv_idx = idx.kv_idx.cpu().numpy()
    # counted: unmasked tile pairs, len(q) * len(k) scores each (L * L unless
    # a tile is cut by the grid border)
    axes = [[min(t, g - i * t) for i in range(-(-g // t))] for g, t in zip(geom.grid, geom.tile)]
    lens = np.einsum("a,b,c->abc", *[np.array(x, np.float64) for x in axes]).ravel()
    pairs = sum(float(lens[q] * lens[kv_idx[h, q, :kv_cnt[h, q]]].sum())
                for h in range(kv_cnt.shape[0]) for q in range(kv_cnt.shape[1]))
    fwd_flop = 4.0 * B * pairs * D
    fwd_flop += 4.0 * B * H * D * float(nt) * (2 * N + nt)          # text rows and columns (joint step)
    step_flop = fwd_flop if fwd_only else 3.5 * fwd_flop            # forward + backward (2.5x)
    value = step_flop / (ms_per_step * 1e-3) / 1e12

    # Algorithmic work of each attention kernel (flop per launch): the forward
    # does QK^T and PV (4 L^2 D per pair); dK/dV must form S, dP, dV and dK
    # (8 L^2 D); dQ adds only the dQ product (2 L^2 D; its S and dP are
    # recomputation).  Together the backward is 10 L^2 D = 2.5x the forward.
    alg = {"fwd": fwd_flop} if fwd_only else {"fwd": fwd_flop, "bwd_dkdv": 2.0 * fwd_flop, "bwd_dq": 0.5 * fwd_flop}
    peak = PEAK_FP8_TFLOPS if prec == sta.STA_PREC_FP8 else PEAK_BF16_TFLOPS
    default_step = (nt == 0 and grid is None and prec == sta.STA_PREC_DEFAULT and radius is None and not raster
                    and not shifted)
    dominant = max(alg, key=lambda n: per[n])
    achieved = alg[dominant] / (per[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "kernel": dominant,
                "traffic": measured_traffic(dominant) if default_step else None,  # counters cover the default step
                "measured_gemm_ceiling": gemm_ceiling(torch, dev)}

    calibration_copy(torch, q)
    power = None
    if not args.no_power:
        if raster:
            calls = {"fwd": lambda: sta.sta_fwd_ex(q, k, v, o, lse, B, H, D, sta.STA_BF16, scale, geom, idx, 0, stream,
                                                   prec, lay)}
            bwd_args = (q, k, v, o, lse, do, dq, dk, dv, delta)
        else:
            calls = {"fwd": lambda: sta.sta_fwd_ex(qt, kt, vt, ot, lse, B, H, D, sta.STA_BF16, scale, geom, idx, nt,
                                                   stream, prec)}
            bwd_args = (qt, kt, vt, ot, lse, dot_, dqt, dkt, dvt, delta)
        if not fwd_only:
            for name, part in (("bwd_dkdv", sta.STA_BWD_DKDV), ("bwd_dq", sta.STA_BWD_DQ)):
                calls[name] = (lambda part=part: sta.sta_bwd_ex(*bwd_args, B, H, D, sta.STA_BF16, scale, geom, idx,
                                                               part, 0 if raster else nt, stream, lay))
        ga = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        calls["gemm_8192"] = lambda: torch.matmul(ga, gb)
        probes, probe_bufs = probe_launchers(torch, dev)
        for name, (fn, _, _) in probes.items():
            calls[name] = fn
        power = power_samples(torch, calls)
        del ga, gb
    scores = fwd_flop / (4.0 * D)
    rate = exp_rate(torch, dev)
    exp_bound = {"exps_per_fwd": scores, "measured_exp_rate_per_s": round(rate, -6),
                 "exp_ms_at_that_rate": round(scores / rate * 1e3, 3),
                 "share_of_fwd_kernel": round(scores / rate * 1e3 / per["fwd"], 4)}
    mrate = mfma_rate(torch, dev)
    matrix_core = {"instr": "v_mfma_f32_32x32x16_bf16", "chain_rate_tflops": round(mrate, 1),
                   "fwd_share_of_it": round(fwd_flop / (per["fwd"] * 1e-3) / 1e12 / mrate, 4)}
    # every bf16 attention kernel reads one 1 KB operand fragment from LDS
    # per 32x32x16 MFMA it executes (32768 flop): LDS bytes = executed flop / 32
    executed = {"fwd": fwd_flop, "bwd_dkdv": 2.0 * fwd_flop, "bwd_dq": 1.5 * fwd_flop}
    lds = {"probe_ds_read_b128_tbs": round(lds_rate(torch, dev), 1),
           "kernels_tbs": {n: round(f / 32.0 / (per[n] * 1e-3) / 1e12, 1) for n, f in executed.items() if n in per}}
    # energy per unit of each probe, and what the attention kernels' units
    # would draw at those energies (video rows only: text rows take other
    # walks; the quantized forward issues other instructions)
    energy = None
    if power is not None and nt == 0 and prec == sta.STA_PREC_DEFAULT:
        rates = {n: timed_rate(torch, fn, u) for n, (fn, u, _) in probes.items()}
        batch = B if idx.num_heads == H else 1
        fwd_copy = block_copy_bytes(lens, kv_idx, kv_cnt, batch, 4 * D)
        scores = fwd_flop / (4.0 * D)
        hbm = lambda n: measured_traffic(n) if default_step else None
        kernels = {"fwd": {"mfma_flop": fwd_flop, "lds_read_bytes": fwd_flop / 32.0, "l2_to_lds_bytes": fwd_copy,
                           "hbm_bytes": hbm("fwd"), "exps": scores}}
        if not fwd_only:
            dkdv_copy = block_copy_bytes(lens, idx.q_idx.cpu().numpy(), idx.q_cnt.cpu().numpy(), batch, 4 * D + 8)
            kernels["bwd_dkdv"] = {"mfma_flop": 2.0 * fwd_flop, "lds_read_bytes": 2.0 * fwd_flop / 32.0,
                                   "l2_to_lds_bytes": dkdv_copy, "hbm_bytes": hbm("bwd_dkdv"), "exps": scores}
            kernels["bwd_dq"] = {"mfma_flop": 1.5 * fwd_flop, "lds_read_bytes": 1.5 * fwd_flop / 32.0,
                                 "l2_to_lds_bytes": fwd_copy, "hbm_bytes": hbm("bwd_dq"), "exps": scores}
        energy = energy_model(power, probes, rates, kernels, per)
    probes = probe_bufs = None                      # frees the probes' source regions
    tensor_bytes = B * H * S * D * 2
    reorder_gbs = 3 * 2 * tensor_bytes / (per["reorder_qkv"] * 1e-3) / 1e9 if "reorder_qkv" in per else None
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
        "dtype": "int8 QK^T + e4m3 PV, bf16 I/O" if prec == sta.STA_PREC_FP8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("720p %s: B=1 H=24 D=128, grid (%d,%d,%d)=%d tokens, tile (6,8,8), %s, %s" % (
                ("deformable-window step" if shifted else "training step",) + tuple(geom.grid) + (N,
                "per-head windows %s and a seeded shift per query tile (%d head-tile pairs listed)" % (
                    "/".join("%dx%dx%d" % c for c in sorted(set(windows))), int(kv_cnt.sum()))
                if shifted else "window 3x3x5 tiles", "forward only" if fwd_only else "forward+backward"))) +
                        ("" if nt == 0 else ", joint with %d text tokens (dense text rows and columns)" % nt) +
                        ("" if radius is None else ", window shifts chosen on device (search radius %s tiles)"
                         % (radius,)) + (", raster layout (no reorder passes)" if raster else ""),
            "global_batch": B,
            "seq_len": S,
            "text_tokens": nt,
            "parallelism": "none (1 GPU)",
            "counted_flop_per_step": step_flop,
            "ms_per_layer_fwd_bwd": round(ms_per_step, 3),
            "ms_per_layer_fwd": round(per.get("reorder_qkv", 0.0) + per.get("shifts", 0.0) + per["index"] + per["fwd"] +
                                      per.get("reorder_o", 0.0), 3),
            "fwd_kernel_ms": round(per["fwd"], 3),
            "fwd_tflops": round(fwd_flop / (per["fwd"] * 1e-3) / 1e12, 1),
            "fwd_frac_of_peak": round(fwd_flop / (per["fwd"] * 1e-3) / 1e12 / peak, 4),
            "bwd_kernels_ms": None if fwd_only else round(per["bwd_delta"] + per["bwd_dkdv"] + per["bwd_dq"], 3),
            "reorder_qkv_gbs": None if reorder_gbs is None else round(reorder_gbs, 1),
            # HBM bytes of one reorder launch from the counters (the
            # algorithmic figure is 2 * one input: read once, written once)
            "reorder_traffic_per_launch": measured_traffic("reorder") if default_step else None,
            "reorder_algorithmic_bytes": 2 * tensor_bytes,
            "measured_copy_ceiling": copy_ceiling(torch, q),
            # the producer reads Q and K once (its tile means); the choice
            # itself touches only the means
            "shifts_hbm_gbs": None if radius is None else round(2 * B * H * N * D * 2 / (per["shifts"] * 1e-3) / 1e9,
                                                               1),
            "per_call_ms": {n: round(t, 4) for n, t in per.items()},
            # the forward's secondary bound: one hardware exponential per
            # counted score (the lazy-max rule redoes a fraction of a percent)
            "exp_bound": exp_bound,
            # what the matrix cores alone sustain on this board (the probe
            # issues nothing but the attention kernels' MFMA, on operands
            # that change every instruction); its power and clock are in
            # `power` under mfma_probe
            "matrix_core_rate": matrix_core,
            # LDS operand reads of the attention kernels against a plain
            # stream of the same reads (the LDS port is not their limit
            # while the first stays well below the second)
            "lds_read": lds,
            # socket power and GFX clock while each call runs back to back
            # (after the timed steps; amdsmi sensors)
            "power": power,
            # energy per unit from the probes above, and each kernel's units
            # priced at them against its measured power (the rest of the
            # vector work is not priced)
            "energy": energy,
        },
        "roofline": roofline,
    }
    if (not args.no_cpu_baseline and grid is None and not fwd_only and radius is None and not raster
            and not shifted):                                           # a sample of the training step
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows, nt)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

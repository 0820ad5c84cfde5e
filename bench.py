#!/usr/bin/env python3
"""Benchmark of the SubMConv3d hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3a] [--no-cpu-baseline]

One step = the whole hot path over one coordinate set already resident in HBM:
build the indice map (hash insert + 27-neighbour lookup + one sync for the
error flags), run every convolution layer of the workload on it, free the map.
The default workload is the 128^3 sphere shell (r = 60, thickness 3; 135,826
voxels), 128 -> 128 channels, bf16 storage, k = 3.

Printed: one JSON line with the step throughput (effective TFLOP/s =
2 * pairs * Cin * Cout per layer, summed over layers, divided by the step
time), the roofline position of the convolution kernel (its average duration
from HIP events around back-to-back launches on the stream it runs on), and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SubMConv3d ms + effective TFLOP/s at 128^3 grid, 128ch bf16 (1 GPU)"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
ELEM = {"bf16": 2, "f16": 2, "f32": 4}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv_traffic.json")
CONV_SOURCE = os.path.join(ROOT, "submanifold_sparse_convolution_amd", "csrc", "conv.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="3a", help="1, 2a (k3 + k1 layer), 3a, 3b, 4, 5")
    p.add_argument("--conv-reps", type=int, default=200, help="back-to-back launches timed for the roofline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target duration of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run 5 plain device copies of MIB MiB (reference for hardware byte counters)")
    return p.parse_args()


def copy_calibration(mib):
    """Five plain device-to-device copies of a known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_copy": n * 4, "copies": 5}), flush=True)


def layer_plan(key):
    """[(ksize, cin, cout, seed_layer)] and whether layers are chained."""
    import synth
    c = synth.config(key)
    if key == "2a":
        return [(3, c.cin, c.cout, 0), (1, c.cin, c.cout, 1)], False
    return [(c.ksize, c.cin, c.cout, l) for l in range(c.layers)], c.chained


def source_hash(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def load_traffic(key, kernel_hash):
    """HBM bytes per conv launch from committed rocprofv3 PMC runs, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = data.get(key)
    if not entry or entry.get("conv_source_sha256") != kernel_hash:
        return None
    return entry.get("bytes_per_launch")


def cpu_baseline(key, coords, feats, weight, bias, nbr_pairs_per_row, cin, cout, budget_s):
    """The oracle as it stands, single-threaded, on a row sample sized to ~budget_s seconds."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    f64 = feats.double().numpy()
    w64 = weight.double().numpy()
    b64 = bias.double().numpy()
    n = coords.shape[0]
    rng = np.random.default_rng(12345)
    with threadpool_limits(limits=1):
        # Two calibration calls fit cost = fixed (dictionary build) + per_row * rows; then one
        # timed call sized to the budget.
        def run(k):
            sel = rng.choice(n, size=min(n, k), replace=False)
            t0 = time.perf_counter()
            oracle.conv3(coords, f64, w64, b64, rows=sel)
            return time.perf_counter() - t0
        t_a, t_b = run(64), run(512)
        per_row = max((t_b - t_a) / (512 - 64), 1e-7)
        fixed = max(t_a - 64 * per_row, 0.0)
        rows_target = int(min(n, max(256, (budget_s - fixed) / per_row)))
        rows = rng.choice(n, size=rows_target, replace=False)
        t0 = time.perf_counter()
        oracle.conv3(coords, f64, w64, b64, rows=rows)
        elapsed = time.perf_counter() - t0
    pairs = int(nbr_pairs_per_row[rows].sum())
    flops = 2.0 * pairs * cin * cout
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"oracle.conv3 (float64 dictionary lookup + per-voxel loop, 1 thread) on {rows_target} random "
                   f"of {n} output rows of workload {key} ({pairs} pairs), including its dictionary build over "
                   f"all {n} rows; {elapsed:.2f} s"),
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the submanifold convolution path here is a single-GPU "
              "build (see the sharding paragraph of the design notes); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import submanifold_sparse_convolution_amd as sc
    import synth

    key = args.workload
    cfg = synth.config(key)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sc.load_library()

    coords_np = synth.coords_for(key)
    n = coords_np.shape[0]
    plan, chained = layer_plan(key)
    coords = torch.from_numpy(coords_np).to(dev)
    x0 = synth.feats_for(cfg.number, 0, n, plan[0][1], cfg.dtype)
    layers = []
    for ks, cin, cout, l in plan:
        w = synth.weight_for(cfg.number, l, ks, cin, cout, cfg.dtype)
        b = synth.bias_for(cfg.number, l, cout, cfg.dtype)
        layers.append((ks, cin, cout, w.to(dev), b.to(dev), w, b))
    x0_dev = x0.to(dev)
    outs = [torch.empty((n, cout), dtype=x0_dev.dtype, device=dev) for (_, _, cout, *_r) in layers]

    def step():
        m = sc.sparse_indice_map_build(coords)
        x = x0_dev
        for (ks, cin, cout, w, b, _, _), out in zip(layers, outs):
            sc.subm_conv3d_forward(m if ks == 3 else None, x, w, b, out=out)
            if chained:
                x = out
        m.free()
        return m

    # Pair counts (from the GPU map; the parity tests pin them to the oracle).
    with sc.sparse_indice_map_build(coords) as m0:
        pairs = m0.pairs
        nbr_rows = (sc.sparse_indice_map_copy_nbr(m0) >= 0).sum(dim=1).cpu().numpy()
    flops_per_step = sum(2.0 * (pairs if ks == 3 else n) * cin * cout for ks, cin, cout, *_ in layers)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps

    # Map build alone (includes its one stream synchronisation).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        sc.sparse_indice_map_build(coords).free()
    torch.cuda.synchronize()
    build_s = (time.perf_counter() - t0) / args.steps

    # Convolution kernel alone: HIP events around each of many back-to-back launches on the
    # stream the library launches on (torch's current stream, passed through the binding).
    stream = torch.cuda.current_stream(dev)
    conv_ms = []
    with sc.sparse_indice_map_build(coords) as m:
        k3 = [(ks, cin, cout, w, b) for ks, cin, cout, w, b, _, _ in layers]
        reps = max(args.conv_reps, len(k3))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for r in range(min(reps, 20)):  # warm
            ks, cin, cout, w, b = k3[r % len(k3)]
            sc.subm_conv3d_forward(m if ks == 3 else None, x0_dev if not chained else outs[0], w, b, out=outs[-1])
        torch.cuda.synchronize()
        per_layer = {i: [] for i in range(len(k3))}
        for r in range(reps):
            i = r % len(k3)
            ks, cin, cout, w, b = k3[i]
            src = x0_dev if not chained else outs[0]
            evs[r][0].record(stream)
            sc.subm_conv3d_forward(m if ks == 3 else None, src, w, b, out=outs[-1])
            evs[r][1].record(stream)
        torch.cuda.synchronize()
        for r in range(reps):
            per_layer[r % len(k3)].append(evs[r][0].elapsed_time(evs[r][1]))
    # Dominant kernel: the k = 3 layer (all layers of a workload share shape except 2a's k = 1).
    dom = 0
    conv_ms = float(np.mean(per_layer[dom]))
    ks, cin, cout = layers[dom][0], layers[dom][1], layers[dom][2]
    s = ELEM[cfg.dtype]
    p_layer = pairs if ks == 3 else n
    flop_launch = 2.0 * p_layer * cin * cout
    bytes_launch = float(n * cin * s + n * cout * s + ks ** 3 * cin * cout * s + cout * s + (n * 27 * 4 if ks == 3 else 0))
    t_mfma = flop_launch / (PEAK_TFLOPS[cfg.dtype] * 1e12)
    t_hbm = bytes_launch / (PEAK_HBM_GBS * 1e9)
    conv_s = conv_ms / 1e3
    kernel_hash = source_hash(CONV_SOURCE)
    traffic = load_traffic(key, kernel_hash)
    if t_mfma >= t_hbm:
        achieved = flop_launch / conv_s / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS[cfg.dtype], "unit": "TFLOP/s",
                    "frac": achieved / PEAK_TFLOPS[cfg.dtype], "traffic": traffic}
    else:
        achieved = bytes_launch / conv_s / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    # The kernel the library picks for this layer shape (16-bit storage: the warp-specialised
    # matrix-core kernel above 32 output channels, the single-role one from 17 to 32).
    if cfg.dtype in ("bf16", "f16") and cout > 32:
        kernel = "subm_conv_ws_kernel"
    elif cfg.dtype in ("bf16", "f16") and cout > 16:
        kernel = "subm_conv_mma_kernel"
    else:
        kernel = "subm_conv_generic_kernel"
    roofline.update({"kernel": kernel, "avg_launch_ms": conv_ms, "launches": len(per_layer[dom]),
                     "algorithmic_flop_per_launch": flop_launch, "algorithmic_bytes_per_launch": bytes_launch})

    value = flops_per_step / step_s / 1e12
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.workload, "key": key, "batch": cfg.batch, "grid": cfg.grid, "voxels": n,
                   "pairs": pairs, "cin": cfg.cin, "cout": cfg.cout,
                   "layers": [f"k{ks} {ci}->{co}" for ks, ci, co, *_ in layers], "chained": chained},
        "roofline": roofline,
        "breakdown": {"map_build_ms": build_s * 1e3,
                      "conv_ms_per_layer": {str(i): float(np.mean(v)) for i, v in per_layer.items()},
                      "conv_tflops_effective": flop_launch / conv_s / 1e12,
                      "voxels_per_s_step": n / step_s,
                      "voxels_per_s_conv": n / conv_s},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        ks, cin, cout, _, _, w_cpu, b_cpu = layers[dom]
        result["cpu_baseline"] = cpu_baseline(key, coords_np, x0, w_cpu, b_cpu, nbr_rows, cin, cout,
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the SubMConv3d hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3a] [--no-cpu-baseline]
    python bench.py --op per-offset|subdivide|downsample|groupnorm|conv-groupnorm [...]

One step = the whole hot path over one coordinate set already resident in HBM:
build the indice map (hash insert + 27-neighbour lookup + one sync for the
error flags), run every convolution layer of the workload on it, free the map.
The default workload is the 128^3 sphere shell (r = 60, thickness 3; 135,826
voxels), 128 -> 128 channels, bf16 storage, k = 3.

Printed: one JSON line with the step throughput (effective TFLOP/s =
2 * pairs * Cin * Cout per layer, summed over layers, divided by the step
time), the roofline position of the convolution kernel (its average duration
over back-to-back calls, from a pair of HIP events bound to the kernel's own
dispatch through subm_timing_events; the whole call, which on the
neighbour-pool path also packs the weights, is reported beside it), the same
kernel with cold caches (1 GiB written between calls), the map build's GPU time
from events, and the CPU
oracle timed on a bounded sample of the same workload in one process per
host core (at most 16).

--op selects another row of the path, each printed as one JSON line of its own:
per-offset (the same convolution computed offset by offset: gather -> GEMM ->
scatter-add), subdivide (children, their features and the derived child map of
the config-5 structure at its last level), downsample (2x cells, max pooling
and the cache-paired upsample of the config-5 coordinate set), groupnorm
(group normalisation + SiLU over the config-5 set, 64 channels, 32 groups) and
conv-groupnorm (one config-5 layer followed by that normalisation, with the
statistics taken in the convolution's epilogue, timed beside conv + norm).
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
CSRC = os.path.join(ROOT, "submanifold_sparse_convolution_amd", "csrc")
MALL_FLUSH_BYTES = 1 << 30  # written between launches for the cold-cache timing (MALL: 256 MB)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="3a", help="1, 2a (k3 + k1 layer), 3a, 3b, 4, 5")
    p.add_argument("--op", default="conv",
                   choices=["conv", "per-offset", "subdivide", "downsample", "groupnorm", "conv-groupnorm"])
    p.add_argument("--conv-reps", type=int, default=200, help="back-to-back launches timed for the roofline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peaks", action="store_true", help="skip the measured GEMM and copy ceilings")
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


def measured_peaks(dev):
    """This GPU's measured ceilings, beside the published ones: a large bf16 GEMM (hipBLASLt
    through torch.matmul, contiguous 2-D operands), a 1 GiB device-to-device copy, and the
    library's loop of register-operand bf16 MFMAs with the clock it ran at."""
    import torch
    out = {}
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    out["bf16_gemm_TFLOPs"] = 10 * 2.0 * m ** 3 / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["copy_GBps"] = 10 * 2.0 * (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    # The matrix cores alone: back-to-back bf16 MFMAs on register operands, one workgroup per CU,
    # and the shader clock they ran at (s_memtime against the 100 MHz s_memrealtime).
    import submanifold_sparse_convolution_amd as sc
    blocks, iters = 256, 40000
    sc.subm_mfma_rate(iters // 10, blocks)  # warm
    torch.cuda.synchronize()
    e0.record()
    _, clocks = sc.subm_mfma_rate(iters, blocks)
    e1.record()
    torch.cuda.synchronize()
    flop = blocks * 4 * iters * 8 * 32768.0
    out["mfma_loop_TFLOPs"] = flop / (e0.elapsed_time(e1) / 1e3) / 1e12
    c = clocks.view(-1, 2).double().cpu()
    out["mfma_loop_clock_GHz"] = float(c[:, 0].sum() / c[:, 1].sum() * 0.1)
    torch.cuda.empty_cache()
    return out


def load_traffic(key, source, kernel_hash):
    """HBM bytes per conv call from committed rocprofv3 PMC runs, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = data.get(key)
    if not entry or entry.get("kernel_source") != source or entry.get("source_sha256") != kernel_hash:
        return None
    return entry.get("bytes_per_launch")


def _oracle_inputs(key, layer, cin, cout):
    import synth
    c = synth.config(key)
    coords = synth.coords_for(key)
    f = synth.feats_for(c.number, 0, len(coords), cin, c.dtype).double().numpy()
    w = synth.weight_for(c.number, layer, 3, cin, cout, c.dtype).double().numpy()
    b = synth.bias_for(c.number, layer, cout, c.dtype).double().numpy()
    return coords, f, w, b


def _oracle_worker(task):
    """One host process: the oracle on its share of the sampled rows, one thread.  Returns the
    seconds of that call and of a one-row call after it (its dictionary build, under the same load
    from the other processes); a first one-row call warms the process up untimed."""
    key, layer, cin, cout, rows = task
    from threadpoolctl import threadpool_limits

    import oracle
    coords, f, w, b = _oracle_inputs(key, layer, cin, cout)
    with threadpool_limits(limits=1):
        oracle.conv3(coords, f, w, b, rows=rows[:1])  # (first call of the process: not timed)
        t0 = time.perf_counter()
        oracle.conv3(coords, f, w, b, rows=rows)
        t1 = time.perf_counter()
        oracle.conv3(coords, f, w, b, rows=rows[:1])
        return t1 - t0, time.perf_counter() - t1


def host_cores():
    """Host cores this process may use, at most 16 (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(key, layer, coords, nbr_pairs_per_row, cin, cout, budget_s):
    """The oracle as it stands (dictionary lookup + per-voxel loop, float64) on P host processes,
    one thread each, each on its share of a random row sample sized to ~budget_s seconds; and the
    same oracle's one-core time for the whole layer, estimated from that run."""
    import multiprocessing

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    n = coords.shape[0]
    procs = host_cores()
    rng = np.random.default_rng(12345)
    _, f64, w64, b64 = _oracle_inputs(key, layer, cin, cout)
    with threadpool_limits(limits=1):
        # Calibration on one core, cost = fixed (the dictionary build over all rows) + per_row *
        # rows: a one-row call gives the fixed part, a 256-row call a first per-row figure that
        # only sizes the sample below (on large sets the fixed part's noise can swamp it).
        def run(k):
            sel = rng.choice(n, size=min(n, k), replace=False)
            t0 = time.perf_counter()
            oracle.conv3(coords, f64, w64, b64, rows=sel)
            return time.perf_counter() - t0
        fixed = run(1)
        k256 = min(n, 256)
        per_row = max((run(k256) - fixed) / max(k256 - 1, 1), 1e-6)
    # (at least 50,000 rows per process where the set has them, so that the per-row work of
    # each process dominates the noise of its dictionary builds)
    rows_each = int(max(256, (budget_s - fixed) / per_row, min(n // procs, 50000)))
    rows = rng.choice(n, size=min(n, rows_each * procs), replace=False)
    chunks = np.array_split(rows, procs)
    ctx = multiprocessing.get_context("spawn")  # no fork of a process that holds the GPU
    with ctx.Pool(procs) as pool:
        res = pool.map(_oracle_worker, [(key, layer, cin, cout, c) for c in chunks])
    secs = [r[0] for r in res]
    elapsed = max(secs)
    pairs = int(nbr_pairs_per_row[rows].sum())
    flops = 2.0 * pairs * cin * cout
    # One core on the whole layer: the dictionary build of the one-row call alone plus every row
    # at the per-row cost the sampled processes measured, each on one core: their call less their
    # own one-row call (the processes run at once and share the host's memory, so the estimate
    # leans slow).
    per_row_mp = max(float(np.mean([(t - t1) / max(len(c) - 1, 1) for (t, t1), c in zip(res, chunks)])), 1e-9)
    layer_one_core_s = fixed + n * per_row_mp
    layer_flops = 2.0 * float(nbr_pairs_per_row.sum()) * cin * cout
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": procs,
        "kind": "oracle",
        "sample": (f"oracle.conv3 (float64 dictionary lookup + per-voxel loop) in {procs} host processes of "
                   f"1 thread, on {len(rows)} random of {n} output rows of workload {key} ({pairs} pairs), each "
                   f"process building the dictionary over all {n} rows; slowest process {elapsed:.2f} s"),
        "single_core": {
            "value": layer_flops / layer_one_core_s / 1e12,
            "unit": "TFLOP/s",
            "layer_s": layer_one_core_s,
            "fit": (f"dictionary build {fixed:.3f} s (one process alone, one output row) + {per_row_mp * 1e6:.1f} us "
                    f"per row (the sampled processes' mean, each less its own one-row call), extrapolated to all {n} rows"),
        },
    }


def per_offset_bytes(n, pairs, cin, cout, s):
    """Algorithmic bytes of one per-offset convolution: every pair reads its input row, the
    weights once, the pair indices, the float32 accumulator rows (written by the centre offset,
    read and written by every other pair, read by the final rounding) and the output."""
    return float(pairs * cin * s + 27 * cin * cout * s + (pairs - n) * 8 + n * cout * 4
                 + (pairs - n) * cout * 8 + n * cout * 4 + n * cout * s)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the submanifold convolution path here is a single-GPU "
              "build (see the sharding paragraph of the design notes); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.op in ("subdivide", "downsample", "groupnorm", "conv-groupnorm"):
        bench_structure(args)
        return
    per_offset = args.op == "per-offset"

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

    def conv(m, ks, x, w, b, out):
        if per_offset and ks == 3:
            return sc.subm_conv3d_forward_per_offset(m, x, w, b, out=out)
        return sc.subm_conv3d_forward(m if ks == 3 else None, x, w, b, out=out)

    # One step: the map build, enqueued with no host wait, then every layer behind it on the
    # same stream; the build's coordinate check (duplicates, ranges) follows the enqueued layers,
    # so the host never stands between the build and the convolutions.
    def step():
        m = sc.sparse_indice_map_build(coords, sync=False)
        x = x0_dev
        for (ks, cin, cout, w, b, _, _), out in zip(layers, outs):
            conv(m, ks, x, w, b, out)
            if chained:
                x = out
        m.check()
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

    # Spread of single steps (outside the timed block): an event on the stream before each step,
    # so consecutive events bracket one step on the GPU timeline.
    stream0 = torch.cuda.current_stream(dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.steps):
        marks[i].record(stream0)
        step()
    marks[-1].record(stream0)
    torch.cuda.synchronize()
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])

    if per_offset:
        # The step above builds a new map every time, so each per-offset call also built that
        # map's pair lists (and synchronised once); the kernel timing below reuses one map.
        pass
    # Map build alone, GPU time: events around the enqueue of each build (no host wait inside).
    stream0.synchronize()
    bmarks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    built = []
    for e0, e1 in bmarks:
        e0.record(stream0)
        built.append(sc.sparse_indice_map_build(coords, sync=False))
        e1.record(stream0)
    torch.cuda.synchronize()
    for m in built:
        m.check()
        m.free()
    build_s = float(np.mean([e0.elapsed_time(e1) for e0, e1 in bmarks])) / 1e3

    # Convolution kernel alone over many back-to-back calls on the stream the library launches
    # on (torch's current stream, passed through the binding).
    stream = torch.cuda.current_stream(dev)
    conv_ms = []
    flush = torch.empty(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    with sc.sparse_indice_map_build(coords) as m:
        k3 = [(ks, cin, cout, w, b) for ks, cin, cout, w, b, _, _ in layers]
        reps = max(args.conv_reps, len(k3))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for r in range(min(reps, 20)):  # warm
            ks, cin, cout, w, b = k3[r % len(k3)]
            conv(m, ks, x0_dev if not chained else outs[0], w, b, outs[-1])
        torch.cuda.synchronize()
        # the kernel's own start and completion (subm_timing_events binds a pair of events to the
        # next convolution kernel's dispatch), beside the whole call between two stream events
        kevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for ka, kb in kevs:  # (torch creates an event on its first record)
            ka.record(stream)
            kb.record(stream)
        torch.cuda.synchronize()
        per_layer = {i: [] for i in range(len(k3))}
        per_layer_call = {i: [] for i in range(len(k3))}
        for r in range(reps):
            i = r % len(k3)
            ks, cin, cout, w, b = k3[i]
            src = x0_dev if not chained else outs[0]
            evs[r][0].record(stream)
            if not per_offset:  # (the per-offset design is 27 + 1 launches per call: timed per call)
                sc.subm_timing_events(*kevs[r])
            conv(m, ks, src, w, b, outs[-1])
            evs[r][1].record(stream)
        torch.cuda.synchronize()
        for r in range(reps):
            call = evs[r][0].elapsed_time(evs[r][1])
            per_layer[r % len(k3)].append(call if per_offset else kevs[r][0].elapsed_time(kevs[r][1]))
            per_layer_call[r % len(k3)].append(call)
        pool_path = (not per_offset and layers[0][0] == 3
                     and sc.sparse_indice_map_plan_state(m) == sc.SUBM_PLAN_READY and layers[0][2] == 128)
        # Cold caches: 1 GiB written between launches (outside the events) evicts the layer's
        # working set from the 256 MB MALL and the L2s.
        cold = []
        for r in range(min(reps, 40)):
            flush.fill_(float(r))
            ks, cin, cout, w, b = k3[0]
            if per_offset:
                evs[r][0].record(stream)
            else:
                sc.subm_timing_events(*kevs[r])
            conv(m, ks, x0_dev if not chained else outs[0], w, b, outs[-1])
            if per_offset:
                evs[r][1].record(stream)
            cold.append(evs[r] if per_offset else kevs[r])
        torch.cuda.synchronize()
        cold_ms = [a.elapsed_time(b) for a, b in cold]
    del flush
    # Dominant kernel: the k = 3 layer (all layers of a workload share shape except 2a's k = 1).
    dom = 0
    conv_ms = float(np.mean(per_layer[dom]))
    call_ms = float(np.mean(per_layer_call[dom]))
    ks, cin, cout = layers[dom][0], layers[dom][1], layers[dom][2]
    s = ELEM[cfg.dtype]
    p_layer = pairs if ks == 3 else n
    flop_launch = 2.0 * p_layer * cin * cout
    bytes_launch = float(n * cin * s + n * cout * s + ks ** 3 * cin * cout * s + cout * s + (n * 27 * 4 if ks == 3 else 0))
    if per_offset and ks == 3:
        bytes_launch = per_offset_bytes(n, pairs, cin, cout, s)
    t_mfma = flop_launch / (PEAK_TFLOPS[cfg.dtype] * 1e12)
    t_hbm = bytes_launch / (PEAK_HBM_GBS * 1e9)
    conv_s = conv_ms / 1e3
    source = "conv_pool.hip" if pool_path else "conv.hip"
    kernel_hash = source_hash(os.path.join(CSRC, source))
    traffic = None if per_offset else load_traffic(key, source, kernel_hash)
    if t_mfma >= t_hbm:
        achieved = flop_launch / conv_s / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS[cfg.dtype], "unit": "TFLOP/s",
                    "frac": achieved / PEAK_TFLOPS[cfg.dtype], "traffic": traffic}
    else:
        achieved = bytes_launch / conv_s / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    # The kernel the library picks for this layer shape (16-bit storage: the warp-specialised
    # matrix-core kernel above 32 output channels, walking several tiles per workgroup for k = 3
    # with whole 16-byte output groups; the single-role one from 17 to 32).
    if per_offset and ks == 3:
        kernel = "offset_gemm_kernel (27 launches, one per offset) + round_out_kernel, per call"
    elif pool_path:
        # the neighbour-pool kernel (the call also packs its weights first: avg_call_ms)
        kernel = "pool_conv_kernel"
    elif (cfg.dtype in ("bf16", "f16") and cout > 32 and ks == 3 and cout % 8 == 0
          and os.environ.get("SUBMCONV_PERSISTENT", "1")[:1] != "0"):
        kernel = "subm_conv_ws_persistent_kernel"
    elif cfg.dtype in ("bf16", "f16") and cout > 32:
        kernel = "subm_conv_ws_kernel"
    elif cfg.dtype in ("bf16", "f16") and cout > 16:
        kernel = "subm_conv_mma_kernel"
    else:
        kernel = "subm_conv_generic_kernel"
    roofline.update({"kernel": kernel, "kernel_source": source, "avg_launch_ms": conv_ms, "avg_call_ms": call_ms,
                     "launches": len(per_layer[dom]),
                     "algorithmic_flop_per_launch": flop_launch, "algorithmic_bytes_per_launch": bytes_launch})
    peaks = None if args.no_peaks else measured_peaks(dev)
    if peaks is not None:
        measured = peaks["bf16_gemm_TFLOPs"] if roofline["bound"] == "mfma" else peaks["copy_GBps"]
        roofline.update({"peak_measured": measured, "frac_measured": roofline["achieved"] / measured,
                         "peak_measured_by": "torch.matmul bf16 8192^3" if roofline["bound"] == "mfma"
                         else "1 GiB device copy (read + write)"})
        if roofline["bound"] == "mfma":
            roofline.update({"mfma_loop_TFLOPs": peaks["mfma_loop_TFLOPs"],
                             "frac_of_mfma_loop": roofline["achieved"] / peaks["mfma_loop_TFLOPs"],
                             "mfma_loop_clock_GHz": peaks["mfma_loop_clock_GHz"]})
    pct = lambda v: {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
                     "p90": float(np.percentile(v, 90))}

    value = flops_per_step / step_s / 1e12
    result = {
        "metric": METRIC if not per_offset else "SubMConv3d per-offset design (gather -> GEMM -> scatter-add): effective TFLOP/s (1 GPU)",
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
        "config": {"workload": cfg.workload, "key": key, "op": args.op, "batch": cfg.batch, "grid": cfg.grid, "voxels": n,
                   "pairs": pairs, "cin": cfg.cin, "cout": cfg.cout,
                   "layers": [f"k{ks} {ci}->{co}" for ks, ci, co, *_ in layers], "chained": chained},
        "roofline": roofline,
        "breakdown": {"map_build_ms": build_s * 1e3,
                      "conv_ms_per_layer": {str(i): float(np.mean(v)) for i, v in per_layer.items()},
                      "conv_tflops_effective": flop_launch / conv_s / 1e12,
                      "voxels_per_s_step": n / step_s,
                      "voxels_per_s_conv": n / conv_s,
                      "step_ms_spread": pct(step_ms),
                      "conv_ms_spread": pct(per_layer[dom]),
                      "conv_ms_cold_mall": float(np.mean(cold_ms)),
                      "conv_ms_cold_mall_spread": pct(cold_ms),
                      "map_build_GBps": float(n * (16 + 108 + 4)) / build_s / 1e9,
                      "measured_peaks": peaks},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        ks, cin, cout = layers[dom][0], layers[dom][1], layers[dom][2]
        result["cpu_baseline"] = cpu_baseline(key, plan[dom][3], coords_np, nbr_rows, cin, cout, args.cpu_seconds)
    print(json.dumps(result), flush=True)


STRUCTURE_METRIC = {
    "subdivide": "subdivide + child features + derived child map: children per second (1 GPU)",
    "downsample": "2x downsample build + max pooling + cached upsample: fine voxels per second (1 GPU)",
    "groupnorm": "group normalisation (32 groups) + SiLU per batch item: voxels per second (1 GPU)",
    "conv-groupnorm": "SubMConv3d + group normalisation + SiLU in one call: voxels per second (1 GPU)",
}


def time_events(fn, reps, stream):
    """Average milliseconds of fn() from HIP events on `stream` around each of `reps` calls."""
    import torch
    for _ in range(min(reps, 10)):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def bench_structure(args):
    """Structure rows of the path on the config-5 coordinate sets (two 512^3 items).

    subdivide: input = the 256^3 level of the config-5 chain (three subdivisions of the r = 28
    shell, before the 25 % selection; 2 x 637,568 voxels), 64 bf16 channels.  One step =
    sparse_subdivide (coords, parent) + sparse_upsample_forward (children's features) +
    sparse_indice_map_subdivide (child map from the parent map) + frees.
    downsample: input = the config-5 set (2,550,313 voxels), 64 bf16 channels.  One step =
    sparse_downsample_build + max pooling + cache-paired upsample + free.
    """
    import numpy as np
    import torch

    import submanifold_sparse_convolution_amd as sc
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sc.load_library()
    stream = torch.cuda.current_stream(dev)
    ch, s = 64, 2
    if args.op == "subdivide":
        base = synth.coords_for("5_parent")
        workload = ("level 2 -> 3 of the config-5 chain: 2 x 256^3 subdivided r = 28 shells "
                    f"({len(base)} voxels) -> 2 x 512^3 ({8 * len(base)} children), 64 bf16 channels")
    elif args.op == "downsample":
        base = synth.coords_for("5")
        workload = ("config-5 coordinate set: 2 x 512^3 subdivided shells keeping 25 % "
                    f"({len(base)} voxels) -> 2x cells, 64 bf16 channels")
    elif args.op == "groupnorm":
        base = synth.coords_for("5")
        workload = ("config-5 coordinate set: 2 x 512^3 subdivided shells keeping 25 % "
                    f"({len(base)} voxels, 2 items), 64 bf16 channels, 32 groups, SiLU")
    else:
        base = synth.coords_for("5")
        workload = ("config-5 layer 0 (2 x 512^3 subdivided shells keeping 25 %, "
                    f"{len(base)} voxels, 2 items, 64->64 bf16, k3) + group norm (32 groups) + SiLU")
    n = len(base)
    coords = torch.from_numpy(base).to(dev)
    feats = synth.round_to(np.random.default_rng(77).standard_normal((n, ch)), "bf16").to(dev)

    if args.op == "subdivide":
        pm = sc.sparse_indice_map_build(coords)
        child_feats = torch.empty((8 * n, ch), dtype=torch.bfloat16, device=dev)

        def step():
            sub = sc.sparse_subdivide(coords)
            sc.sparse_upsample_forward(sub, feats, out=child_feats)
            cm = sc.sparse_indice_map_subdivide(pm, sub)
            cm.free()
            sub.free()

        items = 8 * n
        sub = sc.sparse_subdivide(coords)
        kern = {
            # a subdivide's children copy their parent row: each coarse row read once, no index
            "expand8_kernel": (lambda: sc.sparse_upsample_forward(sub, feats, out=child_feats),
                               float(n * ch * s + 8 * n * ch * s)),
        }
        cm_holder = []

        def child_map():
            cm_holder.append(sc.sparse_indice_map_subdivide(pm, sub))

        kern["child_map_kernel"] = (child_map, float(n * 108 + 8 * n * 112))
    elif args.op == "conv-groupnorm":
        cfg = synth.config("5")
        counts = np.bincount(base[:, 0])
        offsets = torch.tensor([0] + np.cumsum(counts).tolist(), dtype=torch.int64, device=dev)
        w = synth.weight_for(cfg.number, 0, 3, ch, ch, "bf16").to(dev)
        bias = synth.bias_for(cfg.number, 0, ch, "bf16").to(dev)
        gamma = synth.round_to(1.0 + 0.1 * np.random.default_rng(78).standard_normal(ch), "bf16").to(dev)
        beta = synth.round_to(0.1 * np.random.default_rng(79).standard_normal(ch), "bf16").to(dev)
        cmap = sc.sparse_indice_map_build(coords)
        fused_out = torch.empty_like(feats)
        conv_out = torch.empty_like(feats)
        normed = torch.empty_like(feats)

        def fused():
            sc.subm_conv3d_forward_group_norm_act(cmap, feats, w, bias, offsets, 32, gamma, beta, 1e-5,
                                                  sc.SUBM_ACT_SILU, out=fused_out)

        def epilogue_stats():
            os.environ["SUBMCONV_GN_EPILOGUE"] = "1"
            fused()
            os.environ["SUBMCONV_GN_EPILOGUE"] = "0"

        def split():
            sc.subm_conv3d_forward(cmap, feats, w, bias, out=conv_out)
            sc.sparse_group_norm_act(conv_out, offsets, 32, gamma, beta, 1e-5, sc.SUBM_ACT_SILU, out=normed)

        os.environ["SUBMCONV_GN_EPILOGUE"] = "0"
        step = fused
        items = n
        sub = None
        layer_bytes = float(n * ch * s + n * 108 + 27 * ch * ch * s + n * ch * s)  # conv alone, algorithmic
        kern = {"conv + group norm entry point (default: separate statistics pass)": (fused, layer_bytes + 3 * n * ch * s),
                "statistics in the conv epilogue (SUBMCONV_GN_EPILOGUE=1)": (epilogue_stats, layer_bytes + 2 * n * ch * s),
                "conv, then sparse_group_norm_act": (split, layer_bytes + 3 * n * ch * s)}
    elif args.op == "groupnorm":
        counts = np.bincount(base[:, 0])
        offsets = torch.tensor([0] + np.cumsum(counts).tolist(), dtype=torch.int64, device=dev)
        gamma = synth.round_to(1.0 + 0.1 * np.random.default_rng(78).standard_normal(ch), "bf16").to(dev)
        beta = synth.round_to(0.1 * np.random.default_rng(79).standard_normal(ch), "bf16").to(dev)
        normed = torch.empty_like(feats)

        def step():
            sc.sparse_group_norm_act(feats, offsets, 32, gamma, beta, 1e-5, sc.SUBM_ACT_SILU, out=normed)

        items = n
        sub = None
        kern = {"gn (partials + statistics + apply)": (step, float(2 * n * ch * s + n * ch * s))}
    else:
        coarse_out = None

        def step():
            nonlocal coarse_out
            d = sc.sparse_downsample_build(coords)
            coarse_out = sc.sparse_downsample_forward(d, feats, sc.SUBM_POOL_MAX, out=None)
            sc.sparse_upsample_forward(d, coarse_out)
            d.free()

        items = n
        sub = sc.sparse_downsample_build(coords)
        m_cells = sub.n_coarse
        pooled = torch.empty((m_cells, ch), dtype=torch.bfloat16, device=dev)
        up = torch.empty((n, ch), dtype=torch.bfloat16, device=dev)
        kern = {
            "pool_kernel": (lambda: sc.sparse_downsample_forward(sub, feats, sc.SUBM_POOL_MAX, out=pooled),
                            float(n * ch * s + n * 4 + (m_cells + 1) * 4 + m_cells * ch * s)),
            "expand_kernel": (lambda: sc.sparse_upsample_forward(sub, pooled, out=up),
                              float(m_cells * ch * s + n * 4 + n * ch * s)),
        }

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps

    per_kernel = {}
    for name, (fn, nbytes) in kern.items():
        ms = time_events(fn, 50, stream)
        per_kernel[name] = {"avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes,
                            "achieved_GBps": nbytes / (ms / 1e3) / 1e9}
    if args.op == "subdivide":
        for cm in cm_holder:
            cm.free()
        pm.free()
    if args.op == "conv-groupnorm":
        cmap.free()
    if sub is not None:
        sub.free()
    dom = max(per_kernel, key=lambda k: per_kernel[k]["avg_launch_ms"])
    if args.op == "conv-groupnorm":
        dom = "conv + group norm entry point (default: separate statistics pass)"
    achieved = per_kernel[dom]["achieved_GBps"]
    result = {
        "metric": STRUCTURE_METRIC[args.op],
        "value": items / step_s,
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32 coordinates, bf16 features",
        "data": "synthetic",
        "config": {"workload": workload, "op": args.op, "voxels_in": n, "channels": ch},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": dom,
                     "avg_launch_ms": per_kernel[dom]["avg_launch_ms"],
                     "algorithmic_bytes_per_launch": per_kernel[dom]["algorithmic_bytes_per_launch"]},
        "breakdown": per_kernel,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = structure_cpu_baseline(args.op, base, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def structure_cpu_baseline(op, base, budget_s):
    """The oracle's subdivide / downsample (pure Python) on a leading sample of the rows."""
    import numpy as np

    from oracle import structure_ref

    rows = 2000
    t0 = time.perf_counter()
    from oracle import norm_ref

    def run(k):
        if op == "subdivide":
            structure_ref.subdivide(base[:k])
        elif op == "downsample":
            structure_ref.downsample(base[:k])
        else:
            x = np.random.default_rng(1).standard_normal((k, 64))
            norm_ref.group_norm_act(x, [0, k], 32, None, None, 1e-5, "silu")

    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        run(rows)
        per_row = (time.perf_counter() - t0) / rows
        rows = int(min(len(base), max(rows, budget_s / max(per_row, 1e-9))))
        t0 = time.perf_counter()
        run(rows)
        elapsed = time.perf_counter() - t0
    out_rows = 8 * rows if op == "subdivide" else rows
    what = {"subdivide": "structure_ref.subdivide", "downsample": "structure_ref.downsample",
            "groupnorm": "norm_ref.group_norm_act (numpy, 64 channels, 32 groups, one item)",
            "conv-groupnorm": "norm_ref.group_norm_act only (numpy, 64 channels, 32 groups, one item)"}[op]
    return {"value": out_rows / elapsed, "unit": "voxels/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle {what} on the first {rows} of {len(base)} input rows; {elapsed:.2f} s"}


if __name__ == "__main__":
    main()

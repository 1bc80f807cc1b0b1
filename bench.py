#!/usr/bin/env python3
"""Benchmark: block-verify forward through a 40-layer NVFP4 MoE stack at K=2
(--rows 1/4/8/16: the K sweep on the same stack).

Workload: 40 independent MoE layers (hidden 2048, 256 routed experts, top-8
softmax-renormalised, intermediate 512, one shared expert of intermediate
512, NVFP4 expert weights, bf16 routers), K = 2 verify rows, each layer's
output RMS-normalised into the next layer's input.  All weights (18.2 GB)
and a pool of 8 input blocks are resident in HBM before timing; each step
is one captured-graph launch of the whole stack on the next input of the
pool, so the experts each step streams differ.

value = algorithmic bytes per step / measured time per step, where the
bytes are the router, each *unique* routed expert once, the shared expert
and the activations, summed over the 40 layers with the unique-expert
counts the dedup pass reports for that input.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "MoE verify step: weight GB/s and % HBM peak at K=2; µs per 40-layer stack"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def nvfp4_bytes(rows, cols):
    return rows * cols // 2 + rows * cols // 16 + 4


def gateup_bytes(shape, n_unique, K):
    """Algorithmic HBM bytes of one gate/up launch: gate + up of every unique
    expert and the shared expert, x read once, h written once."""
    H, I, Is, k = shape.hidden, shape.inter, shape.shared_inter, shape.top_k
    b = n_unique * 2 * nvfp4_bytes(I, H)
    if Is:
        b += 2 * nvfp4_bytes(Is, H)
    return b + K * H * 2 + (K * k * I + K * Is) * 4


KERNEL_SOURCES = ("speculative_block_verify_amd/csrc/moe_kernels.hip", "speculative_block_verify_amd/csrc/moe_device.h",
                  "speculative_block_verify_amd/csrc/moe_internal.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_gateup_moe_stack_k2_hbm_traffic.txt")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per k_gateup launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the plain-copy
    calibration), or None when the summary is missing or was taken on other
    kernel sources than the ones built now."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    """A plain copy of known size (torch's elementwise negation: one read and
    one write stream of mib MiB each), repeated 5 times; run under
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to calibrate those counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4, "launches": 5}))


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak


def prefill(args):
    """One MoE layer on 512 token rows (the prefill-sized grouped GEMM):
    hidden 2048, 256 experts, top-8, intermediate 512, shared 512.  The layer
    weights rotate over n_layers distinct sets and the inputs over a pool, so
    the 456 MB of each layer are streamed from HBM.  value = algorithmic bytes
    (router, every unique routed expert once, shared expert, activations) /
    time; mfma_util = the expert FLOPs (gate, up and down on the matrix cores,
    2 per multiply-add) / time / the dense fp16 peak."""
    import torch
    from speculative_block_verify_amd import api, inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape, T, NL, POOL, SEED = inputs.LAGUNA, 512, args.prefill_layers, 4, 4096
    layers = inputs.gen_stack(shape, NL, SEED, device=dev)
    xs = [inputs.gen_x(T, shape.hidden, SEED + 1 + i, device=dev) for i in range(POOL)]
    cfg = api.make_cfg(shape, T)
    ws = api.alloc_workspace(cfg, dev)
    wts = [api.make_weights(w) for w in layers]
    y = torch.empty(T, shape.hidden, dtype=torch.int16, device=dev)
    y32 = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    H, I, Is, E, k = shape.hidden, shape.inter, shape.shared_inter, shape.n_experts, shape.top_k
    nu = torch.empty(1, dtype=torch.int32, device=dev)
    step_bytes, step_flops = [], []
    for s in range(NL * POOL):
        api.moe_verify_layer(cfg, wts[s % NL], xs[s % POOL], y, ws, y32=y32, debug=api.make_debug(n_unique=nu))
        torch.cuda.synchronize()
        U = int(nu.item())
        step_bytes.append(api.moe_verify_weight_bytes(cfg, U, T))
        step_flops.append(2.0 * (T * k * 3 * I * H + T * 3 * Is * H))
    for s in range(args.warmup):
        api.moe_verify_layer(cfg, wts[s % NL], xs[s % POOL], y, ws, y32=y32)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for s in range(args.steps):
        api.moe_verify_layer(cfg, wts[s % NL], xs[s % POOL], y, ws, y32=y32)
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[-1])
    per = [ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps)]
    nb = sum(step_bytes[s % (NL * POOL)] for s in range(args.steps))
    nf = sum(step_flops[s % (NL * POOL)] for s in range(args.steps))
    gbs = nb / (total_ms / 1e3) / 1e9
    tflops = nf / (total_ms / 1e3) / 1e12
    log("prefill: %d layers of 512 rows in %.3f ms: %.1f GB/s, %.1f TFLOP/s" % (args.steps, total_ms, gbs, tflops))
    print(json.dumps({
        "metric": "prefill grouped GEMM: weight GB/s and % HBM peak, MFMA utilisation (512 rows)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 mfma / f32 acc", "data": "synthetic",
        "config": {"workload": "one NVFP4 MoE layer on 512 token rows (prefill grouped GEMM)", "rows": T,
                   "hidden": H, "experts": E, "top_k": k, "inter": I, "shared_inter": Is,
                   "layer_weight_sets": NL, "input_pool": POOL},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_layer": {"mean": round(total_ms / args.steps * 1e3, 2),
                         "median": round(statistics.median(per) * 1e3, 2)},
        "bytes_per_layer": round(sum(step_bytes) / len(step_bytes)),
        "expert_tflops": round(tflops, 2),
        "mfma_util": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
    }), flush=True)


def cpu_baseline(layers, xs, shape, K, budget_s, gpu_layer0=None):
    """The oracle (single-threaded C, fp64) chained through the same 40-layer
    stack, input after input of the pool, until budget_s seconds of CPU work;
    GB/s over the same algorithmic byte definition as the GPU figure.  With
    gpu_layer0 (the GPU's fp32 output of the first layer on the first input),
    also the parity of that layer against the oracle's."""
    import oracle as orc
    import numpy as np
    from speculative_block_verify_amd import api
    cfg = api.make_cfg(shape, K)
    host = [{k: (None if v is None else ({kk: vv.cpu() for kk, vv in v.items()} if isinstance(v, dict) else v.cpu()))
             for k, v in w.items()} for w in layers]
    t_total, n_bytes, n_layers, n_inputs = 0.0, 0, 0, 0
    parity = None
    while t_total < budget_s and n_inputs < len(xs):
        xo = xs[n_inputs].cpu().numpy().view(np.uint16)
        n_inputs += 1
        for wh in host:
            t0 = time.perf_counter()
            rec = orc.moe_layer(wh, xo, shape.top_k)
            if gpu_layer0 is not None and parity is None:
                ref = np.asarray(rec["y"], dtype=np.float64)
                d = np.asarray(gpu_layer0, dtype=np.float64) - ref
                parity = {"layer": 0, "input": 0, "max_abs_over_max_ref": float(np.abs(d).max() / np.abs(ref).max()),
                          "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref)), "bar": 2e-3}
            xo = orc.rmsnorm_bf16(rec["y"])
            t_total += time.perf_counter() - t0
            U = orc.dedup(rec["ids"], shape.n_experts)["n_unique"]
            n_bytes += api.moe_verify_weight_bytes(cfg, U, K)
            n_layers += 1
            if t_total >= budget_s:
                break
    return {"value": n_bytes / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d layer evaluations (the 40-layer stack chained over %d inputs of the pool), K=%d; "
                      "%.1f s single-threaded" % (n_layers, n_inputs, K, t_total)}, parity


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timing-steps", type=int, default=16, help="steps of the per-kernel timing pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--workload", choices=("stack", "prefill"), default="stack",
                    help="stack: the 40-layer K=2 verify stack (default); prefill: one 512-row layer")
    ap.add_argument("--prefill-layers", type=int, default=8, help="distinct weight sets the prefill mode rotates")
    ap.add_argument("--rows", type=int, default=2, choices=(1, 2, 4, 8, 16),
                    help="verify rows K of the stack workload: 2 (default) is the headline configuration with "
                         "independent rows; 1, 4, 8, 16 are the K sweep, whose rows 1..K/2 repeat row 0 plus small "
                         "noise so that experts repeat across rows")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU mode "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload == "prefill":
        prefill(args)
        return

    import torch
    from speculative_block_verify_amd import api, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape, L, K, POOL, SEED = inputs.LAGUNA, 40, args.rows, 8, 2024
    t0 = time.time()
    layers = inputs.gen_stack(shape, L, SEED, device=dev)
    if K == 2:
        xs = [inputs.gen_x(K, shape.hidden, SEED + 1 + i, device=dev) for i in range(POOL)]
    else:
        xs = [inputs.gen_x_correlated(K, shape.hidden, SEED + 1 + i, device=dev) for i in range(POOL)]
    torch.cuda.synchronize()
    log("bench: generated %d layers (%.2f GB) in %.1f s" % (
        L, sum(sum(t.numel() for t in (w[m].values() if isinstance(w[m], dict) else [w[m]]))
               for w in layers for m in w if w[m] is not None) / 1e9, time.time() - t0))

    cfg = api.make_cfg(shape, K)
    ws = api.alloc_workspace(cfg, dev)
    wts = [api.make_weights(w) for w in layers]
    y = torch.empty(K, shape.hidden, dtype=torch.int16, device=dev)
    y32 = torch.empty(K, shape.hidden, dtype=torch.float32, device=dev)

    # unique-expert counts per (input, layer) from the dedup pass
    nu = torch.empty(L, dtype=torch.int32, device=dev)
    y32_layers = torch.empty(L, K, shape.hidden, dtype=torch.float32, device=dev)
    step_bytes, gu_bytes, uniques = [], [], []
    gpu_layer0 = None
    for i in range(POOL):
        dbg = api.make_debug(n_unique=nu, y32=y32_layers) if i == 0 else api.make_debug(n_unique=nu)
        api.moe_verify_stack(cfg, wts, xs[i], y, ws, y32=y32, debug=dbg)
        if i == 0:
            torch.cuda.synchronize()
            gpu_layer0 = y32_layers[0].cpu().numpy()
        torch.cuda.synchronize()
        U = nu.cpu().tolist()
        uniques.append(U)
        step_bytes.append(sum(api.moe_verify_weight_bytes(cfg, u, K) for u in U))
        gu_bytes.append([gateup_bytes(shape, u, K) for u in U])
    log("bench: unique experts per layer (mean) %.2f; bytes per step %.4f GB" % (
        sum(map(sum, uniques)) / (POOL * L), sum(step_bytes) / POOL / 1e9))

    graphs = [api.StackGraph(cfg, wts, xs[i], y, ws, y32=y32) for i in range(POOL)]
    for s in range(args.warmup):
        graphs[s % POOL].launch()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    evs[0].record(stream)
    for s in range(args.steps):
        graphs[s % POOL].launch()
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    per_step_ms = [evs[s].elapsed_time(evs[s + 1]) for s in range(args.steps)]
    total_ms = evs[0].elapsed_time(evs[-1])
    total_bytes = sum(step_bytes[s % POOL] for s in range(args.steps))
    gbs = total_bytes / (total_ms / 1e3) / 1e9
    log("bench: %d steps in %.3f ms (wall %.3f ms): %.1f GB/s, %.1f us/stack" % (
        args.steps, total_ms, wall * 1e3, gbs, total_ms / args.steps * 1e3))

    # per-kernel timing pass: same inputs, kernels stamped by their own
    # dispatch (verify-width kernels; from 8 rows the stack runs the grouped
    # kernels, which this pass does not cover)
    kt = {"route": [], "gateup": [], "down": []}
    gu_rates = []
    avg, achieved, gu_avg_bytes = None, None, None
    try:
        for s in range(args.timing_steps):
            ms = api.moe_verify_stack_timed(cfg, wts, xs[s % POOL], y, ws, y32=y32)
            for l, (a, b, c) in enumerate(ms):
                kt["route"].append(a); kt["gateup"].append(b); kt["down"].append(c)
                gu_rates.append(gu_bytes[s % POOL][l])
    except api.MoEError as err:
        if err.code != api.MOE_ERR_UNSUPPORTED:
            raise
        log("bench: no per-kernel timing (%s)" % err)
    if gu_rates:
        avg = {k: sum(v) / len(v) for k, v in kt.items()}
        gu_avg_bytes = sum(gu_rates) / len(gu_rates)
        achieved = gu_avg_bytes / (avg["gateup"] / 1e3) / 1e9
        log("bench: kernel averages (us): route %.2f gateup %.2f down %.2f; gateup %.1f GB/s" % (
            avg["route"] * 1e3, avg["gateup"] * 1e3, avg["down"] * 1e3, achieved))

    for g in graphs:
        g.close()

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "40-layer NVFP4 MoE verify stack, K=%d rows%s" % (
                       K, "" if K == 2 else " (K sweep: rows 1..K/2 repeat row 0 plus noise)"), "hidden": shape.hidden,
                   "experts": shape.n_experts, "top_k": shape.top_k, "inter": shape.inter,
                   "shared_inter": shape.shared_inter, "layers": L, "rows": K, "input_pool": POOL,
                   "weights": "NVFP4 (E2M1 + E4M3/16 + fp32 tensor scale), bf16 router/activations"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_stack": {"mean": round(total_ms / args.steps * 1e3, 2),
                         "median": round(statistics.median(per_step_ms) * 1e3, 2),
                         "min": round(min(per_step_ms) * 1e3, 2), "max": round(max(per_step_ms) * 1e3, 2)},
        "bytes_per_step": round(sum(step_bytes) / POOL),
        "unique_experts_per_layer": round(sum(map(sum, uniques)) / (POOL * L), 3),
        "kernel_us": None if avg is None else {k: round(v * 1e3, 3) for k, v in avg.items()},
        "roofline": None if avg is None else {
            "bound": "hbm", "kernel": "k_gateup", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if K == 2 else None, "bytes_per_launch": round(gu_avg_bytes)},
        "wall_s": round(wall, 4),
    }
    result["seed"] = SEED
    result["device"] = torch.cuda.get_device_name(dev)
    result["rocm"] = torch.version.hip
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host (%.0f s budget)" % args.cpu_seconds)
        result["cpu_baseline"], result["parity"] = cpu_baseline(layers, xs, shape, K, args.cpu_seconds, gpu_layer0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

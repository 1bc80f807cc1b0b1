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
    """Algorithmic HBM bytes of one router + gate/up launch: the bf16 router
    rows, gate + up of every unique expert and of the shared expert, x read
    once, h written once."""
    H, I, Is, k = shape.hidden, shape.inter, shape.shared_inter, shape.top_k
    b = 2 * shape.n_experts * H + n_unique * 2 * nvfp4_bytes(I, H)
    if Is:
        b += 2 * nvfp4_bytes(Is, H)
    return b + K * H * 2 + (K * k * I + K * Is) * 4


KERNEL_SOURCES = ("speculative_block_verify_amd/csrc/moe_kernels.hip", "speculative_block_verify_amd/csrc/moe_device.h",
                  "speculative_block_verify_amd/csrc/moe_internal.h", "speculative_block_verify_amd/csrc/moe_abi.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_route_gateup_moe_stack_k2_hbm_traffic.txt")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per k_route_gateup launch from the committed rocprofv3 counter
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
DTYPE = "nvfp4 weights, bf16 x, f16-MFMA/f32-acc gate-up, f32 down"


def host_info():
    """The host the oracle runs on: logical cores, CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cores": os.cpu_count(), "cpu_model": model,
            "affinity_cores": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def weight_hashes(layers):
    """xxh3-64 of each layer's packed weight bytes (router, every NVFP4
    matrix's codes, scales and tensor scales, norm weight), in a fixed
    order: the record names the exact inputs it measured."""
    import xxhash
    out = []
    for w in layers:
        h = xxhash.xxh3_64()
        for name in ("router_w", "router_bias", "gate", "up", "down", "sh_gate", "sh_up", "sh_down", "norm_w"):
            v = w.get(name)
            if v is None:
                continue
            for t in ([v[k] for k in ("q", "s", "ts")] if isinstance(v, dict) else [v]):
                h.update(t.contiguous().cpu().numpy().tobytes())
        out.append(h.hexdigest())
    return out


def stream_read_ceiling(dev, gib=4, reps=5):
    """A measured streaming-read rate on this GPU: the library's plain read
    kernel (moe_verify_stream_read) over a gib-GiB buffer, best of reps."""
    import torch
    from speculative_block_verify_amd import api
    buf = torch.empty(gib * (1 << 30), dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    api.moe_verify_stream_read(buf, sink)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        api.moe_verify_stream_read(buf, sink)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del buf
    torch.cuda.empty_cache()
    return round(gib * (1 << 30) / (best / 1e3) / 1e9, 1)


def near_tie_rows(logits, k, rtol=1e-5):
    """Rows whose k-th and (k+1)-th largest router logits differ by less than
    rtol * max|logit| (selection there may legitimately go either way)."""
    import numpy as np
    l = np.sort(np.asarray(logits, np.float64), axis=-1)[..., ::-1]
    gap = l[..., k - 1] - l[..., k]
    return int((gap < rtol * np.abs(l).max(axis=-1)).sum())


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
    shape, T, NL, POOL, SEED = inputs.LAGUNA, 512, args.prefill_layers, 8, 4096
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
        "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
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


def prefill_stack(args):
    """The 512-row seed prefill through the target's whole FFN stack: the
    dense first layer (bf16 SwiGLU, intermediate 8192) and 39 MoE layers on
    the grouped kernels, one moe_prefill_stack call per step over a pool of
    inputs (every layer's weights are streamed once per step: 17.9 GB, far
    beyond the memory-side cache).  value = algorithmic bytes (the dense
    layer's weights, each MoE layer's router, unique routed experts and
    shared expert, activations) / time per step; tokens/s = 512 / time."""
    import numpy as np
    import torch
    import oracle as orc
    from speculative_block_verify_amd import api, inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape, T, NL, POOL, SEED, DI = inputs.LAGUNA, 512, 39, 4, 5120, inputs.DENSE_INTER
    H, I, Is, E, k = shape.hidden, shape.inter, shape.shared_inter, shape.n_experts, shape.top_k
    dense = inputs.gen_dense(H, DI, SEED, device=dev)
    layers = inputs.gen_stack(shape, NL, SEED + 1, device=dev)
    xs = [inputs.gen_x(T, H, SEED + 10 + i, device=dev) for i in range(POOL)]
    cfg = api.make_cfg(shape, T)
    wts = [api.make_weights(w) for w in layers]
    ws = torch.empty(api.moe_prefill_workspace_bytes(cfg, DI), dtype=torch.uint8, device=dev)
    y = torch.empty(T, H, dtype=torch.int16, device=dev)
    y32 = torch.empty(T, H, dtype=torch.float32, device=dev)
    nu = torch.empty(NL, dtype=torch.int32, device=dev)
    dense_bytes = 3 * H * DI * 2 + 2 * T * H * 2
    step_bytes = []
    for i in range(POOL):
        api.moe_prefill_stack(cfg, dense, wts, xs[i], y, ws, y32=y32, debug=api.make_debug(n_unique=nu))
        torch.cuda.synchronize()
        step_bytes.append(dense_bytes + sum(api.moe_verify_weight_bytes(cfg, int(u), T) for u in nu.cpu().tolist()))
    flops = 2.0 * (3 * T * H * DI + NL * (T * k * 3 * I * H + T * 3 * Is * H + T * E * H))
    for s in range(args.warmup):
        api.moe_prefill_stack(cfg, dense, wts, xs[s % POOL], y, ws, y32=y32)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for s in range(args.steps):
        api.moe_prefill_stack(cfg, dense, wts, xs[s % POOL], y, ws, y32=y32)
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[-1])
    per = [ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps)]
    med = statistics.median(per)
    nb = sum(step_bytes[s % POOL] for s in range(args.steps))
    gbs = nb / (total_ms / 1e3) / 1e9
    tok_s = T * args.steps / (total_ms / 1e3)
    # the dense layer alone (same inputs, its own calls)
    dws = torch.empty(api.moe_dense_workspace_bytes(H, DI, T), dtype=torch.uint8, device=dev)
    xn = torch.empty(T, H, dtype=torch.int16, device=dev)
    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
    for s in range(3):
        api.moe_dense_mlp(xs[s % POOL], dense, y, y32, dws, x_next=xn)
    dev_ev[0].record(stream)
    for s in range(20):
        api.moe_dense_mlp(xs[s % POOL], dense, y, y32, dws, x_next=xn)
        dev_ev[s + 1].record(stream)
    torch.cuda.synchronize()
    dense_us = statistics.median(dev_ev[s].elapsed_time(dev_ev[s + 1]) for s in range(20)) * 1e3
    dense_tflops = 2.0 * 3 * T * H * DI / (dense_us / 1e6) / 1e12
    log("prefill-stack: %d steps, %.1f us per stack (median %.1f), %.1f GB/s, %.0f tokens/s; dense layer %.1f us "
        "(%.1f TFLOP/s)" % (args.steps, total_ms / args.steps * 1e3, med * 1e3, gbs, tok_s, dense_us, dense_tflops))
    result = {
        "metric": "prefill FFN stack (dense layer + 39 MoE layers, 512 rows): weight GB/s and % HBM peak, tokens/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE + "; dense layer bf16-MFMA/f32-acc", "data": "synthetic",
        "config": {"workload": "512-row prefill through the dense first layer (bf16 SwiGLU, intermediate 8192) and "
                               "39 NVFP4 MoE layers (grouped kernels)", "rows": T, "hidden": H,
                   "dense_inter": DI, "moe_layers": NL, "experts": E, "top_k": k, "inter": I, "shared_inter": Is,
                   "input_pool": POOL},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tok_s, 1),
        "us_per_stack": {"mean": round(total_ms / args.steps * 1e3, 2), "median": round(med * 1e3, 2),
                         "min": round(min(per) * 1e3, 2), "max": round(max(per) * 1e3, 2)},
        "stall_steps_over_4x_median": sum(1 for t in per if t > 4 * med),
        "bytes_per_step": round(sum(step_bytes) / len(step_bytes)),
        "tflops": round(flops / (med / 1e3) / 1e12, 2),
        "dense_layer_us": round(dense_us, 2), "dense_layer_tflops": round(dense_tflops, 2),
        "seed": SEED, "device": torch.cuda.get_device_name(dev), "rocm": torch.version.hip,
    }
    if not args.no_cpu_baseline:
        # the oracle on one row through the whole stack (rows are independent)
        x0 = xs[0][:1].cpu().numpy().view(np.uint16)
        dh = {kk: (None if v is None else v.cpu()) for kk, v in dense.items()}
        lh = [{kk: (None if v is None else ({q: t.cpu() for q, t in v.items()} if isinstance(v, dict) else v.cpu()))
               for kk, v in w.items()} for w in layers]
        old_aff = os.sched_getaffinity(0)
        core = max(old_aff)
        os.sched_setaffinity(0, {core})
        times = []
        try:
            for _ in range(3):
                t1 = time.perf_counter()
                orc.dense_moe_stack(dh, lh, x0, k)
                times.append(time.perf_counter() - t1)
        finally:
            os.sched_setaffinity(0, old_aff)
        med_s = statistics.median(times)
        result["cpu_baseline"] = {
            "value": round(1.0 / med_s, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "one row through the dense layer and the 39 MoE layers (rows are independent), 3 runs, median; "
                      "single-threaded C (fp64), pinned to core %d" % core,
            "us_per_token": round(med_s * 1e6, 1), "runs_s": [round(t, 3) for t in times], "pinned_core": core,
            "host_cores": os.cpu_count(), "gpu_speedup": round(tok_s * med_s, 1)}
    print(json.dumps(result), flush=True)


def lmhead(args):
    """The verify step's head: lm_head over K verify rows (vocabulary 100352,
    hidden 2048, bf16: 0.41 GB), argmax per row and greedy acceptance, one
    call per step.  Two copies of the matrix rotate (822 MB against a 256 MB
    memory-side cache) with a pool of inputs.  value = algorithmic bytes (the
    matrix once, the rows in) / time per step."""
    import numpy as np
    import torch
    import oracle as orc
    from speculative_block_verify_amd import api, inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, V, H, POOL, SEED = args.rows, inputs.VOCAB, 2048, 4, 31
    ws_ = [inputs.gen_lm_head(V, H, SEED + c, device=dev) for c in range(2)]
    xs = [inputs.gen_x(K, H, SEED + 10 + i, device=dev) for i in range(POOL)]
    drafts = [inputs.gen_tokens(max(K - 1, 1), V, SEED + 20 + i, device=dev) for i in range(POOL)]
    out = api.alloc_greedy_out(K, dev)
    wsp = torch.empty(api.moe_verify_lm_head_workspace_bytes(V, K), dtype=torch.uint8, device=dev)

    def step(s):
        api.moe_verify_lm_head_greedy(xs[s % POOL], ws_[s % 2], out, wsp, draft=drafts[s % POOL] if K > 1 else None)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for s in range(args.steps):
        step(s)
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[-1])
    per = [ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps)]
    nbytes = orc.lm_head_bytes(V, H, K)
    gbs = nbytes / (total_ms / args.steps / 1e3) / 1e9
    med = statistics.median(per)
    log("lmhead: %d steps, %.2f us per step (median %.2f), %.1f GB/s" % (args.steps, total_ms / args.steps * 1e3,
                                                                          med * 1e3, gbs))
    result = {
        "metric": "verify-row lm_head + greedy acceptance: weight GB/s and % HBM peak",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 weights and rows, bf16-MFMA/f32-acc", "data": "synthetic",
        "config": {"workload": "verify-row lm_head (vocabulary 100352 x hidden 2048, bf16) + argmax + greedy "
                               "acceptance, K=%d rows" % K, "rows": K, "vocab": V, "hidden": H,
                   "weight_copies": 2, "input_pool": POOL},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_step": {"mean": round(total_ms / args.steps * 1e3, 2), "median": round(med * 1e3, 2),
                        "min": round(min(per) * 1e3, 2), "max": round(max(per) * 1e3, 2)},
        "stall_steps_over_4x_median": sum(1 for t in per if t > 4 * med),
        "bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": "k_lm_head + k_greedy_finalize (whole step)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": nbytes},
        "seed": SEED, "device": torch.cuda.get_device_name(dev), "rocm": torch.version.hip,
    }
    if not args.no_extras:
        result["stream_read_ceiling_gbs"] = stream_read_ceiling(dev)
    if not args.no_cpu_baseline:
        xo = xs[0].cpu().numpy().view(np.uint16)
        wo = ws_[0].cpu().numpy().view(np.uint16)
        do = drafts[0].cpu().numpy()[: K - 1]
        old_aff = os.sched_getaffinity(0)
        core = max(old_aff)
        os.sched_setaffinity(0, {core})
        times = []
        try:
            for r in range(3):
                t0 = time.perf_counter()
                lo = orc.lm_head(xo, wo)
                orc.greedy_accept(lo, do)
                times.append(time.perf_counter() - t0)
                log("lmhead: oracle run %d: %.2f s" % (r + 1, times[-1]))
        finally:
            os.sched_setaffinity(0, old_aff)
        med_s = statistics.median(times)
        cb = {"value": round(nbytes / med_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
              "sample": "one verify step (lm_head over %d rows + greedy acceptance), 3 runs, median; single-threaded "
                        "C (fp64), pinned to core %d" % (K, core),
              "us_per_step": round(med_s * 1e6, 1), "runs_s": [round(t, 3) for t in times], "pinned_core": core,
              "gpu_speedup": round(med_s * 1e6 / (total_ms / args.steps * 1e3), 1)}
        cb.update(host_info())
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


def kv_ring(args):
    """The verify step's sliding-window KV maintenance on the target's shape
    (30 sliding layers, 8 KV heads of head_dim 128, window 512, K=2 rows):
    per step, as a forward makes them, one in-place write of the block's rows
    per layer and one device-side commit of 1 + n_accepted rows.  value =
    microseconds per step; the roofline is the ring write's algorithmic bytes
    (new rows read once, written once) over its time; the concatenating
    cache that rebuilds every window per step is set beside it by its HBM
    lower bound."""
    import torch
    from oracle import kv_oracle
    from speculative_block_verify_amd import api
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, NKV, D, W, K, POOL, SEED = 30, 8, 128, 512, args.rows, 8, 41
    ring = api.KvRing(L, NKV, D, W, K, dev)
    ring.reset(0)
    g = torch.Generator(device=dev).manual_seed(SEED)
    kn = [torch.randint(-32768, 32767, (L, K, NKV, D), generator=g, device=dev, dtype=torch.int16)
          for _ in range(POOL)]
    vn = [torch.randint(-32768, 32767, (L, K, NKV, D), generator=g, device=dev, dtype=torch.int16)
          for _ in range(POOL)]
    nacc = torch.randint(0, K, (POOL, 1), generator=g, device=dev, dtype=torch.int32)

    def step(s):  # the forward's pattern: each layer written before its attention
        for l in range(L):
            ring.write_layer(l, kn[s % POOL][l], vn[s % POOL][l])
        ring.commit(nacc[s % POOL], K)

    def step_batched(s):  # all layers' rows in one launch
        ring.write(kn[s % POOL], vn[s % POOL])
        ring.commit(nacc[s % POOL], K)

    # Steps are captured in HIP graphs (GSTEPS per graph) so the timed region
    # holds the kernels, not the host's launch path: the eager rate is
    # reported beside it.
    GSTEPS = 32

    def capture(fn):
        g_ = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g_, stream=side):
                for s in range(GSTEPS):
                    fn(s)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g_

    stream = torch.cuda.current_stream()

    def timed(fn, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for s in range(n):
            fn(s)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n * 1e3  # us per call

    for s in range(args.warmup):
        step(s)
    us_eager = timed(step, max(1, args.steps // 8))
    g_step = capture(step)
    g_batched = capture(step_batched)
    g_write = capture(lambda s: ring.write_layer(s % L, kn[s % POOL][s % L], vn[s % POOL][s % L]))
    reps = max(1, args.steps // GSTEPS)
    for _ in range(2):
        g_step.replay()
        g_batched.replay()
        g_write.replay()
    us_step = timed(lambda s: g_step.replay(), reps) / GSTEPS
    us_batched = timed(lambda s: g_batched.replay(), reps) / GSTEPS
    us_write = timed(lambda s: g_write.replay(), reps) / GSTEPS
    nbytes = kv_oracle.copy_bytes_in_place(L, NKV, D, K)
    layer_bytes = kv_oracle.copy_bytes_in_place(1, NKV, D, K)
    concat = kv_oracle.copy_bytes_concat(L, NKV, D, W, K)
    gbs = layer_bytes / (us_write * 1e-6) / 1e9
    log("kv: %.2f us per step of %d layer writes + commit in graphs (%.2f us launched one by one from Python; "
        "%.2f us with every layer in one write), %.3f us per layer write (%.1f GB/s); concatenation would move "
        "%.3f GB (>= %.1f us at 8 TB/s)" % (us_step, L, us_eager, us_batched, us_write, gbs, concat / 1e9,
                                           concat / HBM_PEAK_GBS / 1e3))
    result = {
        "metric": "verify-step sliding-window KV maintenance: microseconds per step",
        "value": round(us_step, 3), "unit": "us/step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 rows (copied bit for bit)", "data": "synthetic",
        "config": {"workload": "sliding-window KV ring, 30 layers x 8 KV heads x head_dim 128, window 512, "
                               "K=%d rows per step: an in-place write per layer + device commit" % K,
                   "rows": K, "layers": L, "kv_heads": NKV, "head_dim": D, "window": W,
                   "capacity": ring.shape[2]},
        "us_per_layer_write": round(us_write, 3),
        "us_per_step_one_write_for_all_layers": round(us_batched, 3),
        "us_per_step_eager_launches": round(us_eager, 3),
        "graph_steps": GSTEPS,
        "bytes_per_step": nbytes,
        "concat_bytes_per_step": concat,
        "concat_hbm_lower_bound_us": round(concat / HBM_PEAK_GBS / 1e3, 2),
        "roofline": {"bound": "hbm", "kernel": "k_kv_write, one layer (graph of %d writes; time per write "
                               "includes the gaps between them)" % GSTEPS, "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": layer_bytes},
        "seed": SEED, "device": torch.cuda.get_device_name(dev), "rocm": torch.version.hip,
    }
    if not args.no_cpu_baseline:
        import numpy as np
        rng = np.random.default_rng(SEED)
        hist = kv_oracle.KVHistory(L, NKV, D, W)
        ko = rng.integers(0, 1 << 16, (L, K, NKV, D), dtype=np.uint16)
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 2.0:
            hist.write(ko, ko)
            for l in range(L):  # what the block's last row sees in every layer
                hist.window(l, hist.length - 1)
            hist.commit(n % K)
            n += 1
        sec = (time.perf_counter() - t0) / n
        result["cpu_baseline"] = {"value": round(sec * 1e6, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
                                  "sample": "%d steps of the history model (write, every layer's window, commit), "
                                            "about 2 s" % n}
    print(json.dumps(result), flush=True)


def layer_ksweep(args):
    """Dedup at real expert reuse: single verify layers (the 40 weight sets of
    the stack) on correlated rows -- rows 1..K/2 are row 0 plus noise that
    moves the router logits by ~N(0, 0.01^2), so those rows pick nearly the
    same experts.  Each layer is its own graph, timed launch by launch with
    events.  Per K: unique experts U against the K*k slots a gather without
    dedup streams, and the bytes each reads."""
    import numpy as np
    import torch
    from speculative_block_verify_amd import api, inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape, L, SEED = inputs.LAGUNA, 40, 2024
    layers = inputs.gen_stack(shape, L, SEED, device=dev)
    sweep = []
    for K in (1, 2, 4, 8, 16):
        cfg = api.make_cfg(shape, K)
        ws = api.alloc_workspace(cfg, dev)
        wts = [api.make_weights(w, cfg) for w in layers]
        xs = [inputs.gen_x_correlated(K, shape.hidden, SEED + 100 * K + l, device=dev) for l in range(L)]
        y = torch.empty(K, shape.hidden, dtype=torch.int16, device=dev)
        y32 = torch.empty(K, shape.hidden, dtype=torch.float32, device=dev)
        nu = torch.empty(1, dtype=torch.int32, device=dev)
        U = []
        for l in range(L):
            api.moe_verify_layer(cfg, wts[l], xs[l], y, ws, y32=y32, debug=api.make_debug(n_unique=nu))
            torch.cuda.synchronize()
            U.append(int(nu.item()))
        graphs = [api.StackGraph(cfg, [wts[l]], xs[l], y, ws, y32=y32) for l in range(L)]
        for g in graphs:
            g.launch()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        evs = []
        for r in range(args.layer_reps):
            for g in graphs:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.launch()
                b.record(stream)
                evs.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        for g in graphs:
            g.close()
        med_us = statistics.median(ms) * 1e3
        b_dedup = statistics.mean(api.moe_verify_weight_bytes(cfg, u, K) for u in U)
        b_slots = api.moe_verify_weight_bytes(cfg, K * shape.top_k, K)
        ent = {"rows": K, "regime": "grouped" if K >= 8 else "verify width",
               "us_per_layer": {"median": round(med_us, 2), "min": round(ms[0] * 1e3, 2)},
               "unique_experts_mean": round(float(np.mean(U)), 2), "unique_experts_min": int(min(U)),
               "unique_experts_max": int(max(U)), "no_dedup_slots": K * shape.top_k,
               "bytes_per_layer": round(b_dedup), "bytes_per_layer_no_dedup": b_slots,
               "dedup_byte_saving": round(1.0 - b_dedup / b_slots, 4),
               "gbs": round(b_dedup / (med_us / 1e6) / 1e9, 1)}
        log("layer-ksweep: K=%d U=%.2f of %d slots (saves %.1f%% of bytes), %.2f us per layer, %.1f GB/s" % (
            K, ent["unique_experts_mean"], K * shape.top_k, 100 * ent["dedup_byte_saving"], med_us, ent["gbs"]))
        sweep.append(ent)
        del ws
    k2 = [e for e in sweep if e["rows"] == 2][0]
    print(json.dumps({
        "metric": "single MoE verify layer on correlated rows: weight GB/s and unique experts vs slots, K sweep",
        "value": k2["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.layer_reps * L, "warmup": 1,
        "ms_per_step": round(k2["us_per_layer"]["median"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": "one NVFP4 MoE verify layer per launch over the 40 weight sets of the stack, "
                               "rows 1..K/2 = row 0 + noise (router logits ~N(0, 0.01^2) apart)",
                   "hidden": shape.hidden, "experts": shape.n_experts, "top_k": shape.top_k,
                   "inter": shape.inter, "shared_inter": shape.shared_inter, "weight_sets": L},
        "pct_hbm_peak": round(100 * k2["gbs"] / HBM_PEAK_GBS, 2),
        "sweep": sweep, "seed": SEED, "device": torch.cuda.get_device_name(dev), "rocm": torch.version.hip,
    }), flush=True)


def cpu_baseline(layers, x0, shape, K, runs=3, gpu_layer0=None, gpu_us_per_stack=None, gpu_gbs=None,
                 score_fn=0, rs=1.0, residual=None):
    """The oracle (single-threaded C, fp64), pinned to one host core, chained
    through the whole 40-layer stack on the pool's first input, `runs` times;
    the median run gives µs per stack and GB/s over the same algorithmic
    byte definition as the GPU figure.  With gpu_layer0 (the GPU's fp32
    output of the first layer on that input), also the parity of that layer
    against the oracle's."""
    import oracle as orc
    import numpy as np
    from speculative_block_verify_amd import api
    cfg = api.make_cfg(shape, K)
    host = [{k: (None if v is None else ({kk: vv.cpu() for kk, vv in v.items()} if isinstance(v, dict) else v.cpu()))
             for k, v in w.items()} for w in layers]
    info = host_info()
    core = None
    old_aff = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if old_aff:
        core = max(old_aff)
        os.sched_setaffinity(0, {core})
    times, parity, n_bytes = [], None, 0
    try:
        for run in range(runs):
            xo = x0.cpu().numpy().view(np.uint16)
            ro = None if residual is None else residual.cpu().numpy().view(np.uint16)
            t_run, b_run = 0.0, 0
            for l, wh in enumerate(host):
                t0 = time.perf_counter()
                rec = orc.moe_layer(wh, xo, shape.top_k, score_fn, 1, rs, residual=ro)
                xo = orc.rmsnorm_bf16(rec["y"], 1e-6, wh.get("norm_w"))
                if ro is not None:
                    ro = orc.bf16_round(rec["y"])
                t_run += time.perf_counter() - t0
                if gpu_layer0 is not None and parity is None:
                    ref = np.asarray(rec["y"], dtype=np.float64)
                    d = np.asarray(gpu_layer0, dtype=np.float64) - ref
                    parity = {"layer": 0, "input": 0,
                              "max_abs_over_max_ref": float(np.abs(d).max() / np.abs(ref).max()),
                              "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref)), "bar": 2e-3}
                b_run += api.moe_verify_weight_bytes(cfg, orc.dedup(rec["ids"], shape.n_experts)["n_unique"], K)
            times.append(t_run)
            n_bytes = b_run
            log("bench: oracle run %d: %.2f s for the %d-layer stack" % (run + 1, t_run, len(host)))
    finally:
        if old_aff:
            os.sched_setaffinity(0, old_aff)
    med = statistics.median(times)
    us_stack = med * 1e6
    out = {"value": round(n_bytes / med / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "the %d-layer stack chained on the first input of the pool, K=%d, %d runs, median; "
                     "single-threaded C (fp64), pinned to core %s" % (len(host), K, runs, core),
           "us_per_stack": round(us_stack, 1), "us_per_layer": round(us_stack / len(host), 1),
           "runs_s": [round(t, 3) for t in times], "pinned_core": core}
    out.update(info)
    if gpu_us_per_stack:
        out["gpu_speedup"] = round(us_stack / gpu_us_per_stack, 1)
    return out, parity


def single_layer_timing(cfg, wts, xs, y, ws, y32, reps=3):
    """One verify layer (the 2-row configuration) on its own: a graph per
    weight set (each a one-layer stack), launched in rotation over the 40
    sets and the input pool, every launch bracketed by events on the stream.
    Returns the median and min µs per layer."""
    import torch
    from speculative_block_verify_amd import api
    graphs = [[api.StackGraph(cfg, [w], x, y, ws, y32=y32) for x in xs[:2]] for w in wts]
    stream = torch.cuda.current_stream()
    for g in graphs:
        g[0].launch()
    torch.cuda.synchronize()
    times = []
    for r in range(reps):
        for i, g in enumerate(graphs):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g[(i + r) % 2].launch()
            b.record(stream)
            times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)
    for g in graphs:
        for h in g:
            h.close()
    return {"median": round(statistics.median(ms) * 1e3, 2), "min": round(ms[0] * 1e3, 2), "launches": len(ms)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the single-layer timing, the streaming-read ceiling and the weight hashes")
    ap.add_argument("--timing-steps", type=int, default=16, help="steps of the per-kernel timing pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--workload", choices=("stack", "prefill", "prefill-stack", "lmhead", "layer-ksweep", "kv"),
                    default="stack",
                    help="stack: the 40-layer K=2 verify stack (default); prefill: one 512-row MoE layer; "
                         "prefill-stack: 512 rows through the dense first layer and 39 MoE layers; lmhead: the "
                         "verify rows' lm_head + greedy acceptance; layer-ksweep: one layer per launch on correlated "
                         "rows, K = 1..16; kv: the sliding-window KV ring's write + commit per "
                         "verify step")
    ap.add_argument("--prefill-layers", type=int, default=8, help="distinct weight sets the prefill mode rotates")
    ap.add_argument("--layer-reps", type=int, default=5, help="launches of each layer graph in the layer K sweep")
    ap.add_argument("--one-launch", action="store_true",
                    help="stack: run each layer of at most 2 rows as one launch (router, gate/up and down "
                         "workgroups; slower than the default two launches on MI355X)")
    ap.add_argument("--mode", choices=("softmax", "laguna"), default="softmax",
                    help="stack workload router: softmax top-8 (the benchmark configuration) or the pages' Laguna "
                         "tail (sigmoid + selection bias, routed scale 2.5) with norm weights and the residual stream")
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
    if args.workload == "lmhead":
        lmhead(args)
        return
    if args.workload == "prefill-stack":
        prefill_stack(args)
        return
    if args.workload == "layer-ksweep":
        layer_ksweep(args)
        return
    if args.workload == "kv":
        kv_ring(args)
        return

    import torch
    from speculative_block_verify_amd import api, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape, L, K, POOL, SEED = inputs.LAGUNA, 40, args.rows, 8, 2024
    laguna = args.mode == "laguna"
    t0 = time.time()
    layers = inputs.gen_stack(shape, L, SEED, device=dev, with_bias=laguna)
    residual = None
    if laguna:
        for w, g in zip(layers, inputs.gen_norm_weights(L, shape.hidden, SEED, device=dev)):
            w["norm_w"] = g
        residual = inputs.gen_x(K, shape.hidden, SEED, device=dev, tag="res")
    if K == 2:
        xs = [inputs.gen_x(K, shape.hidden, SEED + 1 + i, device=dev) for i in range(POOL)]
    else:
        xs = [inputs.gen_x_correlated(K, shape.hidden, SEED + 1 + i, device=dev) for i in range(POOL)]
    torch.cuda.synchronize()
    log("bench: generated %d layers (%.2f GB) in %.1f s" % (
        L, sum(sum(t.numel() for t in (w[m].values() if isinstance(w[m], dict) else [w[m]]))
               for w in layers for m in w if w[m] is not None) / 1e9, time.time() - t0))

    score_fn = api.MOE_SCORE_SIGMOID_BIAS if laguna else api.MOE_SCORE_SOFTMAX
    rs = 2.5 if laguna else 1.0
    cfg = api.make_cfg(shape, K, score_fn=score_fn, routed_scale=rs,
                       regime=api.MOE_REGIME_VERIFY_ONE_LAUNCH if args.one_launch else api.MOE_REGIME_AUTO)
    ws = api.alloc_workspace(cfg, dev)
    wts = [api.make_weights(w, cfg) for w in layers]
    y = torch.empty(K, shape.hidden, dtype=torch.int16, device=dev)
    y32 = torch.empty(K, shape.hidden, dtype=torch.float32, device=dev)

    # unique-expert counts and router logits per (input, layer) from the
    # debug copies of a direct stack call
    import numpy as np
    nu = torch.empty(L, dtype=torch.int32, device=dev)
    y32_layers = torch.empty(L, K, shape.hidden, dtype=torch.float32, device=dev)
    lg_layers = torch.empty(L, K, shape.n_experts, dtype=torch.float32, device=dev)
    step_bytes, gu_bytes, layer_bytes, uniques, logits_all = [], [], [], [], []
    gpu_layer0 = None
    for i in range(POOL):
        dbg = api.make_debug(n_unique=nu, logits=lg_layers, **({"y32": y32_layers} if i == 0 else {}))
        api.moe_verify_stack(cfg, wts, xs[i], y, ws, y32=y32, debug=dbg, residual=residual)
        torch.cuda.synchronize()
        if i == 0:
            gpu_layer0 = y32_layers[0].cpu().numpy()
        U = nu.cpu().tolist()
        uniques.append(U)
        logits_all.append(lg_layers.cpu().numpy())
        layer_bytes.append([api.moe_verify_weight_bytes(cfg, u, K) for u in U])
        step_bytes.append(sum(layer_bytes[-1]))
        gu_bytes.append([gateup_bytes(shape, u, K) for u in U])
    logits_all = np.stack(logits_all)                     # [POOL, L, K, E]
    u_by_layer = np.asarray(uniques, np.float64).mean(axis=0)
    log("bench: unique experts per layer (mean) %.2f; bytes per step %.4f GB" % (
        u_by_layer.mean(), sum(step_bytes) / POOL / 1e9))
    if laguna:
        # selection keys of the sigmoid router tail: sigmoid(logit) + bias
        bias = np.stack([w["router_bias"].cpu().numpy() for w in layers])[None, :, None, :]
        ties = near_tie_rows(1.0 / (1.0 + np.exp(-logits_all.astype(np.float64))) + bias, shape.top_k, 1e-6)
    else:
        ties = near_tie_rows(logits_all, shape.top_k)
    logit_dev = None
    if K > 2:
        # realised deviation of the correlated rows' logits from row 0's
        cp = logits_all[:, :, 1:K // 2 + 1, :] - logits_all[:, :, :1, :]
        logit_dev = [round(float(v), 5) for v in cp.std(axis=(0, 2, 3))]

    graphs = [api.StackGraph(cfg, wts, xs[i], y, ws, y32=y32, residual=residual) for i in range(POOL)]
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
    med_ms = statistics.median(per_step_ms)
    stalls = sum(1 for t in per_step_ms if t > 4 * med_ms)
    log("bench: %d steps in %.3f ms (wall %.3f ms): %.1f GB/s, %.1f us/stack" % (
        args.steps, total_ms, wall * 1e3, gbs, total_ms / args.steps * 1e3))

    # per-kernel timing pass: same inputs, kernels stamped by their own
    # dispatch (verify-width kernels; from 8 rows the stack runs the grouped
    # kernels, which this pass does not cover).  A layer of at most 2 rows is
    # one launch (router, gate/up and down workgroups): its down entry is 0
    # and its algorithmic bytes are the whole layer's.
    kt = {"route_gateup": [], "down": []}
    gu_rates, one_launch = [], None
    avg, achieved, gu_avg_bytes = None, None, None
    try:
        for s in range(args.timing_steps):
            ms = api.moe_verify_stack_timed(cfg, wts, xs[s % POOL], y, ws, y32=y32, residual=residual)
            if one_launch is None:
                one_launch = all(b == 0.0 for _, b in ms)
            for l, (a, b) in enumerate(ms):
                kt["route_gateup"].append(a); kt["down"].append(b)
                gu_rates.append((layer_bytes if one_launch else gu_bytes)[s % POOL][l])
    except api.MoEError as err:
        if err.code != api.MOE_ERR_UNSUPPORTED:
            raise
        log("bench: no per-kernel timing (%s)" % err)
    if gu_rates:
        avg = {k: sum(v) / len(v) for k, v in kt.items()}
        gu_avg_bytes = sum(gu_rates) / len(gu_rates)
        achieved = gu_avg_bytes / (avg["route_gateup"] / 1e3) / 1e9
        if one_launch:
            avg = {"layer": avg["route_gateup"]}
            log("bench: kernel average (us): one-launch layer %.2f; %.1f GB/s" % (avg["layer"] * 1e3, achieved))
        else:
            log("bench: kernel averages (us): router+gateup %.2f down %.2f; router+gateup %.1f GB/s" % (
                avg["route_gateup"] * 1e3, avg["down"] * 1e3, achieved))

    for g in graphs:
        g.close()

    one_layer = None
    if K == 2 and not args.no_extras and not laguna:
        one_layer = single_layer_timing(cfg, wts, xs, y, ws, y32)
        one_layer["gbs"] = round(sum(step_bytes) / POOL / L / (one_layer["median"] / 1e6) / 1e9, 1)
        log("bench: single layer %.2f us (median), %.1f GB/s" % (one_layer["median"], one_layer["gbs"]))
    ceiling = None if args.no_extras else stream_read_ceiling(dev)
    if ceiling:
        log("bench: streaming-read ceiling %.1f GB/s" % ceiling)
    hashes = None if args.no_extras else weight_hashes(layers)

    us_stack = total_ms / args.steps * 1e3
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
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": "40-layer NVFP4 MoE verify stack, K=%d rows%s%s" % (
                       K, "" if K == 2 else " (K sweep: rows 1..K/2 repeat row 0 plus noise)",
                       ", Laguna router tail (sigmoid + selection bias, normalised top-8, routed scale 2.5), "
                       "norm weights, residual stream" if laguna else ""), "hidden": shape.hidden,
                   "score_fn": "sigmoid+bias" if laguna else "softmax", "routed_scale": rs,
                   "residual_stream": laguna,
                   "experts": shape.n_experts, "top_k": shape.top_k, "inter": shape.inter,
                   "shared_inter": shape.shared_inter, "layers": L, "rows": K, "input_pool": POOL,
                   "weights": "NVFP4 (E2M1 + E4M3/16 + fp32 tensor scale), bf16 router/activations"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_stack": {"mean": round(us_stack, 2),
                         "median": round(med_ms * 1e3, 2),
                         "min": round(min(per_step_ms) * 1e3, 2), "max": round(max(per_step_ms) * 1e3, 2)},
        "stall_steps_over_4x_median": stalls,
        "bytes_per_step": round(sum(step_bytes) / POOL),
        "unique_experts_per_layer": round(float(u_by_layer.mean()), 3),
        "unique_experts_by_layer": [round(float(u), 2) for u in u_by_layer],
        "no_dedup_slots_per_layer": K * shape.top_k,
        "near_tie_rows": {"count": ties, "of": int(POOL * L * K), "rule": "k-th/(k+1)-th logit gap < 1e-5 max|l|"},
        "kernel_us": None if avg is None else {k: round(v * 1e3, 3) for k, v in avg.items()},
        "single_layer_us": one_layer,
        "stream_read_ceiling_gbs": ceiling,
        "roofline": None if avg is None else {
            "bound": "hbm", "kernel": "k_route_gateup" + (" (whole layer: router, gate/up, down)" if one_launch else ""),
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if K == 2 else None, "bytes_per_launch": round(gu_avg_bytes)},
        "wall_s": round(wall, 4),
    }
    if logit_dev is not None:
        result["correlated_row_logit_dev_by_layer"] = logit_dev
    result["seed"] = SEED
    result["weight_xxh3_by_layer"] = hashes
    result["device"] = torch.cuda.get_device_name(dev)
    result["rocm"] = torch.version.hip
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host (3 runs of the stack on one pinned core)")
        result["cpu_baseline"], result["parity"] = cpu_baseline(layers, xs[0], shape, K, 3, gpu_layer0, us_stack, gbs,
                                                                score_fn, rs, residual)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

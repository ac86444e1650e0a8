#!/usr/bin/env python3
"""Benchmark of the routed WNA16 MoE layer on one MI355X.

One step = one full layer (route + w13/SwiGLU + w2/scatter-add + convert) over
one batch of synthetic tokens, with every input already resident in HBM.
Each step uses a different routing batch drawn from the workload's
distributions (the expert weights stay the same), so consecutive steps touch
mostly different experts and the weight stream comes from HBM rather than
from the 256 MB last-level cache.

The default workload is the largest one, the large prefill (T=8192, hidden
4096, intermediate 2048, 256 experts, top-8, w13 4-bit group 128, w2 2-bit
group 64, Zipf routing), which is MFMA-bound; the same line carries, under
"decode", the decode-sized W2A16 layer (T=4, top-6, 2-bit group 128), which
is HBM-bound.  `--config 2/3/4` selects another workload as the headline.

Decode-shaped workloads run on codes in the prepared order by default: the
one-time moe_wna16_prepare reorder runs before warmup, outside the timed
region, and every step calls moe_wna16_forward_prepared (`--codes packed`
times the checkpoint order through moe_wna16_forward instead).  Prefill-shaped
workloads always use the checkpoint order.

Prints ONE JSON line.  `value` and `ms_per_step` come from K steps through the
plain entry point (no events).  The same K steps are then run again with
per-launch events (moe_wna16_forward_profiled, or the prepared entry with its
event array), whose kernel dispatches carry their own start/stop events;
`roofline` is for the kernel with the longest average duration in that pass,
and the per-step and per-launch p10/p50/p90 come from that pass.
`algorithmic_bytes` counts the packed codes and scales of the experts routed
to plus x and out; `implementation_bytes` lists this implementation's other
traffic (act round trip, FP32 sum).  `cpu_baseline` is the CPU oracle on a
bounded sample of the same workload.

`--quantize` measures the quantizer instead and prints its own line.
"""
import argparse
import ctypes
import ctypes.util
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, TFLOP/s
KERNEL_SOURCE = os.path.join(ROOT, "weight_only_bit_moe_amd", "csrc", "kernels.hip")
QUANT_SOURCE = os.path.join(ROOT, "weight_only_bit_moe_amd", "csrc", "quantize.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=5, choices=[2, 3, 4, 5])
    ap.add_argument("--no-decode-extra", dest="decode_extra", action="store_false",
                    help="do not add the decode workload's figures to a prefill line")
    ap.add_argument("--no-shards", dest="shards", action="store_false",
                    help="do not add the one-GPU shares of the sharded layer (expert "
                         "parallelism 8, tensor parallelism 4) to a prefill line")
    ap.add_argument("--batches", type=int, default=64,
                    help="distinct routing batches cycled over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline (0 disables it)")
    ap.add_argument("--traffic-file", default=None,
                    help="rocprofv3 counter summary holding the dominant kernel's HBM traffic")
    ap.add_argument("--codes", choices=["auto", "prepared", "packed"], default="auto",
                    help="code order: 'prepared' (moe_wna16_prepare once, outside the timed "
                         "region, then moe_wna16_forward_prepared; decode-shaped workloads "
                         "only), 'packed' (the checkpoint order), 'auto' = prepared for "
                         "decode-shaped workloads, packed otherwise")
    ap.add_argument("--quantize", action="store_true",
                    help="measure the quantizer instead of the layer (its own JSON line)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 times) "
                         "and exit: the reference reading for HBM byte counters")
    return ap.parse_args()


def copy_probe(mib):
    """Plain copy of a known size, for calibrating FETCH_SIZE / WRITE_SIZE."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_bytes": mib << 20, "repeats": 5}), flush=True)


class Hip:
    """The few HIP runtime calls the benchmark needs (events)."""

    def __init__(self):
        path = ctypes.util.find_library("amdhip64") or "/opt/rocm/lib/libamdhip64.so"
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, e, stream):
        if self.lib.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def per_expert_bytes(bits, group, rows, K):
    """Packed codes + FP16 scales of one expert's projection."""
    return rows * K * bits // 8 + rows * (K // group) * 2


def kernel_traffic(path, kernel, source=KERNEL_SOURCE):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    if not path or not os.path.exists(path):
        return None
    text = open(path).read()
    want = hashlib.sha256(open(source, "rb").read()).hexdigest()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(rf"traffic_bytes_per_launch\[{re.escape(kernel)}\]:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != want:
        return None
    return float(m_b.group(1))


def main():
    args = parse()
    if args.copy_mib:
        copy_probe(args.copy_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this layer has no multi-GPU path here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.quantize:
        bench_quantize(args)
        return

    import weight_only_bit_moe_amd as M
    if not os.path.exists(M.LIB_PATH):
        from weight_only_bit_moe_amd import build as hip_build
        hip_build.build()

    cfg = args.config
    result, L = measure_layer(cfg, args, args.steps, args.warmup, args.codes)
    if args.decode_extra and cfg not in (2, 3):
        # the decode half of the metric (HBM-bound, 4 tokens) on the same GPU,
        # with its own step counts: a ~40 us step needs a few hundred untimed
        # calls before the host's enqueue path and the clocks are steady
        dec, _ = measure_layer(2, args, None, None, "auto")
        result["decode"] = {k: dec[k] for k in (
            "value", "unit", "ms_per_step", "steps", "warmup", "config", "roofline", "kernel_ms",
            "step_ms_percentiles", "layer_hbm_gbs", "layer_hbm_frac", "experts_touched_per_step",
            "algorithmic_bytes")}
    if args.shards and cfg not in (2, 3):
        # one GPU's share of the sharded layer at its real shape: expert
        # parallelism over 8 GPUs (32 local experts) and tensor parallelism
        # over 4 (intermediate 512), for the decode and 2048-token workloads
        from weight_only_bit_moe_amd.inputs import shard_spec
        result["shards"] = {}
        for c in (2, 4):
            for sh in ("ep8", "tp4"):
                r, _ = measure_layer(c, args, None, None, "auto", spec=shard_spec(c, sh))
                result["shards"][r["config"]["workload"]] = {k: r[k] for k in (
                    "value", "unit", "ms_per_step", "steps", "warmup", "roofline", "kernel_ms",
                    "layer_hbm_frac", "layer_mfma_frac", "experts_touched_per_step",
                    "pairs_per_step")}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(L, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def percentiles(v):
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90))}


def measure_layer(cfg, args, steps, warmup, codes, spec=None):
    """Time `steps` layer calls on workload `cfg` (or `spec`, drawn with seed
    `cfg`) after `warmup` untimed ones.  Returns (the JSON dict of the
    measurement, the host layer)."""
    import numpy as np
    import torch

    import weight_only_bit_moe_amd as M
    from weight_only_bit_moe_amd.inputs import make_batch, make_config, make_layer

    decode = cfg in (2, 3)
    # Decode steps are ~40 us: a few hundred untimed calls bring the host's
    # enqueue path and the clocks to steady state (after 20 the launches of
    # one step were still ~3 us apart).
    steps = steps if steps is not None else (1000 if decode else 20)
    warmup = warmup if warmup is not None else (500 if decode else 10)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    L = make_config(cfg) if spec is None else make_layer(spec, cfg)
    sp = L.spec
    T, H, I, E, k = sp.T, sp.H, sp.I, sp.E, sp.topk
    P = T * k
    q13, q2 = (sp.bits13, sp.group13), (sp.bits2, sp.group2)
    plan = M.moe_wna16_plan(T, H, I, E, k, q13, q2)
    decode_shaped = plan["w13_variant"] == 2 and plan["w2_variant"] == 2
    if codes == "prepared" and not decode_shaped:
        print("--codes prepared needs a decode-shaped workload (--config 2 or 3)",
              file=sys.stderr)
        sys.exit(2)
    prepared = codes == "prepared" or (codes == "auto" and decode_shaped)
    w13 = torch.from_numpy(L.w13.view(np.int32)).to(dev)
    s13 = torch.from_numpy(L.s13).to(dev)
    w2 = torch.from_numpy(L.w2.view(np.int32)).to(dev)
    s2 = torch.from_numpy(L.s2).to(dev)
    if prepared:   # one-time setup, outside the timed region
        w13 = M.prepare(w13, sp.bits13, sp.group13)
        w2 = M.prepare(w2, sp.bits2, sp.group2)
        torch.cuda.synchronize(dev)
    nb = max(1, min(args.batches, steps))
    host_batches = [(L.topk_ids, L.topk_w, L.x)]
    for i in range(1, nb):
        host_batches.append(make_batch(sp, seed=cfg * 100000 + i,
                                       outlier_channels=L.outlier_channels))
    batches = []
    for ids, w, x in host_batches:
        batches.append((torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16),
                        torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)))
    ws = M.workspace_for(T, H, I, E, k, dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    fixed = (w13.data_ptr(), s13.data_ptr(), w2.data_ptr(), s2.data_ptr())
    call_args = []
    for x, ids, w in batches:
        call_args.append((x.data_ptr(), ids.data_ptr(), w.data_ptr()) + fixed +
                         (T, H, I, E, k, q13, q2, sp.alpha, sp.beta, sp.clamp, out.data_ptr(),
                          ws.data_ptr(), ws.numel(), stream))

    def step_plain(i):
        if prepared:
            st = M.moe_wna16_forward_prepared(*call_args[i % nb], None)
        else:
            st = M.moe_wna16_forward(*call_args[i % nb])
        if st != 0:
            raise M.MoeWna16Error(st, "moe_wna16_forward")

    hip = Hip()
    events = [(ctypes.c_void_p * 8)(*[hip.event() for _ in range(8)]) for _ in range(steps)]

    for i in range(warmup):
        step_plain(i)
    torch.cuda.synchronize(dev)

    # timed region: K steps through the plain entry point
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(steps):
        step_plain(i)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps

    # kernel durations: the same K steps again, each dispatch carrying start/stop
    # events in its own packet (the events add a gap after every kernel, so
    # this pass is not the one whose wall time is reported)
    torch.cuda.synchronize(dev)
    t2 = time.perf_counter()
    profiled = M.moe_wna16_forward_prepared if prepared else M.moe_wna16_forward_profiled
    for i in range(steps):
        st = profiled(*call_args[i % nb], events[i])
        if st != 0:
            raise M.MoeWna16Error(st, "moe_wna16_forward_profiled")
    torch.cuda.synchronize(dev)
    t3 = time.perf_counter()
    ms_events = (t3 - t2) * 1e3 / steps
    meta = M.workspace_meta(ws, T, H, I, E, k).cpu().numpy()
    if meta[2] != 0:
        raise RuntimeError(f"{meta[2]} fused decode waits gave up: the output is unreliable")

    # one entry per launch: steps that share a launch (plan: single_launch,
    # gemms_one_launch, convert_in_w2) are timed as that launch; with 64-row
    # tiles the routing step also holds the split of the tile kernels' items
    # over the XCDs
    one = bool(plan["gemms_one_launch"])
    if plan["single_launch"]:
        launches = [("layer", 0, 5)]
    else:
        launches = [("route" if decode_shaped else "route+split", 0, 1)]
        launches += [("w13+w2", 2, 5)] if one else [("w13", 2, 3), ("w2", 4, 5)]
        if not plan["convert_in_w2"]:
            launches.append(("convert", 6, 7))
    kern_ms = {name: [] for name, _, _ in launches}
    step_gpu_ms = []
    last_stop = launches[-1][2]
    for i in range(steps):
        ev = events[i]
        for name, a0, a1 in launches:
            kern_ms[name].append(hip.elapsed_ms(ev[a0], ev[a1]))
        step_gpu_ms.append(hip.elapsed_ms(ev[0], ev[last_stop]))
    avg = {n: float(np.mean(v)) for n, v in kern_ms.items()}
    for e in events:
        for h in e:
            hip.destroy(h)

    # algorithmic work of each step (bookkeeping from the routing ids):
    # bytes = packed codes + scales of the distinct experts routed to + x
    # (read by w13) + out (written after w2); flops = 2 P (2I H + H I)
    b13 = per_expert_bytes(sp.bits13, sp.group13, 2 * I, H)
    b2 = per_expert_bytes(sp.bits2, sp.group2, H, I)
    touched, pairs = [], []
    for i in range(steps):
        ids = host_batches[i % nb][0]
        local = ids[(ids >= 0) & (ids < E)]
        touched.append(len(np.unique(local)))
        pairs.append(local.size)   # pairs routed to this layer's experts
    mean_touched = float(np.mean(touched))
    Pl = float(np.mean(pairs))
    alg_bytes = {"w13": mean_touched * b13 + T * H * 2, "w2": mean_touched * b2 + T * H * 2}
    alg_flops = {"w13": 2.0 * Pl * 2 * I * H, "w2": 2.0 * Pl * H * I}
    alg_bytes["w13+w2"] = alg_bytes["w13"] + alg_bytes["w2"]
    alg_flops["w13+w2"] = alg_flops["w13"] + alg_flops["w2"]
    alg_bytes["layer"] = alg_bytes["w13+w2"]   # the single launch: the routing reads ids only
    alg_flops["layer"] = alg_flops["w13+w2"]
    layer_bytes = alg_bytes["w13+w2"]
    layer_flops = alg_flops["w13+w2"]
    # traffic of this implementation outside those bytes (not algorithmic):
    # act written by w13 and read by w2, the FP32 sum (atomics, then rounding)
    impl_bytes = {"act_write_read": 2.0 * P * I * 2, "fp32_sum": 3.0 * T * H * 4}

    dom = max((n for n in avg if n.startswith("w") or n == "layer"), key=lambda n: avg[n])
    if decode:
        achieved = alg_bytes[dom] / (avg[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = alg_flops[dom] / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS}
    roof["kernel"] = dom
    roof["kernel_ms"] = avg[dom]
    roof["algorithmic_bytes" if decode else "algorithmic_flops"] = (
        alg_bytes[dom] if decode else alg_flops[dom])
    traffic_file = args.traffic_file if cfg == args.config else None
    traffic_file = traffic_file or os.path.join(
        ROOT, "profiles", f"counters_{sp.name}{'-prepared' if prepared else ''}.md")
    roof["traffic"] = kernel_traffic(traffic_file, dom)

    value = T / (ms_per_step * 1e-3)
    result = {
        "metric": "routed-MoE layer tokens/s on 1 MI355X",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; fresh routing batch per step)",
        "config": {"workload": sp.name, "T": T, "hidden": H, "intermediate": I, "experts": E,
                   "routing_experts": sp.routing_experts or E,
                   "topk": k, "w13": f"W{sp.bits13} g{sp.group13}",
                   "w2": f"W{sp.bits2} g{sp.group2}", "block_m": plan["block_m"],
                   "codes": "prepared order" if prepared else "checkpoint order",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "kernel_ms": avg,
        "kernel_ms_percentiles": {n: percentiles(v) for n, v in kern_ms.items()},
        "step_ms_percentiles": percentiles(step_gpu_ms),
        "kernel_timing": "HIP events in each launch's dispatch packet, second pass of the "
                         "same K steps (same kernels) on the same stream; percentiles over "
                         "the K steps of that pass",
        "ms_per_step_with_events": ms_events,
        "gpu_ms_per_step_events": float(np.mean(step_gpu_ms)),
        "algorithmic_bytes": layer_bytes,
        "algorithmic_flops": layer_flops,
        "kernel_algorithmic_bytes": {n: alg_bytes[n] for n in avg if n in alg_bytes},
        "kernel_algorithmic_flops": {n: alg_flops[n] for n in avg if n in alg_flops},
        "implementation_bytes": impl_bytes,
        "layer_hbm_gbs": layer_bytes / (ms_per_step * 1e-3) / 1e9,
        "layer_hbm_frac": layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "layer_mfma_frac": layer_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "experts_touched_per_step": mean_touched,
        "pairs_per_step": Pl,
    }
    del batches, w13, w2, s13, s2, ws, out
    torch.cuda.empty_cache()
    return result, L


# Lane operations per (weight, candidate) of the quantizer's definition: the
# division, the rounding, two clamp comparisons, s*q, the subtraction, two
# multiplications by imp and d, and the addition into the group's error.
QUANT_OPS_PER_EVAL = 9
# One VALU lane operation per lane per clock: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def bench_quantize(args):
    """All routed experts of one layer quantized on the GPU (2-bit, group 128,
    16-candidate importance-weighted scale search): the fused gate/up matrices
    [256*4096, 4096] and the down matrices [256*4096, 2048]."""
    import numpy as np
    import torch

    import weight_only_bit_moe_amd as M
    from weight_only_bit_moe_amd.inputs import (QUANT_WORKLOAD, make_dense_weights_device,
                                                make_importance)

    if not os.path.exists(M.LIB_PATH):
        from weight_only_bit_moe_amd import build as hip_build
        hip_build.build()
    steps = args.steps if args.steps is not None else 10
    warmup = args.warmup if args.warmup is not None else 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ops = []
    for j, sp in enumerate(QUANT_WORKLOAD):
        w = make_dense_weights_device(sp.rows, sp.K, 1000 + j, dev, sp.w_std)
        imp = torch.from_numpy(make_importance(sp.K, 2000 + j, sp.imp_sigma, sp.outlier_frac,
                                               sp.outlier_mult)).to(dev)
        codes = torch.empty((sp.rows, sp.K * sp.bits // 32), dtype=torch.int32, device=dev)
        scales = torch.empty((sp.rows, sp.K // sp.group), dtype=torch.float16, device=dev)
        sums = torch.empty(4, dtype=torch.float64, device=dev)
        ops.append((sp, w, imp, codes, scales, sums))
    torch.cuda.synchronize(dev)

    def call(sp, w, imp, codes, scales, sums):
        st = M.moe_wna16_quantize(w.data_ptr(), imp.data_ptr(), sp.rows, sp.K,
                                  (sp.bits, sp.group), sp.ncand, codes.data_ptr(),
                                  scales.data_ptr(), sums.data_ptr(), stream)
        if st != 0:
            raise M.MoeWna16Error(st, "moe_wna16_quantize")

    hip = Hip()
    evs = [[(hip.event(), hip.event()) for _ in ops] for _ in range(steps)]
    for _ in range(warmup):
        for o in ops:
            call(*o)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(steps):
        for j, o in enumerate(ops):
            hip.record(evs[i][j][0], stream)
            call(*o)
            hip.record(evs[i][j][1], stream)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    call_ms = [float(np.mean([hip.elapsed_ms(*evs[i][j]) for i in range(steps)]))
               for j in range(len(ops))]
    for row in evs:
        for a, b in row:
            hip.destroy(a)
            hip.destroy(b)

    n_weights = sum(sp.rows * sp.K for sp, *_ in ops)
    j = int(np.argmax(call_ms))
    sp = ops[j][0]
    evals = sp.rows * sp.K * sp.ncand
    achieved = QUANT_OPS_PER_EVAL * evals / (call_ms[j] * 1e-3) / 1e12
    hbm_bytes = sp.rows * sp.K * (2 + sp.bits / 8) + sp.rows * (sp.K // sp.group) * 2
    workload = "quantize-E256-H4096-I2048-w2g128-C16"
    traffic_file = args.traffic_file or os.path.join(ROOT, "profiles",
                                                     f"counters_{workload}.md")
    roof = {"bound": "alu", "achieved": achieved, "peak": ALU_PEAK_TOPS, "unit": "Top/s",
            "frac": achieved / ALU_PEAK_TOPS,
            "traffic": kernel_traffic(traffic_file, sp.name, QUANT_SOURCE),
            "kernel": "quantize_kernel (" + sp.name + ")", "kernel_ms": call_ms[j],
            "algorithmic_ops": QUANT_OPS_PER_EVAL * evals,
            "hbm_gbs": hbm_bytes / (call_ms[j] * 1e-3) / 1e9}

    # weighted reconstruction error of the search against plain RTN (one
    # candidate) on 24 single-expert matrices: 12 experts' gate/up and down
    red = []
    for e in range(12):
        for sp_, w, imp, codes, scales, sums in ops:
            rows = sp_.rows // 256
            sub = w[e * rows:(e + 1) * rows]
            r1 = M.quantize(sub, sp_.bits, sp_.group, 1, imp)["sums"]
            rc = M.quantize(sub, sp_.bits, sp_.group, sp_.ncand, imp)["sums"]
            red.append(1.0 - float(rc[2]) / float(r1[2]))
    result = {
        "metric": "routed-expert weights quantized per second on 1 MI355X",
        "value": n_weights / (ms_per_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+f64",
        "data": "synthetic (seeded Student-t weights, lognormal importance with 1% hot channels)",
        "config": {"workload": workload,
                   "matrices": [f"{sp_.name}: [{sp_.rows}, {sp_.K}]" for sp_, *_ in ops],
                   "bits": sp.bits, "group": sp.group, "candidates": sp.ncand,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "call_ms": call_ms,
        "weighted_error_reduction_vs_rtn": {
            "median": float(np.median(red)), "min": float(np.min(red)),
            "max": float(np.max(red)), "matrices": len(red)},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_quantize(ops[0], args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def cpu_baseline_quantize(op, budget_s):
    """The CPU oracle's quantizer (single thread, float64 errors) on leading
    rows of the first matrix, as many as fit the time budget."""
    import numpy as np
    import torch

    from oracle import oracle

    sp, w, imp, *_ = op
    imp_h = imp.cpu().numpy()
    rows = 64
    t0 = time.perf_counter()
    oracle.quantize(w[:rows].view(torch.int16).cpu().numpy().view(np.uint16), sp.bits, sp.group,
                    sp.ncand, imp_h)
    per_row = (time.perf_counter() - t0) / rows
    rows = int(max(rows, min(sp.rows, budget_s / max(per_row, 1e-9))))
    wh = w[:rows].view(torch.int16).cpu().numpy().view(np.uint16)
    t0 = time.perf_counter()
    oracle.quantize(wh, sp.bits, sp.group, sp.ncand, imp_h)
    el = time.perf_counter() - t0
    return {"value": rows * sp.K / el, "unit": "weights/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {sp.rows} rows of {sp.name}, {el:.1f} s"}


def cpu_baseline(L, budget_s):
    """The CPU oracle (float64, OpenMP over (token, slot) pairs) timed on this
    host over a bounded sample of the workload's tokens."""
    import numpy as np

    from oracle import oracle

    sp = L.spec
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    # sample: whole batches when the batch is small, else a slice of tokens;
    # the probe holds enough pairs to keep every thread busy, like the sample
    n0 = min(sp.T, -(-threads // sp.topk))
    t0 = time.perf_counter()
    probe = oracle.forward_layer(L, tokens=list(range(n0)), nthreads=threads)
    per_token = (time.perf_counter() - t0) / n0
    ntok = int(max(1, min(sp.T, budget_s / max(per_token, 1e-6))))
    tokens = list(range(ntok))
    done, elapsed, reps = 0, 0.0, 0
    while elapsed < budget_s or reps == 0:
        t0 = time.perf_counter()
        oracle.forward_layer(L, tokens=tokens, nthreads=threads)
        elapsed += time.perf_counter() - t0
        done += ntok
        reps += 1
        if ntok < sp.T:
            break
    used = min(threads, ntok * sp.topk)
    del probe
    return {"value": done / elapsed, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{ntok} of {sp.T} tokens x {reps} pass(es) of workload {sp.name}, "
                      f"{elapsed:.1f} s, float64"}


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


if __name__ == "__main__":
    main()

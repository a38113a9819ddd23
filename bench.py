"""Benchmark of the routed MoE expert-FFN layer on one MI355X.

Workload (the headline one): single-token decode, M=1, hidden 2048,
per-expert intermediate 768, 128 experts, top-8, AWQ-style int4 weights with
group 128 (fp16 scales, uint8 zeros), bf16 activations. A step is one call of
the whole layer (moe_ffn_forward; at M=1 the automatic path is the
output-stationary decode path, which has no alignment step by design). Every
step uses the next of 16 device copies of the packed layer (16 x 316 MB, more
than the 256 MB Infinity Cache) and the next of 64 seeded routings, so each
call streams cold weights from HBM. The timed region replays a HIP graph of K
steps between two synchronised events.

Printed: one JSON line with tokens/s, the per-kernel roofline of the dominant
kernel (decode gate/up, timed with events around each kernel in a separate
pass), the oracle's CPU throughput on a bounded sample, and the M=21 / M=256
layer numbers as extra context.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_LAYER_COPIES = 16
N_ROUTINGS = 64
FLOPS_PER_ROUTE = None  # set from the shapes: 2 * (2I*H + H*I)


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_counters.json")
KERNEL_SOURCES = {
    # kernel family -> sources its code is built from
    "decode": ["decode.hip", "common.hpp"],
    "grouped": ["grouped.hip", "common.hpp"],
}


def source_hash(family):
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mixture_experts_ffn_align_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, family):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    FETCH_SIZE / WRITE_SIZE counter passes (calibrated on a plain copy), or
    None when there is no record or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = rec.get("kernels", {}).get(f"{workload}:{kernel}")
    if not entry or entry.get("source_hash") != source_hash(family):
        return None
    return int(entry["hbm_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 64 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 20}), flush=True)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="decode_m1")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the M=21 / M=256 context numbers")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 64 MiB device copy (the counter calibration kernel) and exit")
    p.add_argument("--grouped-sweep", default=None, metavar="FMT",
                   help="only run the grouped-GEMM shape sweep on the batched layout (int4 or mxfp8) and exit")
    return p.parse_args()


def _clone_projection(p):
    import mixture_experts_ffn_align_amd as moe
    return moe.DeviceProjection(p.fmt, p.group, p.q.clone(), p.scale.clone(),
                                None if p.zero is None else p.zero.clone())


class Rotation:
    """Device inputs for one workload: layer copies and routings."""

    def __init__(self, name, n_layers, n_routings, seed=0):
        import torch
        import mixture_experts_ffn_align_amd as moe
        from workloads import CONFIGS, make_weights
        from workloads.gen import make_routing, make_x
        self.cfg = cfg = CONFIGS[name]
        w13, w2 = make_weights(cfg, seed, 0)
        self.w13_host, self.w2_host = w13, w2
        base13 = moe.DeviceProjection.from_host(w13, "cuda")
        base2 = moe.DeviceProjection.from_host(w2, "cuda")
        self.layers = []
        for i in range(n_layers):
            p13 = base13 if i == 0 else _clone_projection(base13)
            p2 = base2 if i == 0 else _clone_projection(base2)
            self.layers.append(moe.MoeLayer(p13, p2, cfg.E, cfg.H, cfg.I, cfg.k, cfg.b))
        self.inputs = []
        self.host_inputs = []
        for r in range(n_routings):
            ids, w = make_routing(cfg, seed, r)
            x = make_x(cfg, seed, r)
            self.host_inputs.append((x, ids, w))
            self.inputs.append((torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16),
                                torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()))
        self.y = torch.empty((cfg.M, cfg.H), dtype=torch.float32, device="cuda")
        d = self.layers[0].desc(cfg.M)
        self.ws = torch.empty(moe.moe_ffn_workspace_size(d), dtype=torch.uint8, device="cuda")
        self.touched = [len(np.unique(h[1])) for h in self.host_inputs]

    def step(self, i, profiled_events=None):
        import mixture_experts_ffn_align_amd as moe
        layer = self.layers[i % len(self.layers)]
        x, ids, w = self.inputs[i % len(self.inputs)]
        d = layer.desc(self.cfg.M)
        if profiled_events is None:
            moe.moe_ffn_forward(d, x, ids, w, self.y, self.ws)
        else:
            moe.moe_ffn_forward_profiled(d, x, ids, w, self.y, self.ws, profiled_events)

    def expert_bytes(self):
        return self.w13_host.expert_bytes() + self.w2_host.expert_bytes(), \
            self.w13_host.expert_bytes(), self.w2_host.expert_bytes()


def time_graph(rot, steps, warmup):
    """Milliseconds for `steps` layer calls replayed from HIP graphs."""
    import torch
    stream = torch.cuda.Stream()
    chunk = min(steps, 1024)
    graphs = []
    with torch.cuda.stream(stream):
        for i in range(3):            # eager warm-up of the code objects
            rot.step(i)
    torch.cuda.synchronize()

    def capture(n, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                rot.step(start + i)
        return g

    full, rem = divmod(steps, chunk)
    g_main = capture(chunk, 0)
    g_rem = capture(rem, chunk) if rem else None
    wg = capture(max(1, min(warmup, 1024)), 7) if warmup > 0 else None
    torch.cuda.synchronize()
    if wg is not None:
        for _ in range(max(1, warmup // 1024)):
            wg.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    t0.record(cur)
    for _ in range(full):
        g_main.replay()
    if g_rem is not None:
        g_rem.replay()
    t1.record(cur)
    torch.cuda.synchronize()
    del graphs
    return t0.elapsed_time(t1)


def stage_times(rot, steps):
    """Average duration (us) of each stage of the layer, each replayed alone
    from a HIP graph over the same rotation (moe_ffn_gate_up, then
    moe_ffn_down_combine). On the decode path each stage is exactly one
    kernel, so this is the per-kernel duration a kernel trace reports."""
    import torch
    import mixture_experts_ffn_align_amd as moe

    def gate_up(i):
        layer = rot.layers[i % len(rot.layers)]
        x, ids, _ = rot.inputs[i % len(rot.inputs)]
        moe.moe_ffn_gate_up(layer.desc(rot.cfg.M), x, ids, rot.ws)

    def down(i):
        layer = rot.layers[i % len(rot.layers)]
        _, ids, w = rot.inputs[i % len(rot.inputs)]
        moe.moe_ffn_down_combine(layer.desc(rot.cfg.M), ids, w, rot.y, rot.ws)

    out = {}
    for name, fn in (("gate_up", gate_up), ("down_combine", down)):
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for i in range(3):
                fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        out[name] = t0.elapsed_time(t1) * 1e3 / steps
    return out


def cpu_baseline(rot, seconds):
    """The fp64 oracle on the host: tokens/s over a bounded sample of the same
    workload (rotating routings; one layer)."""
    import psutil
    import oracle
    cfg = rot.cfg
    proc = psutil.Process()
    n = 0
    c0 = proc.cpu_times()
    t0 = time.perf_counter()
    while True:
        x, ids, w = rot.host_inputs[n % len(rot.host_inputs)]
        oracle.ffn(x, ids, w, rot.w13_host, rot.w2_host, cfg.E)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    wall = time.perf_counter() - t0
    c1 = proc.cpu_times()
    busy = (c1.user - c0.user) + (c1.system - c0.system)
    return {
        "value": n * cfg.M / wall, "unit": "tokens/s",
        "cores": max(1, int(math.ceil(busy / wall - 0.05))),
        "kind": "oracle",
        "sample": f"{n} layer calls of the {cfg.name} workload (M={cfg.M}) on one layer, "
                  f"{wall:.1f} s wall, {busy / wall:.2f} average busy threads "
                  f"of {len(os.sched_getaffinity(0))} available",
    }


def layer_numbers(rot, steps):
    ms = time_graph(rot, steps, warmup=min(steps, 64))
    t = ms / steps * 1e-3
    cfg = rot.cfg
    per_expert, _, _ = rot.expert_bytes()
    touched = float(np.mean([rot.touched[i % len(rot.touched)] for i in range(steps)]))
    bytes_per_call = touched * per_expert
    flops = cfg.M * cfg.k * 2 * (2 * cfg.I * cfg.H + cfg.H * cfg.I)
    return {
        "tokens_per_s": cfg.M / t, "us_per_layer": t * 1e6,
        "effective_weight_GBps": bytes_per_call / t / 1e9,
        "hbm_frac": bytes_per_call / t / 1e9 / HBM_PEAK_GBPS,
        "mfma_frac_bf16": flops / t / 1e12 / BF16_PEAK_TFLOPS,
        "touched_experts_mean": touched,
    }


SWEEP_G = (8, 16, 32, 64, 128)
SWEEP_N = (16, 32, 64, 128, 256, 512, 1024)
SWEEP_COLD_BYTES = 640 << 20    # weight copies rotated per point: more than the 256 MB Infinity Cache


def grouped_sweep(fmt):
    """The two grouped GEMMs of a Qwen3-30B-A3B-shaped layer (gate/up: 1536 x
    2048, down: 2048 x 768; H = 2048, I = 768) on the fixed-capacity batched
    layout, over G experts and a maximum of N tokens per expert with the
    ragged counts {N, 3N/4, N/2, N/4} repeated over the experts. Median
    graph-replay latency per call over cold weight copies; TFLOP/s_eff counts
    2 M K sum(N_g) (unpadded); weight GB/s counts the G experts' packed bytes."""
    import dataclasses
    import statistics
    import torch
    import mixture_experts_ffn_align_amd as moe
    from workloads import CONFIGS, make_weights
    base = CONFIGS["mxfp8_m64" if fmt == "mxfp8" else "batch_m256_zipf"]
    cfg = dataclasses.replace(base, E=max(SWEEP_G), b=64)
    w13, w2 = make_weights(cfg, 0, 0)
    H, I = cfg.H, cfg.I
    full13 = moe.DeviceProjection.from_host(w13, "cuda")
    full2 = moe.DeviceProjection.from_host(w2, "cuda")
    per13 = full13.nbytes() / cfg.E
    per2 = full2.nbytes() / cfg.E
    rng = np.random.default_rng(0)
    rows = []
    for G in SWEEP_G:
        def take(p):
            return moe.DeviceProjection(p.fmt, p.group, p.q[:G].clone(), p.scale[:G].clone(),
                                        None if p.zero is None else p.zero[:G].clone())
        copies = max(2, int(math.ceil(SWEEP_COLD_BYTES / (G * (per13 + per2)))))
        layers = [moe.MoeLayer(take(full13), take(full2), G, H, I, 1, 64) for _ in range(copies)]
        for N in SWEEP_N:
            counts_l = [[N, 3 * N // 4, N // 2, N // 4][e % 4] for e in range(G)]
            counts = torch.tensor(counts_l, dtype=torch.int32, device="cuda")
            xv = rng.standard_normal((G, N, H)).astype(np.float32)
            xb = torch.from_numpy((xv.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).cuda() \
                .view(torch.bfloat16)
            a16 = torch.zeros((G, N, I), dtype=torch.float16, device="cuda")
            asc = torch.zeros((G, N, I // 128, 4), dtype=torch.float32, device="cuda")
            yb = torch.zeros((G, N, H), dtype=torch.float32, device="cuda")
            descs = [L.desc(1) for L in layers]
            stages = {
                "gate_up": (lambda d: moe.moe_ffn_gate_up_batched(d, xb, counts, a16, asc), 2 * I, H, per13),
                "down": (lambda d: moe.moe_ffn_down_batched(d, a16, asc, counts, yb), H, I, per2),
            }
            for name, (fn, Mdim, Kdim, per) in stages.items():
                stream = torch.cuda.Stream()
                with torch.cuda.stream(stream):
                    for d in descs[:2]:
                        fn(d)
                torch.cuda.synchronize()
                reps = max(copies, 16)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(reps):
                        fn(descs[i % copies])
                g.replay()
                torch.cuda.synchronize()
                times = []
                for _ in range(5):
                    t0 = torch.cuda.Event(enable_timing=True)
                    t1 = torch.cuda.Event(enable_timing=True)
                    t0.record()
                    g.replay()
                    t1.record()
                    torch.cuda.synchronize()
                    times.append(t0.elapsed_time(t1) * 1e3 / reps)
                us = statistics.median(times)
                flops = 2.0 * Mdim * Kdim * sum(counts_l)
                rows.append({"layer": name, "G": G, "N": N, "us": round(us, 2),
                             "tflops_eff": round(flops / (us * 1e-6) / 1e12, 2),
                             "weight_GBps": round(G * per / (us * 1e-6) / 1e9, 1),
                             "hbm_frac": round(G * per / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                             "mfma_frac": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)})
                log(json.dumps(rows[-1]))
            del xb, a16, asc, yb
        del layers
        torch.cuda.empty_cache()
    print(json.dumps({"grouped_sweep": fmt, "shapes": "Qwen3-30B-A3B H=2048 I=768", "rows": rows}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the layer is measured on one GPU; sharding across GPUs is a design, not run here: use --gpus 1"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.grouped_sweep:
        grouped_sweep(args.grouped_sweep)
        return
    import mixture_experts_ffn_align_amd as moe
    moe.lib()  # fail loudly if the HIP library is missing

    log("preparing", args.workload)
    rot = Rotation(args.workload, N_LAYER_COPIES, N_ROUTINGS)
    cfg = rot.cfg
    log("timing", args.steps, "steps")
    ms = time_graph(rot, args.steps, args.warmup)
    t_step = ms / args.steps
    tokens_s = cfg.M * args.steps / (ms * 1e-3)
    per_expert, b13, b2 = rot.expert_bytes()
    touched = float(np.mean([rot.touched[i % N_ROUTINGS] for i in range(args.steps)]))
    layer_gbps = touched * per_expert / (t_step * 1e-3) / 1e9

    log("per-stage timing")
    st_us = stage_times(rot, 512)
    d = rot.layers[0].desc(cfg.M)
    path = "decode" if moe.moe_ffn_kernel_count(d) == 2 else "grouped"
    # Algorithmic bytes of a stage: the packed weights (values, scales, zeros)
    # of every touched expert for that projection, each read once.
    stage_bytes = {"gate_up": touched * b13, "down_combine": touched * b2}
    dom = max(st_us, key=st_us.get)
    names = {"gate_up": moe.moe_ffn_kernel_name(d, 0 if path == "decode" else 1),
             "down_combine": moe.moe_ffn_kernel_name(d, 1 if path == "decode" else 2)}
    achieved = stage_bytes[dom] / (st_us[dom] * 1e-6) / 1e9
    traffic = measured_traffic(names[dom], cfg.name, path)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": names[dom], "kernel_us": round(st_us[dom], 3),
                "algorithmic_bytes": int(stage_bytes[dom]),
                "stage_us": {k: round(v, 3) for k, v in st_us.items()},
                "stage_GBps": {k: round(stage_bytes[k] / (v * 1e-6) / 1e9, 1) for k, v in st_us.items()}}

    extra = {}
    if not args.no_extra:
        for name in ("batch_m21", "batch_m256_zipf", "mxfp8_m64"):
            log("context workload", name)
            r2 = Rotation(name, 8, 16)
            extra[name] = {k: (round(v, 4) if isinstance(v, float) else v)
                           for k, v in layer_numbers(r2, 64).items()}
            del r2
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(rot, args.cpu_seconds)

    out = {
        "metric": "MoE-layer tokens/s and effective weight GB/s at M=1/21/256; % HBM/MFMA peak",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; int4 weights drawn uniformly, bf16 N(0,1) activations, softmax top-k routing)",
        "config": {"workload": f"{cfg.name}: M={cfg.M} H={cfg.H} I={cfg.I} E={cfg.E} top-{cfg.k} "
                               f"int4 AWQ g{cfg.g}, cold weights ({N_LAYER_COPIES} layer copies x "
                               f"{N_ROUTINGS} routings rotated)",
                   "M": cfg.M, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k, "group": cfg.g,
                   "path": path,
                   "parallelism": "single GPU"},
        "effective_weight_GBps": round(layer_gbps, 1),
        "hbm_frac_layer": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "other_workloads": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Decode MoE layer benchmark on one MI355X.

Workload: the Flint-shaped W4A16 layer (hidden 2048, 256 NVFP4 experts, top-6, one
NVFP4 shared expert, intermediate 768) on synthetic seeded weights and tokens.

A step is one decode pass of the whole layer (router + top-k, gate/up + SwiGLU, down +
combine) over one batch of T tokens, through each of R distinct device replicas of the
layer (same bytes at different addresses, so neither the L2 nor the 256 MB Infinity
Cache can serve a later layer's weights). The R passes are captured once into a HIP
graph, and one replay is one step. Per-layer time is step time / R.

Reported value: achieved HBM GB/s of the layer = algorithmic bytes per layer / time per
layer, where the bytes are the FP32 router weight, the unique experts the routing
actually selected, the shared expert, and x and y (BF16). The same line carries the
other batch sizes of the 1-8 sweep, the decode points of the other configurations
(Inkling-shaped W4A4 and MXFP8, Mistral-shaped MXFP4 with BF16, FP8 or MXFP4 activations,
Flint-shaped BF16; "configs"), the roofline of the dominant kernel (its own bytes over its
own average duration, from start/stop events the library takes around each dispatch),
and the CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer decode µs/layer and achieved HBM GB/s (% of peak) at batch 1–8"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_bit_fp32_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("src_sha") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def requant_bench(args, dev) -> int:
    """Load-time requantization of the Flint-shaped routed gate/up stack (256 experts x
    [2I = 1536][H = 2048] BF16, 805 MB, seeded N(0, 0.02) drawn on the device) to MXFP4,
    MXFP8 and NVFP4 (512 tensors: gate and up of each expert). Algorithmic bytes: the BF16
    input read once plus the codes and scales (and tensor scales) written."""
    import torch

    import block_scaled_bit_fp32_amd as moe
    import synth

    cfg = synth.CONFIGS["flint_bf16"]
    E, I, H = cfg.E, cfg.I, cfg.H
    gen = torch.Generator(device=dev).manual_seed(0x4F36)
    w = (torch.randn(E * 2 * I, H, device=dev, generator=gen) * 0.02).to(torch.bfloat16).view(torch.int16)
    n = w.numel()
    runs = {
        "mxfp4": (lambda: moe.requant_mxfp4(w), n * 2 + n // 2 + n // 32),
        "mxfp8": (lambda: moe.requant_mxfp8(w), n * 2 + n + n // 32),
        "nvfp4": (lambda: moe.requant_nvfp4(w.view(E * 2, I, H)), n * 2 + n // 2 + n // 16 + 4 * E * 2),
    }
    res = {}
    for name, (fn, nbytes) in runs.items():
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(args.steps):
            fn()
        s1.record()
        torch.cuda.synchronize()
        us = s0.elapsed_time(s1) * 1e3 / args.steps
        res[name] = {"us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}
        log(f"[bench] requant {name}: {us:.1f} us for {nbytes / 1e6:.1f} MB, {nbytes / us / 1e3:.0f} GB/s")
    print(json.dumps({"metric": "load-time requantization, achieved HBM GB/s", "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                      "config": {"workload": f"BF16 routed gate/up stack E={E} x [{2 * I}][{H}]"},
                      "dtype": "bf16->fp4/fp8", "peak": HBM_PEAK_GBPS, "results": res}))
    return 0


def cpu_info() -> dict:
    """The host's CPU model and numpy's BLAS, for the CPU baseline's record."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy as np
        deps = np.__config__.CONFIG.get("Build Dependencies", {})
        b = deps.get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


# Decode points of the other configurations, timed after the headline sweep (the
# quantized-activation layers run the in-kernel token and h quantizers; Mistral a8w4 at
# 64 tokens and Flint BF16 at 256 run the grouped MFMA kernels).
EXTRA_CONFIGS = [("inkling_w4a4", (1, 4, 8)), ("mistral_mxfp4_a8", (1, 8, 64)), ("mistral_mxfp4_a4", (1, 8)),
                 ("mistral_mxfp4", (1, 8)), ("inkling_mxfp8_a8", (1, 8)), ("flint_bf16", (1, 8, 256))]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="flint_w4a16")
    ap.add_argument("--batch", type=int, default=8, help="tokens per step for the headline value")
    ap.add_argument("--sweep", default="1,2,4,8", help="batch sizes also reported")
    ap.add_argument("--replicas", type=int, default=0, help="0: enough to touch >= 1 GiB per step")
    ap.add_argument("--cpu-sample-s", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations' decode points")
    ap.add_argument("--requant", action="store_true",
                    help="time the load-time requantizers instead (BF16 -> MXFP4 / MXFP8 / NVFP4)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: it measures the decode MoE layer on a single "
              "MI355X (across GPUs the layer would be split over the expert intermediate "
              "dimension with one all-reduce of y); pass --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_scaled_bit_fp32_amd as moe
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.requant:
        return requant_bench(args, dev)

    # copy bandwidth of this GPU, for reference (2 GiB read + 2 GiB written)
    src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 31) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    def time_layer(cfg, dl0, Ts, steps, warmup, kernels=True, replicas=0):
        """Graph-timed decode points of one layer: R device replicas (distinct addresses, so
        the caches cannot serve a later replica's weights), one moe_forward per replica per
        step; per-kernel times from the library's dispatch events."""
        layer_bytes_total = sum(v.numel() * v.element_size() for part in dl0.t.values() if part is not None
                                for v in (part.values() if isinstance(part, dict) else [part]) if v is not None)
        per_expert = dl0.nbytes_expert("routed", 0)
        shared_b = dl0.nbytes_expert("shared", 0) if cfg.has_shared else 0
        b_t1 = cfg.E * cfg.H * 4 + cfg.k * per_expert + shared_b
        R = replicas or max(8, math.ceil((1 << 30) / b_t1))
        R = max(1, min(R, int(150e9 // layer_bytes_total)))
        log(f"[bench] {cfg.name}: {R} replicas of {layer_bytes_total / 1e6:.0f} MB")
        layers = [dl0] + [dl0.copy() for _ in range(R - 1)]
        torch.cuda.synchronize()
        w13 = dl0.t["w13"]
        per13 = sum(v[0].numel() * v.element_size() for v in w13.values() if v is not None)
        sh13 = sum(v[0].numel() * v.element_size() for v in dl0.t["sh13"].values()
                   if v is not None) if cfg.has_shared else 0

        def bytes_of(kind: str, U: int, T: int) -> int:
            """Algorithmic HBM bytes one launch of a kernel moves."""
            xb = T * cfg.H * 2
            P = T * cfg.k + (T if cfg.has_shared else 0)
            if kind == "route":
                return cfg.E * cfg.H * 4 + (cfg.E * 4 if cfg.router_bias else 0) + xb
            if kind == "topk":
                return T * cfg.E * 4 + T * cfg.k * 8
            if kind == "combine":
                return P * cfg.H * 4 + T * cfg.k * 4 + xb
            if kind == "hquant":
                return T * cfg.k * cfg.I * 4
            if kind == "gateup":
                return U * per13 + sh13 + xb
            return U * (per_expert - per13) + (shared_b - sh13) + xb  # down: weights + y (BF16)

        points = []
        for T in Ts:
            x = torch.from_numpy(synth.make_x(cfg, T).view(np.int16)).to(dev)
            ws = moe.Workspace(dl0, T, device=dev)
            y, ids, w, xq = moe.forward(dl0, x, ws)
            torch.cuda.synchronize()
            U = len(np.unique(ids.cpu().numpy()))
            bpl = moe.routed_bytes(dl0, ids.cpu().numpy(), T)

            def one_pass():   # one moe_forward call per layer: router, experts, combine
                for dl in layers:
                    moe.forward(dl, x, ws, out=(y, ids, w, xq))

            one_pass()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_pass()
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            for _ in range(steps):
                g.replay()
            s1.record()
            torch.cuda.synchronize()
            ms_step = s0.elapsed_time(s1) / steps
            us_layer = ms_step * 1e3 / R
            kern = {}
            if kernels:   # per-kernel device time, same replicas, eager launches with dispatch events
                moe.profile_begin()
                for _ in range(max(1, steps // 4)):
                    one_pass()
                prof = moe.profile_end()
                for kind in ("route", "topk", "gateup", "hquant", "down", "combine"):
                    n, tot = prof.get(kind, (0, 0.0))
                    if n:
                        us = tot * 1e3 / n
                        kb = bytes_of(kind, U, T)
                        kern[kind] = {"us": round(us, 3), "bytes": kb, "GBps": round(kb / us / 1e3, 1)}
            gbps = bpl / us_layer / 1e3
            pt = {"T": T, "us_per_layer": round(us_layer, 3), "tokens_per_s": round(T / us_layer * 1e6),
                  "unique_experts": U, "bytes_per_layer": bpl, "GBps": round(gbps, 1),
                  "frac_peak": round(gbps / HBM_PEAK_GBPS, 4), "frac_copy": round(gbps / copy_gbps, 4),
                  "ms_per_step": ms_step, "replicas": R}
            if kernels:
                pt["kernels"] = kern
            points.append(pt)
            log(f"[bench] {cfg.name} T={T} U={U} {us_layer:.2f} us/layer {gbps:.0f} GB/s "
                f"({100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s) kernels {kern}")
            del g
            torch.cuda.synchronize()
        del layers
        torch.cuda.empty_cache()
        return points

    cfg = synth.CONFIGS[args.config]
    sweep = sorted(set([int(t) for t in args.sweep.split(",") if t] + [args.batch]))
    log(f"[bench] drawing layer {cfg.name}")
    host = synth.make_layer(cfg)
    dl0 = moe.DeviceLayer.from_host(host, device=dev)
    points = time_layer(cfg, dl0, sweep, args.steps, args.warmup, replicas=args.replicas)
    head = next(p for p in points if p["T"] == args.batch)
    head_ms = head.pop("ms_per_step")
    R = head["replicas"]
    for p in points:
        p.pop("ms_per_step", None)
    dom = max(head["kernels"].items(), key=lambda kv: kv[1]["us"])
    sha = kernel_sources_sha()
    workload = f"{cfg.name}_T{args.batch}"
    roofline = {"bound": "hbm", "kernel": dom[0], "achieved": dom[1]["GBps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dom[1]["GBps"] / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic(dom[0], workload, sha),
                "algorithmic_bytes": dom[1]["bytes"], "avg_us": dom[1]["us"]}
    del dl0
    torch.cuda.empty_cache()

    configs = []
    if not args.no_configs:
        shared_draws = {}
        for name, Ts in EXTRA_CONFIGS:
            c = synth.CONFIGS[name]
            key = (c.cid, c.wfmt, c.shared_wfmt, c.I, c.Ish, c.H, c.E)
            if key not in shared_draws:   # layers with the same draws share one upload
                shared_draws.clear()
                torch.cuda.empty_cache()
                log(f"[bench] drawing layer {name}")
                shared_draws[key] = moe.DeviceLayer.from_host(synth.make_layer(c), device=dev)
            d = moe.DeviceLayer(c, shared_draws[key].t)
            pts = time_layer(c, d, Ts, max(5, args.steps // 2), max(2, args.warmup // 2))
            for p in pts:
                p.pop("ms_per_step", None)
            configs.append({"config": name, "H": c.H, "I": c.I, "E": c.E, "k": c.k,
                            "shared": int(c.has_shared), "weights": c.wfmt, "activations": c.afmt,
                            "points": pts})
        shared_draws.clear()
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import layer as OL  # the CPU baseline leg: the oracle as it stands
        x_np = synth.make_x(cfg, args.batch)
        runs, t_tot = 0, 0.0
        while runs < 1 or (t_tot < args.cpu_sample_s and runs < 100):
            t0 = time.perf_counter()
            OL.moe_layer(host, x_np)
            t_tot += time.perf_counter() - t0
            runs += 1
        per = t_tot / runs
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = len(os.sched_getaffinity(0))
        cpu = {"value": round(head["bytes_per_layer"] / per / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle", "us_per_layer": round(per * 1e6, 1),
               "sample": f"{runs} full FP64 oracle layer pass(es) of {cfg.name} at T={args.batch} "
                         f"({head['unique_experts']} touched experts), {t_tot:.1f} s total",
               **cpu_info()}

    out = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} decode MoE layer (H={cfg.H}, E={cfg.E}, top-{cfg.k}, "
                               f"I={cfg.I}, shared={int(cfg.has_shared)}, {cfg.wfmt} weights, "
                               f"{cfg.afmt} activations), T={args.batch}",
                   "global_batch": args.batch, "replicas": R, "parallelism": "single-gpu"},
        "us_per_layer": head["us_per_layer"],
        "frac_peak": head["frac_peak"],
        "copy_GBps": round(copy_gbps, 1),
        "points": points,
        "configs": configs,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_src_sha": sha,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())

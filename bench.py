"""Throughput of the fused top-k MoE layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--M M]

A step is one full pass of the layer (route -> align -> gate/up GEMM with
SiLU-and-mul -> down GEMM -> combine) over one batch of M tokens, with
inputs and weights resident in HBM.  The timed region is K steps of
fused_moe bracketed by device synchronisations.  A second timed region runs
the same kernels through the per-step entry points with HIP events (on the
stream the kernels are launched on) around each kernel, which gives the
per-kernel durations used for the roofline.  The CPU baseline is the CPU
oracle timed on this host on the same batch.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_decode_bf16")
    ap.add_argument("--M", type=int, default=None, help="tokens per batch (default: the largest decode batch)")
    ap.add_argument("--sweep", default="", help="extra batch sizes timed for context, e.g. 1,8,32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device-to-device copy of MB MiB three times (counter calibration)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the code the grouped-GEMM kernels are built from (comments and
    whitespace removed): measured counter traffic of the gate/up launch is only
    reported for the kernel code it was taken on."""
    import hashlib
    import re
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "moe_layer_topk_amd", "csrc", n) for n in ("gemm.hip", "moe_device.h", "moe_launch.h")]
    files.append(os.path.join(ROOT, "include", "moe.h"))
    for f in files:
        with open(f) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, M: int):
    """HBM bytes per gate/up launch from profiles/traffic.json (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    scaled by the same counters on a copy of known size), if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    entry = t.get("gate_up", {}).get(f"{workload}/M={M}")
    return None if entry is None else entry.get("bytes_per_launch")


def layer_bytes(cfg, M, n_active, wbytes, xbytes, obytes):
    """Algorithmic HBM bytes of one layer pass: each active expert's weights
    once, the token rows in and out, routing metadata."""
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.topk
    return n_active * 3 * H * I * wbytes + M * H * (xbytes + obytes) + 4 * M * E + 8 * M * k


def gate_up_bytes(cfg, M, n_active, wbytes, xbytes):
    """Algorithmic bytes of the gate/up GEMM launch: active experts' W1 once,
    x rows in, act rows out (bf16; float32 for the f32 and e4m3 layers)."""
    H, I, k = cfg.H, cfg.I, cfg.topk
    return n_active * 2 * I * H * wbytes + M * H * xbytes + M * k * I * (2 if cfg.dtype == "bf16" else 4)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is not sharded across GPUs",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return

    import moe_layer_topk_amd as moe
    from workloads import CONFIGS, layer_batch, layer_weights

    cfg = CONFIGS[args.workload]
    M = args.M or max(cfg.Ms)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()
    wb = {"bf16": 2, "fp8": 1, "f32": 4}[cfg.dtype]
    ob = 4 if cfg.dtype == "f32" else 2

    t0 = time.time()
    w = layer_weights(cfg, dev)
    torch.cuda.synchronize()
    print(f"[bench] weights for {cfg.name} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def fused(b, ws, out, ids):
        moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, x_scale=b["x_scale"],
                      w1_scale=w["w1_scale"], w2_scale=w["w2_scale"], workspace=ws, out=out, topk_ids=ids)

    def run_case(Mc, steps, warmup, events=True):
        b = layer_batch(cfg, Mc, dev)
        I, H, E, k = cfg.I, cfg.H, cfg.E, cfg.topk
        dt = moe.moe_dtype(w["w1"])
        ws = torch.empty(moe.fused_moe_workspace_size(dt, Mc, E, k, H, I), dtype=torch.uint8, device=dev)
        out = torch.empty((Mc, H), dtype=torch.float32 if cfg.dtype == "f32" else torch.bfloat16, device=dev)
        ids = torch.empty((Mc, k), dtype=torch.int32, device=dev)
        for _ in range(warmup):
            fused(b, ws, out, ids)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            fused(b, ws, out, ids)
        torch.cuda.synchronize()
        fused_s = (time.perf_counter() - t) / steps
        n_active = int(torch.unique(ids).numel())
        res = {"M": Mc, "ms_per_step": fused_s * 1e3, "tokens_per_s": Mc / fused_s, "active_experts": n_active}
        lb = layer_bytes(cfg, Mc, n_active, wb, wb if cfg.dtype != "f32" else 4, ob)
        fl = 6.0 * Mc * k * H * I
        res["layer_hbm_frac"] = lb / fused_s / (HBM_PEAK_GBS * 1e9)
        res["layer_mfma_frac"] = fl / fused_s / (MFMA_PEAK_TFLOPS[cfg.dtype] * 1e12)
        t_roof = max(lb / (HBM_PEAK_GBS * 1e9), fl / (MFMA_PEAK_TFLOPS[cfg.dtype] * 1e12))
        res["roofline_frac"] = t_roof / fused_s
        if not events:
            return res
        # cold cache: a 512 MiB read (twice the 256 MiB Infinity Cache) before each step, outside the
        # event pair around the step, so a small layer's weights are not served from the cache.  A read, not
        # a write: dirty lines left in the cache would be written back during the step and steal bandwidth
        flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        cold = []
        for i in range(min(steps, 20)):
            flush.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fused(b, ws, out, ids)
            e1.record()
            e1.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
        cold.sort()
        res["cold_ms_per_step"] = cold[len(cold) // 2]
        res["cold_p10_p90_ms"] = [cold[len(cold) // 10], cold[(9 * len(cold)) // 10]]
        res["cold_roofline_frac"] = t_roof / (res["cold_ms_per_step"] * 1e-3)
        # the same step captured once in a HIP graph and replayed (launch overhead removed)
        g = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        cap_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap_stream):
            fused(b, ws, out, ids)  # first call on this stream outside capture
            cap_stream.synchronize()
            with torch.cuda.graph(g, stream=cap_stream):
                fused(b, ws, out, ids)
        torch.cuda.current_stream().wait_stream(cap_stream)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = (time.perf_counter() - t) / steps * 1e3
        # per-kernel durations through the per-step entry points, events around each launch
        # the tile height fused_moe picks for this batch
        pe = (Mc * k) // E
        block_m = 128 if pe > (32 if cfg.dtype == "fp8" else 64) else 16
        fp8 = cfg.dtype == "fp8"
        # e4m3: the decode kernel with one token tile quantises the float32 intermediate on load; the
        # tile kernels read codes quantised once (the library's own rule, repeated here for the staged calls)
        avg = Mc * k / E
        q_on_load = fp8 and block_m == 16 and avg + 3.0 * avg ** 0.5 + 1.0 <= 16.0
        codes = fp8 and not q_on_load
        names = ["route", "align", "gate_up"] + (["quant_act"] if codes else []) + ["down", "combine"]
        nk = len(names)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
        amax = torch.empty(1, dtype=torch.float32, device=dev) if fp8 else None
        act = torch.empty((Mc * k, I), dtype=torch.float32 if fp8 else out.dtype, device=dev)
        act_q = torch.empty((Mc * k, I), dtype=torch.float8_e4m3fn, device=dev) if codes else None
        y = torch.empty((Mc * k, H), dtype=out.dtype, device=dev)
        wts = torch.empty((Mc, k), dtype=torch.float32, device=dev)

        def staged(e):
            i = 0
            if e: e[i].record()
            moe.moe_route(b["logits"], k, topk_ids=ids, topk_weights=wts)
            i += 1
            if e: e[i].record()
            al = moe.moe_align(ids, E, block_m)
            i += 1
            if e: e[i].record()
            moe.moe_grouped_gemm(moe.MOE_GEMM_GATE_UP_SILU, b["x"], w["w1"], al, Mc, k, a_scale=b["x_scale"],
                                 w_scale=w["w1_scale"], c=act, c_amax=amax)
            i += 1
            if e: e[i].record()
            if codes:
                moe.moe_quant_act(act, amax, out=act_q)
                i += 1
                if e: e[i].record()
                moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN_E4M3_ACT, act_q, w["w2"], al, Mc, k, a_scale=amax,
                                     w_scale=w["w2_scale"], c=y)
            elif fp8:
                moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, act, w["w2"], al, Mc, k, a_scale=amax,
                                     w_scale=w["w2_scale"], c=y)
            else:
                moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, act, w["w2"], al, Mc, k, c=y)
            i += 1
            if e: e[i].record()
            moe.moe_combine(y, wts, k, out=out)
            i += 1
            if e: e[i].record()

        for _ in range(warmup):
            staged(None)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for s in range(steps):
            staged(ev[s])
        torch.cuda.synchronize()
        res["staged_ms_per_step"] = (time.perf_counter() - t) / steps * 1e3
        ms = np.array([[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(nk)] for s in range(steps)])
        res["kernel_us"] = {n: float(ms[:, i].mean() * 1e3) for i, n in enumerate(names)}
        gu = gate_up_bytes(cfg, Mc, n_active, wb, wb if cfg.dtype != "f32" else 4)
        res["gate_up_bytes"] = gu
        res["gate_up_GBs"] = gu / (res["kernel_us"]["gate_up"] * 1e-6) / 1e9
        res["gate_up_flops"] = 4.0 * Mc * k * H * I
        dn = n_active * H * I * wb + Mc * k * I * (1 if codes else 4 if fp8 else 2) + Mc * k * H * 2
        res["down_GBs"] = dn / (res["kernel_us"]["down"] * 1e-6) / 1e9
        return res

    main_res = run_case(M, args.steps, args.warmup)
    sweep = []
    for m in [int(v) for v in args.sweep.split(",") if v.strip()]:
        if m != M:
            r = run_case(m, args.steps, args.warmup)
            sweep.append({k2: r[k2] for k2 in ("M", "ms_per_step", "tokens_per_s", "roofline_frac", "layer_hbm_frac",
                                                "cold_ms_per_step", "cold_roofline_frac", "graph_ms_per_step",
                                                "kernel_us", "gate_up_GBs", "down_GBs", "active_experts")})

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        b = layer_batch(cfg, M, "cpu")
        wh = {k2: (v.cpu() if v is not None else None) for k2, v in w.items()}
        # the whole batch, repeated until about 10 s of CPU work (at most 8 passes)
        passes, el = 0, 0.0
        while passes == 0 or (el < 10.0 and passes < 8):
            amax = None
            t = time.perf_counter()
            if cfg.dtype == "fp8":
                amax = oracle.act_amax("fp8", b["x"], b["x_scale"], b["logits"], wh["w1"], wh["w1_scale"], cfg.topk)
            oracle.moe_layer(cfg.dtype, b["x"], b["x_scale"], b["logits"], wh["w1"], wh["w1_scale"], wh["w2"],
                             wh["w2_scale"], cfg.topk, act_amax_value=amax)
            el += time.perf_counter() - t
            passes += 1
        cpu = {"value": M * passes / el, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"the full {M}-token batch of the timed workload, {passes} pass(es) ({el:.2f} s)"}

    # roofline of the dominant kernel (gate/up): HBM-bound when its weight
    # bytes take longer at peak bandwidth than its flops at peak MFMA rate
    gu_s = main_res["kernel_us"]["gate_up"] * 1e-6
    mfma_peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    if main_res["gate_up_flops"] / (mfma_peak * 1e12) > main_res["gate_up_bytes"] / (HBM_PEAK_GBS * 1e9):
        achieved = main_res["gate_up_flops"] / gu_s / 1e12
        roof = {"bound": "mfma", "kernel": "gate_up grouped GEMM", "achieved": achieved, "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": achieved / mfma_peak}
    else:
        achieved = main_res["gate_up_bytes"] / gu_s / 1e9
        roof = {"bound": "hbm", "kernel": "gate_up grouped GEMM", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS}
    roof["traffic"] = measured_traffic(cfg.name, M)
    line = {
        "metric": "MoE layer tokens/s; decode HBM GB/s & prefill MFMA TFLOP/s as % of peak",
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3", "f32": "f32"}[cfg.dtype],
        "data": "synthetic (seeded counter-based normals; random-init weights)",
        "config": {"workload": cfg.name, "M": M, "E": cfg.E, "topk": cfg.topk, "hidden": cfg.H,
                   "intermediate": cfg.I, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer": {k2: main_res[k2] for k2 in ("roofline_frac", "layer_hbm_frac", "layer_mfma_frac", "cold_ms_per_step",
                                              "cold_p10_p90_ms", "cold_roofline_frac", "graph_ms_per_step",
                                              "kernel_us", "staged_ms_per_step", "gate_up_GBs", "down_GBs",
                                              "active_experts")},
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

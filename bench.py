"""Throughput of the fused top-k MoE layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME --M M] [--sweep 1,8] [--no-cpu-baseline]
python bench.py --traffic DIR     (CPU only: rocprofv3 counter CSVs -> profiles/traffic.json)

A step is one full pass of the layer (route -> align -> gate/up GEMM with
SiLU-and-mul -> down GEMM -> combine) over one batch of M tokens, with
inputs and weights resident in HBM.  The timed region is K steps of
fused_moe bracketed by device synchronisations.  A second timed region runs
the same kernels through the per-step entry points with HIP events (on
torch's current stream, the stream the library launches on) around each
kernel, which gives the per-kernel durations used for the rooflines.  The
CPU baseline is the CPU oracle timed on this host on (a stated sample of)
the same batch.

With no workload given, the line's `value` is the Mixtral-shaped bf16 decode
layer at 64 tokens, and `workloads` adds the two other halves of the metric:
the 4096-token Zipf-routed prefill layer (MFMA roofline) and the 64-expert
e4m3 layer at 32 tokens (HBM roofline); `sweep` adds the decode layer at 1, 8
and 32 tokens for context; `streaming` times the bf16 and int4-weight
decode layers with host-resident experts behind a 4-slot GPU cache.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3, "w4a16": 2500.0}  # dense MFMA peaks (W4A16: bf16)
# bytes per weight (W4A16: a 4-bit code and 1/128 of a float32 scale) and per activation
W_BYTES = {"bf16": 2, "fp8": 1, "f32": 4, "w4a16": 0.5 + 4 / 128}
X_BYTES = {"bf16": 2, "fp8": 1, "f32": 4, "w4a16": 2}
DTYPE_NAME = {"bf16": "bf16", "fp8": "fp8_e4m3", "f32": "f32", "w4a16": "int4_weights_bf16_act"}
METRIC = "MoE layer tokens/s; decode HBM GB/s & prefill MFMA TFLOP/s as % of peak"

MAIN = ("mixtral_decode_bf16", 64)
EXTRA = (("mixtral_prefill_bf16", 4096), ("fp8_e4m3", 32), ("mixtral_decode_w4a16", 64))
MAIN_SWEEP = (1, 8, 32)
# expert streaming: the layers above behind a 4-slot GPU cache, 32 one-token
# decode steps with Zipf(1.1)-skewed routing
STREAM_CAPACITY, STREAM_STEPS = 4, 32
STREAMED = ("mixtral_decode_bf16", "mixtral_decode_w4a16")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="time only this workload (default: the three-line set)")
    ap.add_argument("--M", type=int, default=None, help="tokens per batch for --workload (default: its largest)")
    ap.add_argument("--sweep", default=None, help="extra batch sizes of the main workload, e.g. 1,8,32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream", action="store_true", help="with --workload: also time it behind the expert cache")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device-to-device copy of MB MiB three times (counter calibration)")
    ap.add_argument("--traffic", default=None, metavar="DIR",
                    help="reduce rocprofv3 FETCH_SIZE/WRITE_SIZE passes under DIR into profiles/traffic.json")
    return ap.parse_args()


# ------------------------------------------------------------ algorithmic work

def layer_bytes(cfg, M, n_active, wbytes, xbytes, obytes):
    """Algorithmic HBM bytes of one layer pass: each active expert's weights
    once, the token rows in and out, routing metadata."""
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.topk
    return n_active * 3 * H * I * wbytes + M * H * (xbytes + obytes) + 4 * M * E + 8 * M * k


def act_elem_bytes(cfg):
    """Bytes per element of the stored intermediate: bf16 for the bf16 and
    W4A16 layers, float32 for the f32 and e4m3 layers."""
    return 2 if cfg.dtype in ("bf16", "w4a16") else 4


def gate_up_bytes(cfg, M, n_active, wbytes, xbytes):
    """Algorithmic bytes of the gate/up GEMM launch: active experts' W1 once,
    x rows in, act rows out."""
    H, I, k = cfg.H, cfg.I, cfg.topk
    return n_active * 2 * I * H * wbytes + M * H * xbytes + M * k * I * act_elem_bytes(cfg)


def down_bytes(cfg, M, n_active, wbytes, act_bytes):
    """Algorithmic bytes of the down GEMM launch: active experts' W2 once, act
    rows in (as the kernel reads them), y rows (bf16) out."""
    H, I, k = cfg.H, cfg.I, cfg.topk
    return n_active * H * I * wbytes + M * k * I * act_bytes + M * k * H * 2


def fused_block_m(cfg, M):
    """The tile height fused_moe picks for a batch (the library's rule)."""
    if cfg.dtype in ("f32", "w4a16"):
        return 16
    pe = (M * cfg.topk) // cfg.E
    if cfg.dtype == "fp8":
        return 128 if pe > 32 else (64 if M >= 2 else 16)
    return 128 if pe > 48 else (64 if pe > 24 else 16)


def fp8_quantises_on_load(cfg, M):
    """e4m3: the decode kernel with one 16-row token tile quantises the float32
    intermediate as it loads it; the tile kernels read codes quantised once
    (the library's rule, repeated here for the per-step calls)."""
    avg = M * cfg.topk / cfg.E
    return cfg.dtype == "fp8" and fused_block_m(cfg, M) == 16 and avg + 3.0 * avg ** 0.5 + 1.0 <= 16.0


# ----------------------------------------------------------- counter traffic

def kernel_source_hash() -> str:
    """Hash of the code the grouped-GEMM kernels are built from (comments and
    whitespace removed): measured counter traffic of a launch is only
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


def measured_traffic(workload: str, M: int, kind: str = "gate_up"):
    """HBM bytes per launch from profiles/traffic.json (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by the
    same counters on a copy of known size), if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    entry = t.get(kind, {}).get(f"{workload}/M={M}")
    return None if entry is None else entry.get("bytes_per_launch")


def _pmc_rows(path, pred):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 --pmc CSV."""
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if pred(r["Kernel_Name"]):
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def reduce_traffic(d: str) -> dict:
    """profiles/traffic.json from rocprofv3 counter passes under d.

    Expected layout (one pass per counter, as the profile summaries list):
      d/pmc_FETCH_SIZE_copy/*counter_collection.csv, d/pmc_WRITE_SIZE_copy/...:  bench.py --copy-probe 1024
      d/pmc_FETCH_SIZE_<workload>_<M>/..., d/pmc_WRITE_SIZE_<workload>_<M>/...: bench.py --workload W --M M
    The copy passes calibrate the counters (KiB counted per KiB moved by a
    plain 1 GiB copy); each grouped-GEMM dispatch's FETCH_SIZE and WRITE_SIZE
    (KiB) are scaled by them and averaged over the dispatches of one kernel.
    The kernel is the gate/up GEMM when its first template argument is 0
    (MOE_GEMM_GATE_UP_SILU), the down GEMM otherwise.
    """
    import glob
    from workloads import CONFIGS

    def one(sub):
        hits = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not hits:
            raise FileNotFoundError(f"no counter CSV under {os.path.join(d, sub)}")
        return hits[0]

    moved_kib = 1024.0 * 1024.0
    fc = [v for vs in _pmc_rows(one("pmc_FETCH_SIZE_copy"), lambda n: "copy" in n.lower()).values() for v in vs]
    wc = [v for vs in _pmc_rows(one("pmc_WRITE_SIZE_copy"), lambda n: "copy" in n.lower()).values() for v in vs]
    fetch_scale = moved_kib / (sum(fc) / len(fc))
    write_scale = moved_kib / (sum(wc) / len(wc))
    out = {"source_hash": kernel_source_hash(), "fetch_scale": fetch_scale, "write_scale": write_scale,
           "gate_up": {}, "down": {}}
    for sub in sorted(os.listdir(d)):
        if (not sub.startswith("pmc_FETCH_SIZE_") or sub.endswith("_copy")
                or not os.path.isdir(os.path.join(d, sub))):
            continue
        rest = sub[len("pmc_FETCH_SIZE_"):]
        name, M = rest.rsplit("_", 1)
        cfg, M = CONFIGS[name], int(M)
        f = _pmc_rows(one(sub), lambda n: "moe::gemm" in n)
        w = _pmc_rows(one("pmc_WRITE_SIZE_" + rest), lambda n: "moe::gemm" in n)
        for kern, fv in f.items():
            kind = "gate_up" if "kernel<0," in kern else "down"
            fk, wk = sum(fv) / len(fv), sum(w[kern]) / len(w[kern])
            out[kind][f"{name}/M={M}"] = {"kernel": kern.split("(")[0], "launches": len(fv),
                                          "fetch_kib": fk, "write_kib": wk,
                                          "bytes_per_launch": (fk * fetch_scale + wk * write_scale) * 1024.0}
    return out


# ------------------------------------------------------------------ GPU work

def measure(moe, torch, np, cfg, w, M, steps, warmup, dev, events=True):
    """Time one workload: back-to-back fused steps, cold-cache and graph-replay
    steps, and per-kernel HIP-event times through the per-step entry points."""
    from workloads import layer_batch
    b = layer_batch(cfg, M, dev)
    I, H, E, k = cfg.I, cfg.H, cfg.E, cfg.topk
    wb, xb = W_BYTES[cfg.dtype], X_BYTES[cfg.dtype]
    ob = 4 if cfg.dtype == "f32" else 2
    dt = moe.moe_dtype(w["w1"])
    ws = torch.empty(moe.fused_moe_workspace_size(dt, M, E, k, H, I), dtype=torch.uint8, device=dev)
    out = torch.empty((M, H), dtype=torch.float32 if cfg.dtype == "f32" else torch.bfloat16, device=dev)
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)

    def fused():
        moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], k, x_scale=b["x_scale"], w1_scale=w["w1_scale"],
                      w2_scale=w["w2_scale"], workspace=ws, out=out, topk_ids=ids)

    for _ in range(warmup):
        fused()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        fused()
    torch.cuda.synchronize()
    fused_s = (time.perf_counter() - t) / steps
    n_active = int(torch.unique(ids).numel())
    res = {"M": M, "ms_per_step": fused_s * 1e3, "tokens_per_s": M / fused_s, "active_experts": n_active}
    lb = layer_bytes(cfg, M, n_active, wb, xb, ob)
    fl = 6.0 * M * k * H * I
    peak_f = MFMA_PEAK_TFLOPS[cfg.dtype] * 1e12
    res["layer_bytes"], res["layer_flops"] = lb, fl
    res["layer_hbm_frac"] = lb / fused_s / (HBM_PEAK_GBS * 1e9)
    res["layer_mfma_frac"] = fl / fused_s / peak_f
    t_roof = max(lb / (HBM_PEAK_GBS * 1e9), fl / peak_f)
    res["roofline_frac"] = t_roof / fused_s
    if not events:
        return res
    # cold cache: a 512 MiB read (twice the 256 MiB Infinity Cache) before each step, outside the event
    # pair around the step, so a small layer's weights are not served from the cache.  A read, not a
    # write: dirty lines left in the cache would be written back during the step and steal bandwidth
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(min(steps, 20)):
        flush.max()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fused()
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
        fused()  # first call on this stream outside capture
        cap_stream.synchronize()
        with torch.cuda.graph(g, stream=cap_stream):
            fused()
    torch.cuda.current_stream().wait_stream(cap_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    res["graph_ms_per_step"] = (time.perf_counter() - t) / steps * 1e3
    del g

    # the layer from the hidden states: router scores x . Wg^T on the GPU first
    # (fused_moe_router; router weights float32 [E, H] ~ N(0, 0.02))
    from workloads.gen import S_WG, normal_f32
    wg = normal_f32(0, S_WG, (E, H), 0.02, dev)
    lg = torch.empty((M, E), dtype=torch.float32, device=dev)

    def routed():
        moe.fused_moe_router(b["x"], wg, w["w1"], w["w2"], k, x_scale=b["x_scale"], w1_scale=w["w1_scale"],
                             w2_scale=w["w2_scale"], workspace=ws, out=out, logits=lg, topk_ids=ids)

    for _ in range(warmup):
        routed()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        routed()
    torch.cuda.synchronize()
    rs = (time.perf_counter() - t) / steps
    res["router_ms_per_step"] = rs * 1e3
    # its own routing activates its own experts: roofline on those
    ra = int(torch.unique(ids).numel())
    res["router_active_experts"] = ra
    res["router_roofline_frac"] = max(layer_bytes(cfg, M, ra, wb, xb, ob) / (HBM_PEAK_GBS * 1e9), fl / peak_f) / rs
    del wg, lg

    # per-kernel durations through the per-step entry points (the kernels fused_moe launches, except
    # that the per-step down GEMM does not split K), HIP events around each launch on torch's stream
    block_m = fused_block_m(cfg, M)
    fp8 = cfg.dtype == "fp8"
    codes = fp8 and not fp8_quantises_on_load(cfg, M)
    names = ["route", "align", "gate_up"] + (["quant_act"] if codes else []) + ["down", "combine"]
    nk = len(names)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
    amax = torch.empty(1, dtype=torch.float32, device=dev) if fp8 else None
    act = torch.empty((M * k, I), dtype=torch.float32 if fp8 else out.dtype, device=dev)
    act_q = torch.empty((M * k, I), dtype=torch.float8_e4m3fn, device=dev) if codes else None
    y = torch.empty((M * k, H), dtype=out.dtype, device=dev)
    wts = torch.empty((M, k), dtype=torch.float32, device=dev)

    def staged(e):
        rec = (lambda i: e[i].record()) if e else (lambda i: None)
        i = 0
        rec(i)
        moe.moe_route(b["logits"], k, topk_ids=ids, topk_weights=wts)
        i += 1
        rec(i)
        al = moe.moe_align(ids, E, block_m)
        i += 1
        rec(i)
        moe.moe_grouped_gemm(moe.MOE_GEMM_GATE_UP_SILU, b["x"], w["w1"], al, M, k, a_scale=b["x_scale"],
                             w_scale=w["w1_scale"], c=act, c_amax=amax)
        i += 1
        rec(i)
        if codes:
            moe.moe_quant_act(act, amax, out=act_q)
            i += 1
            rec(i)
            moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN_E4M3_ACT, act_q, w["w2"], al, M, k, a_scale=amax,
                                 w_scale=w["w2_scale"], c=y)
        else:
            moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, act, w["w2"], al, M, k, a_scale=amax, w_scale=w["w2_scale"], c=y)
        i += 1
        rec(i)
        moe.moe_combine(y, wts, k, out=out)
        i += 1
        rec(i)

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
    res["gate_up_bytes"] = gate_up_bytes(cfg, M, n_active, wb, xb)
    res["gate_up_flops"] = 4.0 * M * k * H * I
    res["gate_up_GBs"] = res["gate_up_bytes"] / (res["kernel_us"]["gate_up"] * 1e-6) / 1e9
    res["gate_up_TFLOPs"] = res["gate_up_flops"] / (res["kernel_us"]["gate_up"] * 1e-6) / 1e12
    dn = down_bytes(cfg, M, n_active, wb, 1 if codes else act_elem_bytes(cfg))
    res["down_GBs"] = dn / (res["kernel_us"]["down"] * 1e-6) / 1e9
    res["down_TFLOPs"] = 2.0 * M * k * H * I / (res["kernel_us"]["down"] * 1e-6) / 1e12
    return res


def roofline(cfg, res):
    """Roofline of the dominant kernel (the gate/up GEMM): MFMA-bound when its
    flops at the dense peak take longer than its bytes at the HBM peak."""
    gu_s = res["kernel_us"]["gate_up"] * 1e-6
    peak_f = MFMA_PEAK_TFLOPS[cfg.dtype]
    if res["gate_up_flops"] / (peak_f * 1e12) > res["gate_up_bytes"] / (HBM_PEAK_GBS * 1e9):
        achieved = res["gate_up_flops"] / gu_s / 1e12
        roof = {"bound": "mfma", "kernel": "gate_up grouped GEMM", "achieved": achieved, "peak": peak_f,
                "unit": "TFLOP/s", "frac": achieved / peak_f}
    else:
        achieved = res["gate_up_bytes"] / gu_s / 1e9
        roof = {"bound": "hbm", "kernel": "gate_up grouped GEMM", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS}
    roof["traffic"] = measured_traffic(cfg.name, res["M"])
    return roof


def cpu_baseline(cfg, w, M, budget_s):
    """The CPU oracle on this host over (a sample of) the same batch, as
    tokens/s: the first n tokens, n grown (up to the whole batch) until one
    pass takes about a third of budget_s, then passes repeated until about
    budget_s of CPU work (at most 8)."""
    import oracle
    from workloads import layer_batch
    b = layer_batch(cfg, M, "cpu")
    wh = {k: (v.cpu() if v is not None else None) for k, v in w.items()}

    def one_pass(n):
        t = time.perf_counter()
        amax = None
        if cfg.dtype == "fp8":  # the batch statistic the layer needs, over the whole batch
            amax = oracle.act_amax("fp8", b["x"], b["x_scale"], b["logits"], wh["w1"], wh["w1_scale"], cfg.topk)
        oracle.moe_layer(cfg.dtype, b["x"], b["x_scale"], b["logits"], wh["w1"], wh["w1_scale"], wh["w2"],
                         wh["w2_scale"], cfg.topk, tokens=list(range(n)), act_amax_value=amax)
        return time.perf_counter() - t

    n = max(1, min(M, 8))
    el = one_pass(n)
    while el < budget_s / 3 and n < M:
        n = min(M, max(n + 1, int(n * budget_s / 3 / max(el, 1e-3))))
        el = one_pass(n)
    total, passes = el, 1
    while total < budget_s and passes < 8:
        total += one_pass(n)
        passes += 1
    what = "the whole batch" if n == M else f"tokens 0..{n - 1} of the {M}-token batch"
    if cfg.dtype == "fp8":
        what += " (each pass also computes the batch-wide intermediate amax over all its tokens)"
    return {"value": n * passes / total, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{cfg.name}: {what}, {passes} pass(es), {total:.2f} s"}


def measure_streaming(moe, torch, cfg, w, dev, capacity=STREAM_CAPACITY, nsteps=STREAM_STEPS, warm=6):
    """Expert streaming (host-resident experts, `capacity` GPU slots): one-token
    decode steps over Zipf-routed batches, timed end to end (each step waits
    for its routing on the host), once with copies on demand only and once
    with the next step's routed experts prefetched while the current step
    computes (the routed set known ahead: a perfect predictor, the upper
    bound of prediction).  The resident layer runs the same batches."""
    from dataclasses import replace

    from workloads import layer_batch
    zc = replace(cfg, router="zipf")
    n = warm + nsteps
    batches = [layer_batch(zc, 1, dev, seed=1000 + t) for t in range(n)]
    routed = [moe.moe_route(b["logits"], zc.topk)[0].cpu().ravel().tolist() for b in batches]
    host = {k: (None if v is None else v.cpu().pin_memory()) for k, v in w.items()}  # pinned once, used in place

    def timed(step):
        for t in range(warm):
            step(t)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(warm, n):
            step(t)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / nsteps

    res = {"workload": zc.name, "M": 1, "capacity": capacity, "E": zc.E, "topk": zc.topk, "steps": nsteps,
           "routing": f"Zipf({zc.zipf_s})", "dtype": DTYPE_NAME[zc.dtype]}
    res["resident_ms_per_step"] = timed(lambda t: moe.fused_moe(batches[t]["x"], batches[t]["logits"], w["w1"],
                                                                w["w2"], zc.topk, w1_scale=w["w1_scale"],
                                                                w2_scale=w["w2_scale"]))
    for name, pre in (("on_demand", False), ("prefetch_next", True)):
        cache = moe.ExpertCache(host["w1"], host["w2"], capacity, w1_scale=host["w1_scale"],
                                w2_scale=host["w2_scale"], device=dev)
        marks = {}

        def step(t):
            if t == warm:
                marks["s0"] = cache.stats()
            cache(batches[t]["x"], batches[t]["logits"], zc.topk)
            if pre and t + 1 < n:
                cache.prefetch(routed[t + 1])

        ms = timed(step)
        s1 = cache.stats()
        d = {k: s1[k] - marks["s0"][k] for k in s1}
        cache.close()
        res[name] = {"ms_per_step": ms, "tokens_per_s": 1e3 / ms, "misses_per_step": d["misses"] / nsteps,
                     "prefetched_per_step": d["prefetched"] / nsteps,
                     "hit_rate": d["hits"] / max(d["hits"] + d["misses"], 1),
                     "h2d_GBs": d["h2d_bytes"] / (ms * 1e-3 * nsteps) / 1e9}
    # the host link: one expert's bytes from pinned memory, timed with events
    eb = sum(v[0].numel() * v.element_size() for k, v in host.items() if v is not None)
    src = torch.empty(eb, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(eb, dtype=torch.uint8, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src, non_blocking=True)
    a.record()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    res["expert_MB"] = eb / 1e6
    res["host_link_GBs"] = 3 * eb / (a.elapsed_time(b) * 1e-3) / 1e9
    for name in ("on_demand", "prefetch_next"):
        res[name]["link_frac"] = res[name]["h2d_GBs"] / res["host_link_GBs"]
    return res


def line_entry(cfg, res, cpu):
    keys = ("ms_per_step", "tokens_per_s", "roofline_frac", "layer_hbm_frac", "layer_mfma_frac", "cold_ms_per_step",
            "cold_p10_p90_ms", "cold_roofline_frac", "graph_ms_per_step", "router_ms_per_step",
            "router_active_experts", "router_roofline_frac", "staged_ms_per_step",
            "kernel_us",
            "gate_up_GBs", "gate_up_TFLOPs", "down_GBs", "down_TFLOPs", "active_experts")
    e = {"workload": cfg.name, "M": res["M"], "dtype": DTYPE_NAME[cfg.dtype],
         "E": cfg.E, "topk": cfg.topk, "hidden": cfg.H, "intermediate": cfg.I}
    e.update({k2: res[k2] for k2 in keys if k2 in res})
    e["roofline"] = roofline(cfg, res)
    if cpu is not None:
        e["cpu_baseline"] = cpu
    return e


def main():
    args = parse()
    if args.traffic:
        t = reduce_traffic(args.traffic)
        path = os.path.join(ROOT, "profiles", "traffic.json")
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps({"traffic": path, "entries": {k: sorted(t[k]) for k in ("gate_up", "down")}}))
        return
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
    from workloads import CONFIGS, layer_weights

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()

    if args.workload:
        main_cfg = CONFIGS[args.workload]
        main_M = args.M or max(main_cfg.Ms)
        extra = []
        sweep_ms = [int(v) for v in (args.sweep or "").split(",") if v.strip()]
    else:
        main_cfg, main_M = CONFIGS[MAIN[0]], MAIN[1]
        extra = [(CONFIGS[n], m) for n, m in EXTRA]
        sweep_ms = [int(v) for v in args.sweep.split(",") if v.strip()] if args.sweep is not None else list(MAIN_SWEEP)

    weights = {}

    def weights_for(cfg):
        key = (cfg.E, cfg.H, cfg.I, cfg.dtype)  # the prefill and decode Mixtral layers share their weights
        if cfg.dtype == "w4a16":
            weights.clear()  # free the bf16/e4m3 layers first
        if key not in weights:
            t0 = time.time()
            weights[key] = layer_weights(cfg, dev)
            torch.cuda.synchronize()
            print(f"[bench] weights for {cfg.name} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        return weights[key]

    w = weights_for(main_cfg)
    main_res = measure(moe, torch, np, main_cfg, w, main_M, args.steps, args.warmup, dev)
    print(f"[bench] {main_cfg.name} M={main_M}: {main_res['ms_per_step']:.4f} ms", file=sys.stderr, flush=True)
    sweep = []
    for m in sweep_ms:
        if m != main_M:
            r = measure(moe, torch, np, main_cfg, w, m, args.steps, args.warmup, dev)
            sweep.append(line_entry(main_cfg, r, None))
            print(f"[bench] {main_cfg.name} M={m}: {r['ms_per_step']:.4f} ms", file=sys.stderr, flush=True)
    streaming = []

    def stream(cfg, wx):
        if args.workload and not args.stream:
            return
        if cfg.name in STREAMED:
            r = measure_streaming(moe, torch, cfg, wx, dev)
            streaming.append(r)
            print(f"[bench] {cfg.name} streamed through {r['capacity']} slots: on demand "
                  f"{r['on_demand']['ms_per_step']:.3f} ms, prefetch {r['prefetch_next']['ms_per_step']:.3f} ms, "
                  f"resident {r['resident_ms_per_step']:.3f} ms per step", file=sys.stderr, flush=True)

    stream(main_cfg, w)
    lines = []
    for cfg, m in extra:
        wx = weights_for(cfg)
        r = measure(moe, torch, np, cfg, wx, m, args.steps, args.warmup, dev)
        print(f"[bench] {cfg.name} M={m}: {r['ms_per_step']:.4f} ms", file=sys.stderr, flush=True)
        cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, wx, m, 4.0)
        lines.append(line_entry(cfg, r, cpu))
        stream(cfg, wx)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(main_cfg, w, main_M, 10.0)
        print(f"[bench] cpu baseline: {cpu['sample']}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[main_cfg.dtype],
        "data": "synthetic (seeded counter-based normals; random-init weights)",
        "config": {"workload": main_cfg.name, "M": main_M, "E": main_cfg.E, "topk": main_cfg.topk,
                   "hidden": main_cfg.H, "intermediate": main_cfg.I, "parallelism": "single GPU"},
        "roofline": roofline(main_cfg, main_res),
        "cpu_baseline": cpu,
        "layer": {k2: main_res[k2] for k2 in ("roofline_frac", "layer_hbm_frac", "layer_mfma_frac", "cold_ms_per_step",
                                              "cold_p10_p90_ms", "cold_roofline_frac", "graph_ms_per_step",
                                              "router_ms_per_step", "router_active_experts",
                                              "router_roofline_frac",
                                              "kernel_us", "staged_ms_per_step", "gate_up_GBs", "down_GBs",
                                              "active_experts")},
        "workloads": lines,
        "sweep": sweep,
        "streaming": streaming,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

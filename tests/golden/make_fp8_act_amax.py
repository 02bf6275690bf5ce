"""Writes fp8_act_amax.json: the oracle's batch-wide max |intermediate| of the
per-tensor-scaled e4m3 workload (64 experts, top-8, hidden 4096,
intermediate 8192) for each of its batch sizes, seed 0.

The statistic needs every (token, slot) pair's gate/up projection, which is
too slow to recompute inside a test at the 512-token size; this script runs
the oracle once (minutes on a few cores) and stores the result together with
fingerprints of the seeded inputs it used.  Only oracle/ and the input
generator are called.

usage: python tests/golden/make_fp8_act_amax.py
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import torch  # noqa: E402

import oracle  # noqa: E402
from workloads import CONFIGS, layer_batch, layer_weights  # noqa: E402


def main():
    cfg = CONFIGS["fp8_e4m3"]
    t0 = time.time()
    w = layer_weights(cfg, "cpu")
    print(f"weights generated in {time.time() - t0:.0f}s", flush=True)
    out = {"workload": cfg.name, "seed": 0, "amax": {}, "fingerprint": {}}
    Mmax = max(cfg.Ms)
    b = layer_batch(cfg, Mmax, "cpu")
    t0 = time.time()
    per_tok = oracle.act_amax_per_token("fp8", b["x"], b["x_scale"], b["logits"], w["w1"], w["w1_scale"], cfg.topk)
    print(f"oracle per-token amax in {time.time() - t0:.0f}s ({oracle.num_threads()} threads)", flush=True)
    for M in cfg.Ms:
        # the x scale is per batch, so each batch size is its own quantised input
        bm = layer_batch(cfg, M, "cpu")
        if M == Mmax:
            am = float(per_tok.max())
        else:
            am = float(oracle.act_amax_per_token("fp8", bm["x"], bm["x_scale"], bm["logits"], w["w1"], w["w1_scale"],
                                                 cfg.topk).max())
        out["amax"][str(M)] = am
        out["fingerprint"][str(M)] = {"x_scale": float(bm["x_scale"][0]),
                                      "x_code_sum": int(bm["x"].view(torch.uint8).long().sum())}
    out["fingerprint"]["w1_scale"] = [float(v) for v in w["w1_scale"][:8]]
    out["fingerprint"]["w2_scale"] = [float(v) for v in w["w2_scale"][:8]]
    with open(os.path.join(HERE, "fp8_act_amax.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out["amax"]))


if __name__ == "__main__":
    main()

"""GPU parity of the weight-only int4 layer (W4A16: 4-bit weight codes with a
float32 scale per 128 k of a row, bf16 activations) against the CPU oracle,
which decodes the same codes and scales to float64.  Bar: the bf16 one,
max|gpu - oracle| <= 1e-2 * max|oracle| (the oracle applies the same
quantised weights)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, layer_batch, layer_weights
from workloads.gen import S_ACT, normal_bf16

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_layer_topk_amd as moe
    moe.lib()
    return torch.device("cuda:0")


def rel_err(gpu, ref):
    g = gpu.float().cpu().numpy().astype(np.float64)
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))


# E, k, H, I, M: one and two 16-row token tiles, many passes (many rows per
# expert), K of one to sixteen steps, 1/2/4 row groups per workgroup
GEMM = [(8, 2, 512, 256, 40), (16, 4, 256, 512, 8), (64, 8, 1024, 768, 3), (4, 2, 256, 256, 200),
        (8, 2, 4096, 1024, 1), (128, 8, 2048, 768, 16)]


@pytest.mark.parametrize("E,k,H,I,M", GEMM)
def test_w4a16_grouped_gemm(dev, E, k, H, I, M):
    import moe_layer_topk_amd as moe
    print(f"w4a16 gemm E={E} k={k} H={H} I={I} M={M}", flush=True)
    cfg = replace(CONFIGS["finegrained_w4a16"], E=E, topk=k, H=H, I=I)
    w = layer_weights(cfg, "cpu", seed=1)
    b = layer_batch(cfg, M, "cpu", seed=1)
    rid, _ = oracle.route(b["logits"], k)
    al = moe.moe_align(torch.from_numpy(rid).to(dev), E, 16)
    pairs = np.arange(M * k)
    act, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_GATE_UP_SILU, b["x"].to(dev), w["w1"].to(dev), al, M, k,
                                  w_scale=w["w1_scale"].to(dev))
    torch.cuda.synchronize()
    ref = oracle.pairs_gate_up("w4a16", b["x"], None, rid, w["w1"], w["w1_scale"], pairs)
    err = rel_err(act, ref)
    print(f"  gate_up rel err {err:.2e}", flush=True)
    assert err <= TOL
    a_in = normal_bf16(seed=5, stream=S_ACT, shape=(M * k, I), std=0.1, device=dev)
    y, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, a_in, w["w2"].to(dev), al, M, k, w_scale=w["w2_scale"].to(dev))
    torch.cuda.synchronize()
    yref = oracle.pairs_down("w4a16", a_in.cpu(), rid, w["w2"], w["w2_scale"], pairs)
    err = rel_err(y, yref)
    print(f"  down rel err {err:.2e}", flush=True)
    assert err <= TOL


LAYERS = [("mixtral_decode_w4a16", {}, 1), ("mixtral_decode_w4a16", {}, 8), ("mixtral_decode_w4a16", {}, 64),
          ("finegrained_w4a16", {}, 1), ("finegrained_w4a16", {}, 16), ("finegrained_w4a16", {"E": 4, "topk": 2}, 300)]


@pytest.mark.parametrize("name,shape,M", LAYERS)
def test_w4a16_fused_layer(dev, name, shape, M):
    import moe_layer_topk_amd as moe
    cfg = replace(CONFIGS[name], **shape)
    print(f"w4a16 fused {cfg.name} E={cfg.E} k={cfg.topk} M={M}", flush=True)
    w = layer_weights(cfg, dev)
    b = layer_batch(cfg, M, dev)
    ids = torch.empty((M, cfg.topk), dtype=torch.int32, device=dev)
    out = moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, w1_scale=w["w1_scale"],
                        w2_scale=w["w2_scale"], topk_ids=ids)
    torch.cuda.synchronize()
    rid, _ = oracle.route(b["logits"].cpu(), cfg.topk)
    assert np.array_equal(ids.cpu().numpy(), rid)
    tok = np.arange(M) if M <= 64 else np.arange(0, M, 11)
    wh = {k2: v.cpu() for k2, v in w.items()}
    ref = oracle.moe_layer("w4a16", b["x"].cpu(), None, b["logits"].cpu(), wh["w1"], wh["w1_scale"], wh["w2"],
                           wh["w2_scale"], cfg.topk, tokens=tok)
    err = rel_err(out.cpu()[torch.from_numpy(tok)], ref)
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL
    # deterministic: the same call gives the same bits
    out2 = moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, w1_scale=w["w1_scale"],
                         w2_scale=w["w2_scale"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2)

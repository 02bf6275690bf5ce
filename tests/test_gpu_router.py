"""GPU router scores and the layer from hidden states (router on the GPU)
against the CPU oracle.

Scores: within 1e-5 * max|oracle| of the oracle's float64 x . Wg^T (float32
accumulation over H).  Routing is decided on the GPU's own scores: ids must
equal the oracle's routing of those same float32 scores bit for bit, weights
within 1e-6; the layer output within the dtype's bar of the oracle's layer
on those scores.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, layer_batch, layer_weights
from workloads.gen import S_WG, normal_f32

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 3e-2}


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


ROUTER_SHAPES = [("bf16", 1, 8, 4096), ("bf16", 300, 8, 4096), ("bf16", 33, 128, 2048), ("f32", 16, 8, 256),
                 ("fp8", 70, 64, 4096), ("bf16", 5, 256, 128),
                 # 8 tokens x 4 experts per wavefront, E not a multiple of 4, H an odd multiple of 128
                 ("bf16", 2048, 130, 384), ("f32", 9, 3, 384)]


@pytest.mark.parametrize("dtype,M,E,H", ROUTER_SHAPES)
def test_router_logits(dev, dtype, M, E, H):
    import moe_layer_topk_amd as moe
    print(f"router {dtype} M={M} E={E} H={H}", flush=True)
    cfg = replace(CONFIGS["fp8_e4m3" if dtype == "fp8" else "tiny_f32"], dtype=dtype, E=E, H=H, router="normal")
    b = layer_batch(cfg, M, "cpu", seed=2)
    wg = normal_f32(4, S_WG, (E, H), 0.02, "cpu")
    xs = b["x_scale"].to(dev) if b["x_scale"] is not None else None
    lg = moe.moe_router_logits(b["x"].to(dev), wg.to(dev), x_scale=xs)
    torch.cuda.synchronize()
    ref = oracle.router_logits(dtype, b["x"], b["x_scale"], wg)
    assert rel_err(lg, ref) <= 1e-5


# (base workload, shape overrides, M): one-launch router + route + align for
# up to 16 tokens with at most 64 K router weights, two launches otherwise;
# one bf16 / e4m3 token: the router launch, then GEMMs that route the token
# themselves
LAYERS = [("mixtral_decode_bf16", {}, 1), ("mixtral_decode_bf16", {}, 16), ("mixtral_decode_bf16", {}, 64),
          ("finegrained_bf16", {"H": 512}, 4), ("finegrained_bf16", {}, 3), ("tiny_f32", {}, 16),
          ("fp8_e4m3", {"E": 16, "I": 1024}, 8), ("mixtral_prefill_bf16", {"H": 1024, "I": 1024}, 700),
          ("finegrained_bf16", {}, 1), ("fp8_e4m3", {"E": 16, "I": 1024}, 1)]


@pytest.mark.parametrize("name,shape,M", LAYERS)
def test_fused_moe_router(dev, name, shape, M):
    import moe_layer_topk_amd as moe
    cfg = replace(CONFIGS[name], **shape)
    print(f"fused router {cfg.name} E={cfg.E} H={cfg.H} I={cfg.I} M={M}", flush=True)
    w = layer_weights(cfg, dev)
    b = layer_batch(cfg, M, dev, seed=1)
    wg = normal_f32(3, S_WG, (cfg.E, cfg.H), 0.02 if cfg.dtype != "f32" else 0.1, dev)
    ids = torch.empty((M, cfg.topk), dtype=torch.int32, device=dev)
    wts = torch.empty((M, cfg.topk), dtype=torch.float32, device=dev)
    out, lg = moe.fused_moe_router(b["x"], wg, w["w1"], w["w2"], cfg.topk, x_scale=b["x_scale"],
                                   w1_scale=w["w1_scale"], w2_scale=w["w2_scale"], topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    bh = {k: (v.cpu() if v is not None else None) for k, v in b.items()}
    wh = {k: (v.cpu() if v is not None else None) for k, v in w.items()}
    # scores against the oracle's float64 ones, and the same bits as the
    # stand-alone router call (one definition whichever launch computes them)
    assert rel_err(lg, oracle.router_logits(cfg.dtype, bh["x"], bh["x_scale"], wg.cpu())) <= 1e-5
    assert torch.equal(lg, moe.moe_router_logits(b["x"], wg, x_scale=b["x_scale"]))
    # routing on the GPU's scores, bit-exact
    glg = lg.cpu()
    rid, rw = oracle.route(glg, cfg.topk)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(wts.cpu().numpy() - rw).max() <= 1e-6
    # the layer on those scores
    tok = np.arange(M) if M <= 64 else np.arange(0, M, 9)
    ref = oracle.moe_layer(cfg.dtype, bh["x"], bh["x_scale"], glg, wh["w1"], wh["w1_scale"], wh["w2"],
                           wh["w2_scale"], cfg.topk, tokens=tok)
    err = rel_err(out.cpu()[torch.from_numpy(tok)], ref)
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL[cfg.dtype]
    # the same layer through fused_moe on those scores gives the same output
    out2 = moe.fused_moe(b["x"], lg, w["w1"], w["w2"], cfg.topk, x_scale=b["x_scale"], w1_scale=w["w1_scale"],
                         w2_scale=w["w2_scale"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2)

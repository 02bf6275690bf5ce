"""One-token layers whose decode GEMMs route the token themselves (bf16,
e4m3 and W4A16, no route / align launch): routing ids bit-exact against the
oracle on crafted logits (integer ties, +0/-0 ties, topk = E, E = 256 with
topk = 16), weights within 1e-6 with and without renormalisation, and the
layer output against the oracle (e4m3: the intermediate's amax passed from
the gate/up to the down launch as partial maxima, checked through the
output at the e4m3 bar)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, counter_normal, layer_batch, layer_weights

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "w4a16": 1e-2, "fp8": 3e-2}
BASE = {"bf16": "finegrained_bf16", "w4a16": "finegrained_w4a16", "fp8": "fp8_e4m3"}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import moe_layer_topk_amd as moe
    moe.lib()
    return torch.device("cuda:0")


def crafted_logits(kind, E, seed):
    g = counter_normal(seed, 2, E, "cpu").float()
    if kind == "ties":  # integer values: many equal logits
        return torch.round(g * 2.0)
    if kind == "zeros":  # +0 and -0 tie; the rest below them
        lg = torch.full((E,), -0.0)
        lg[::3] = 0.0
        lg[1::5] = -1.0
        return lg
    return g


CASES = [
    ("bf16", 16, 4, True, "ties"),
    ("bf16", 8, 8, True, "normal"),        # topk = E
    ("bf16", 16, 2, False, "normal"),      # softmax over all E at the selected experts
    ("bf16", 64, 8, True, "zeros"),
    ("bf16", 256, 16, True, "normal"),     # the largest E and topk the ABI takes
    ("w4a16", 16, 4, True, "ties"),
    ("w4a16", 32, 2, False, "normal"),
    ("fp8", 64, 8, True, "normal"),        # the 64-expert e4m3 layer's routing
    ("fp8", 16, 4, True, "ties"),
    ("fp8", 32, 2, False, "zeros"),
]


@pytest.mark.parametrize("dtype,E,k,renorm,kind", CASES)
def test_one_token_self_routing(dev, dtype, E, k, renorm, kind):
    import moe_layer_topk_amd as moe
    cfg = replace(CONFIGS[BASE[dtype]], E=E, topk=k, H=256, I=256)
    print(f"self-route {dtype} E={E} k={k} renorm={renorm} {kind}", flush=True)
    w = layer_weights(cfg, "cpu", seed=3)
    b = layer_batch(cfg, 1, "cpu", seed=3)
    lg = crafted_logits(kind, E, seed=7 + E).reshape(1, E).contiguous()
    wd = {n: (v.to(dev) if v is not None else None) for n, v in w.items()}
    x = b["x"].to(dev)
    ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, k), dtype=torch.float32, device=dev)
    xs = b["x_scale"].to(dev) if b.get("x_scale") is not None else None
    out = moe.fused_moe(x, lg.to(dev), wd["w1"], wd["w2"], k, x_scale=xs, w1_scale=wd["w1_scale"],
                        w2_scale=wd["w2_scale"], renormalize=renorm, topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    rid, rw = oracle.route(lg, k, renormalize=renorm)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(wts.cpu().numpy() - rw).max() <= 1e-6
    ref = oracle.moe_layer(dtype, b["x"], b.get("x_scale"), lg, w["w1"], w["w1_scale"], w["w2"], w["w2_scale"], k,
                           renormalize=renorm)
    ref = torch.from_numpy(np.asarray(ref, dtype=np.float64))
    err = float((out.cpu().double() - ref).abs().max() / ref.abs().max().clamp_min(1e-30))
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]

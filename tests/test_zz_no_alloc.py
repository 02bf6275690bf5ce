"""fused_moe_noalloc (static device scratch, no workspace argument) against
fused_moe with a caller workspace: the same kernels over the same layout, so
the outputs are equal bit for bit.  Two calls in a row, the second with a
smaller batch, so the second runs over the first one's leftovers."""
from dataclasses import replace

import pytest
import torch

from workloads import CONFIGS, layer_batch, layer_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_layer_topk_amd as moe
    moe.lib()
    return torch.device("cuda:0")


CASES = [("mixtral_decode_bf16", 64, 5, {}),
         ("fp8_e4m3", 32, 3, {"E": 16, "H": 1024, "I": 2048}),
         # one e4m3 token: self-routed, its amax partials in the static scratch
         ("fp8_e4m3", 4, 1, {"E": 16, "H": 1024, "I": 2048}),
         ("finegrained_bf16", 40, 1, {}),
         ("tiny_f32", 16, 7, {})]


@pytest.mark.parametrize("name,M1,M2,shape", CASES)
def test_noalloc_matches_fused(dev, name, M1, M2, shape):
    import moe_layer_topk_amd as moe
    cfg = replace(CONFIGS[name], **shape)
    print(f"noalloc {cfg.name} E={cfg.E} H={cfg.H} I={cfg.I} M={M1} then M={M2}", flush=True)
    w = layer_weights(cfg, dev)
    for M in (M1, M2):
        b = layer_batch(cfg, M, dev, seed=M)
        kw = dict(x_scale=b["x_scale"], w1_scale=w["w1_scale"], w2_scale=w["w2_scale"])
        ids_a = torch.empty((M, cfg.topk), dtype=torch.int32, device=dev)
        ids_b = torch.empty_like(ids_a)
        wts_a = torch.empty((M, cfg.topk), dtype=torch.float32, device=dev)
        wts_b = torch.empty_like(wts_a)
        ref = moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, topk_ids=ids_a, topk_weights=wts_a,
                            **kw)
        got = moe.fused_moe_noalloc(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, topk_ids=ids_b,
                                    topk_weights=wts_b, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"M={M}"
        assert torch.equal(ids_a, ids_b) and torch.equal(wts_a, wts_b)


def test_noalloc_rejects_sizes_beyond_scratch(dev):
    """The 4096-token Mixtral-shaped layer needs far more than the scratch:
    rejected with MOE_ERR_SCRATCH before any HIP call (so the buffer passed
    for every tensor is never read)."""
    import moe_layer_topk_amd as moe
    cfg = CONFIGS["mixtral_prefill_bf16"]
    buf = torch.empty(64, dtype=torch.float32, device=dev)
    p = moe._p(buf)
    st = moe.lib().fused_moe_noalloc(moe.MOE_BF16, p, None, p, p, None, p, None, 4096, cfg.E, cfg.topk, cfg.H, cfg.I,
                                     1, p, None, None, moe._stream(buf))
    assert st == moe.MOE_ERR_SCRATCH

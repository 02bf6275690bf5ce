"""The seeded input generator: determinism, prefix property, distributions."""
import numpy as np
import torch

from workloads import CONFIGS, counter_normal, layer_batch, layer_weights
from workloads.gen import _lowbias32, _lowbias32_py, zipf_log_prior


def test_hash_tensor_matches_python_ints():
    xs = [0, 1, 2, 0xFFFFFFFF, 0x12345678, 0x80000000, 0x7FEB352D]
    got = _lowbias32(torch.tensor(xs, dtype=torch.int64)).tolist()
    assert got == [_lowbias32_py(v) for v in xs]


def test_counter_normal_deterministic_and_prefix():
    a = counter_normal(0, 1, 5000, "cpu")
    b = counter_normal(0, 1, 5000, "cpu")
    assert torch.equal(a, b)
    c = counter_normal(0, 1, 1000, "cpu", offset=2000)
    assert torch.equal(a[2000:3000], c)
    assert not torch.equal(a, counter_normal(1, 1, 5000, "cpu"))
    assert not torch.equal(a, counter_normal(0, 2, 5000, "cpu"))


def test_counter_normal_moments():
    z = counter_normal(0, 3, 1 << 20, "cpu").numpy()
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert abs((z ** 4).mean() - 3) < 0.05  # Gaussian kurtosis
    assert abs((np.abs(z) < 1).mean() - 0.6827) < 3e-3


def test_batch_prefix_property():
    cfg = CONFIGS["mixtral_decode_bf16"]
    b64 = layer_batch(cfg, 64, "cpu")
    b8 = layer_batch(cfg, 8, "cpu")
    assert torch.equal(b64["x"][:8], b8["x"]) and torch.equal(b64["logits"][:8], b8["logits"])
    assert b64["x"].dtype == torch.bfloat16 and b64["logits"].dtype == torch.float32


def test_fp8_storage_and_scales():
    from dataclasses import replace
    cfg = replace(CONFIGS["fp8_e4m3"], E=2, H=128, I=128)
    w = layer_weights(cfg, "cpu")
    assert w["w1"].dtype == torch.float8_e4m3fn and w["w1_scale"].shape == (2,)
    # the largest code of each expert matrix is +-448 (scale = amax/448)
    assert float(w["w1"][0].float().abs().max()) == 448.0
    sd = (w["w1"][0].float() * w["w1_scale"][0]).std().item()
    assert abs(sd - 0.02) < 2e-3
    b = layer_batch(cfg, 32, "cpu")
    assert b["x"].dtype == torch.float8_e4m3fn and float(b["x"].float().abs().max()) == 448.0


def test_zipf_prior_skews_expert_zero():
    lp = zipf_log_prior(8, 1.1)
    assert abs(sum(np.exp(lp)) - 1) < 1e-12 and all(np.diff(lp) < 0)
    cfg = CONFIGS["mixtral_prefill_bf16"]
    lg = layer_batch(cfg, 512, "cpu")["logits"]
    counts = np.bincount(lg.argmax(1).numpy(), minlength=8)
    assert counts[0] == counts.max() and counts[0] > 2 * counts[7]


def test_tiny_router_logits_are_x_wg():
    cfg = CONFIGS["tiny_f32"]
    b = layer_batch(cfg, 16, "cpu")
    assert b["logits"].shape == (16, 8) and b["x"].dtype == torch.float32
    assert torch.equal(layer_batch(cfg, 16, "cpu")["logits"], b["logits"])


def test_whole_tensor_weights_equal_per_expert_draws():
    """layer_weights draws all experts in one fill; expert e must hold the same
    bytes as its own draw at offset e * (elements per expert matrix)."""
    from dataclasses import replace
    from workloads.gen import S_W1, S_W2, normal_bf16, normal_f32
    for name, mk in (("finegrained_bf16", normal_bf16), ("tiny_f32", normal_f32)):
        cfg = replace(CONFIGS[name], E=5, H=128, I=256)
        w = layer_weights(cfg, "cpu")
        sub = layer_weights(cfg, "cpu", experts=[1, 4])
        n1, n2 = 2 * cfg.I * cfg.H, cfg.H * cfg.I
        for e in range(cfg.E):
            assert torch.equal(w["w1"][e], mk(0, S_W1, (2 * cfg.I, cfg.H), cfg.weight_std, "cpu", offset=e * n1))
            assert torch.equal(w["w2"][e], mk(0, S_W2, (cfg.H, cfg.I), cfg.weight_std, "cpu", offset=e * n2))
        assert torch.equal(sub["w1"][4], w["w1"][4]) and not sub["w1"][0].any()

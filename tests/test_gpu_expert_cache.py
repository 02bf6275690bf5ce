"""Expert streaming (FusedMoE vs MegaMoE post, sections 4.1-4.3) on the GPU:
host-resident experts, a pool of GPU slots with least-recently-used
replacement, prefetch on a copy stream, and the fused layer over the slots.

The layer over the cache must give the same bits as fused_moe with every
expert resident (the slots are a renaming of the experts, and each routed
pair's products do not depend on where its expert's weights sit), and the
routed ids must be the oracle's.  One batch per sequence is also checked
against the CPU oracle directly.  Routing follows a Zipf(1.1) prior over the
experts, the skew the layer's prefill workload uses."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, layer_batch, layer_weights

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2, "w4a16": 1e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_layer_topk_amd as moe
    moe.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def small(dtype, E=32, topk=2, H=256, I=256):
    base = {"bf16": "finegrained_bf16", "fp8": "fp8_e4m3", "w4a16": "finegrained_w4a16", "f32": "tiny_f32"}[dtype]
    return replace(CONFIGS[base], E=E, topk=topk, H=H, I=I, router="zipf")


def host_parts(w):
    return {k: (None if v is None else v.cpu()) for k, v in w.items()}


def make_cache(moe, wh, capacity, dev):
    return moe.ExpertCache(wh["w1"], wh["w2"], capacity, w1_scale=wh["w1_scale"], w2_scale=wh["w2_scale"],
                           device=dev)


def fused(moe, cfg, w, b, ids=None):
    return moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, x_scale=b["x_scale"],
                         w1_scale=w["w1_scale"], w2_scale=w["w2_scale"], topk_ids=ids)


class LruModel:
    """The replacement rule written out on the host: a request marks its
    resident experts used; each missing expert takes an empty slot (lowest
    index first), else the slot used longest ago that the request does not
    keep (lowest index among equals)."""

    def __init__(self, capacity):
        self.expert = [-1] * capacity
        self.stamp = [0] * capacity
        self.clock = 0

    def request(self, experts):
        self.clock += 1
        keep, misses = set(), 0
        for e in experts:
            if e in self.expert:
                s = self.expert.index(e)
                keep.add(s)
                self.stamp[s] = self.clock
        for e in experts:
            if e in self.expert:
                continue
            free = [s for s in range(len(self.expert)) if s not in keep]
            empty = [s for s in free if self.expert[s] < 0]
            s = empty[0] if empty else min(free, key=lambda t: (self.stamp[t], t))
            self.expert[s], self.stamp[s] = e, self.clock
            keep.add(s)
            misses += 1
        return len(experts) - misses, misses


def expert_bytes(cfg):
    H, I = cfg.H, cfg.I
    if cfg.dtype == "w4a16":
        return 3 * H * I // 2 + (H // 128) * 2 * I * 4 + (I // 128) * H * 4
    eb = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.dtype]
    return 3 * H * I * eb + (8 if cfg.dtype == "fp8" else 0)


def oracle_check(cfg, b, wh, out):
    bh = {k: (v.cpu() if v is not None else None) for k, v in b.items()}
    amax = None
    if cfg.dtype == "fp8":
        amax = oracle.act_amax("fp8", bh["x"], bh["x_scale"], bh["logits"], wh["w1"], wh["w1_scale"], cfg.topk)
    ref = oracle.moe_layer(cfg.dtype, bh["x"], bh["x_scale"], bh["logits"], wh["w1"], wh["w1_scale"], wh["w2"],
                           wh["w2_scale"], cfg.topk, act_amax_value=amax)
    g = out.float().cpu().numpy().astype(np.float64)
    err = float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))
    say(f"  oracle rel err {err:.2e}")
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "w4a16", "f32"])
def test_cache_sequence_matches_resident_layer(dev, dtype):
    """A sequence of Zipf-routed batches (1 to 4 tokens, top-2 over 32
    experts) through an 8-slot cache, half of it on a second stream: every
    output bit-identical to fused_moe over all experts, ids equal to the
    oracle's, hits and misses as the LRU rule predicts."""
    import moe_layer_topk_amd as moe
    cfg = small(dtype)
    say(f"cache sequence {dtype} E={cfg.E} C=8")
    w = layer_weights(cfg, dev)
    wh = host_parts(w)
    cache = make_cache(moe, wh, 8, dev)
    model = LruModel(8)
    side = torch.cuda.Stream(dev)
    hits = misses = 0
    for t in range(16):
        M = 1 + t % 4
        b = layer_batch(cfg, M, dev, seed=100 + t)
        rid, _ = oracle.route(b["logits"].cpu(), cfg.topk)
        h, m = model.request(sorted(set(rid.ravel().tolist())))
        hits, misses = hits + h, misses + m
        ids = torch.empty((M, cfg.topk), dtype=torch.int32, device=dev)
        ref = fused(moe, cfg, w, b)
        if t >= 8:
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                out = cache(b["x"], b["logits"], cfg.topk, x_scale=b["x_scale"], topk_ids=ids)
            torch.cuda.current_stream(dev).wait_stream(side)
        else:
            out = cache(b["x"], b["logits"], cfg.topk, x_scale=b["x_scale"], topk_ids=ids)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), rid), t
        assert torch.equal(out, ref), (t, (out.float() - ref.float()).abs().max().item())
    st = cache.stats()
    say(f"  stats {st}, model hits {hits} misses {misses}")
    assert (st["hits"], st["misses"], st["prefetched"]) == (hits, misses, 0)
    assert st["h2d_bytes"] == misses * expert_bytes(cfg)
    oracle_check(cfg, b, wh, out)
    cache.close()


def test_cache_prefetch_removes_misses(dev):
    """Prefetching each batch's routed experts before the call leaves the call
    nothing to copy: misses stay at zero, the copies count as prefetched."""
    import moe_layer_topk_amd as moe
    cfg = small("bf16", E=64, topk=4)
    w = layer_weights(cfg, dev)
    wh = host_parts(w)
    cache = make_cache(moe, wh, 16, dev)
    copies = 0
    model = LruModel(16)
    for t in range(10):
        b = layer_batch(cfg, 3, dev, seed=200 + t)
        rid, _ = oracle.route(b["logits"].cpu(), cfg.topk)
        need = sorted(set(rid.ravel().tolist()))
        cache.prefetch(rid.ravel().tolist())
        copies += model.request(need)[1]
        assert model.request(need) == (len(need), 0)
        out = cache(b["x"], b["logits"], cfg.topk)
        assert torch.equal(out, fused(moe, cfg, w, b)), t
    torch.cuda.synchronize()
    st = cache.stats()
    say(f"  prefetch stats {st}")
    assert st["misses"] == 0 and st["prefetched"] == copies and st["hits"] > 0
    cache.close()


def test_cache_copies_wait_for_readers(dev):
    """Two slots and top-2 routing: every prefetch evicts the experts the call
    just queued is still reading.  The copies must wait for that call, so every
    output still equals the resident layer's."""
    import moe_layer_topk_amd as moe
    cfg = small("bf16", E=8, topk=2, H=2048, I=2048)
    w = layer_weights(cfg, dev)
    wh = host_parts(w)
    cache = make_cache(moe, wh, 2, dev)
    batches = [layer_batch(cfg, 1, dev, seed=300 + t) for t in range(12)]
    routed = [oracle.route(b["logits"].cpu(), cfg.topk)[0].ravel().tolist() for b in batches]
    outs = []
    for t, b in enumerate(batches):
        outs.append(cache(b["x"], b["logits"], cfg.topk))
        if t + 1 < len(batches):
            cache.prefetch(routed[t + 1])  # queued while call t may still run
    torch.cuda.synchronize()
    for t, b in enumerate(batches):
        assert torch.equal(outs[t], fused(moe, cfg, w, b)), t
    st = cache.stats()
    say(f"  reader-wait stats {st}")
    assert st["misses"] == 2  # only the first call finds its experts missing
    cache.close()


def test_cache_capacity_exceeded(dev):
    """A batch routed to more distinct experts than slots is an error
    (MOE_ERR_UNSUPPORTED, after routing); the cache keeps working."""
    import moe_layer_topk_amd as moe
    cfg = small("bf16", E=32, topk=4)
    w = layer_weights(cfg, dev)
    wh = host_parts(w)
    cache = make_cache(moe, wh, 4, dev)
    b = layer_batch(cfg, 16, dev, seed=400)
    assert len(set(oracle.route(b["logits"].cpu(), 4)[0].ravel().tolist())) > 4
    with pytest.raises(moe.MoeError) as ei:
        cache(b["x"], b["logits"], cfg.topk)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError):
        cache(b["x"], b["logits"], 5)  # topk above the slots
    with pytest.raises(moe.MoeError):
        cache.prefetch(range(5))
    b1 = layer_batch(cfg, 1, dev, seed=401)
    assert torch.equal(cache(b1["x"], b1["logits"], cfg.topk), fused(moe, cfg, w, b1))
    assert cache.stats()["misses"] == 4
    cache.close()


@pytest.mark.parametrize("dtype", ["bf16", "w4a16"])
def test_cache_mixtral_decode_steps(dev, dtype):
    """The page's setting at full size: a Mixtral-8x7B-shaped layer (8 experts,
    top-2, H 4096, I 14336) behind a 4-slot cache, 8 single-token decode
    steps with Zipf routing, bit-identical to the resident layer."""
    import moe_layer_topk_amd as moe
    name = {"bf16": "mixtral_decode_bf16", "w4a16": "mixtral_decode_w4a16"}[dtype]
    cfg = replace(CONFIGS[name], router="zipf")
    say(f"cache mixtral {dtype}")
    w = layer_weights(cfg, dev)
    cache = make_cache(moe, host_parts(w), 4, dev)
    for t in range(8):
        b = layer_batch(cfg, 1, dev, seed=500 + t)
        ids = torch.empty((1, 2), dtype=torch.int32, device=dev)
        out = cache(b["x"], b["logits"], cfg.topk, topk_ids=ids)
        ref = fused(moe, cfg, w, b)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), oracle.route(b["logits"].cpu(), 2)[0])
        assert torch.equal(out, ref), t
    say(f"  stats {cache.stats()}")
    cache.close()
    del w
    torch.cuda.empty_cache()


def test_cache_prefill_batch(dev):
    """A 1024-token batch (128 pairs per expert: the tile kernels) through a
    cache that holds every expert: the same bits as the resident layer; and a
    batch routed to 8 of 16 experts through an 8-slot cache, against the
    oracle (the slot count changes the tile-height choice, so bits may
    differ from the resident layer's)."""
    import moe_layer_topk_amd as moe
    cfg = small("bf16", E=16, topk=2, H=512, I=512)
    w = layer_weights(cfg, dev)
    wh = host_parts(w)
    cache = make_cache(moe, wh, 16, dev)
    b = layer_batch(cfg, 1024, dev, seed=600)
    out = cache(b["x"], b["logits"], cfg.topk)
    assert torch.equal(out, fused(moe, cfg, w, b))
    cache.close()
    cache = make_cache(moe, wh, 8, dev)
    b = layer_batch(cfg, 512, dev, seed=601)
    b["logits"][:, 8:] -= 100.0  # route among experts 0..7 only
    ids = torch.empty((512, 2), dtype=torch.int32, device=dev)
    out = cache(b["x"], b["logits"], cfg.topk, topk_ids=ids)
    torch.cuda.synchronize()
    assert int(ids.max()) < 8
    bh = {k: (v.cpu() if v is not None else None) for k, v in b.items()}
    tok = np.arange(0, 512, 17)
    ref = oracle.moe_layer("bf16", bh["x"], None, bh["logits"], wh["w1"], None, wh["w2"], None, cfg.topk, tokens=tok)
    g = out.float().cpu().numpy().astype(np.float64)[tok]
    assert np.abs(g - ref).max() <= TOL["bf16"] * np.abs(ref).max()
    assert cache.stats()["misses"] == 8
    cache.close()

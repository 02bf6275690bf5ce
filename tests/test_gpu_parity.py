"""GPU parity: every C-ABI step and the fused layer against the CPU oracle.

Bars: routing ids and the alignment are bit-exact; routing weights within
1e-6; float32 outputs within 1e-5*max|oracle|, bfloat16 within
1e-2*max|oracle|, fp8 within 3e-2*max|oracle| (the oracle applies the same
quantised weights).
"""
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, counter_normal, layer_batch, layer_weights
from workloads.gen import S_ACT, S_WTS, S_Y, counter_uniform_int, normal_bf16, normal_f32

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 3e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_layer_topk_amd as moe
    moe.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def rel_err(gpu, ref):
    g = gpu.float().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) else gpu
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))


# ----------------------------------------------------------------- route

ROUTE_SHAPES = [(16, 8, 2), (64, 8, 2), (4096, 8, 2), (2048, 128, 8), (512, 64, 8), (1, 8, 2), (7, 5, 5),
                (33, 256, 16), (100, 3, 1)]


@pytest.mark.parametrize("M,E,k", ROUTE_SHAPES)
@pytest.mark.parametrize("renorm", [1, 0])
def test_route(dev, M, E, k, renorm):
    import moe_layer_topk_amd as moe
    say(f"route M={M} E={E} k={k} renorm={renorm}")
    lg = counter_normal(M + E, 2, M * E, dev).reshape(M, E).float()
    ids, w = moe.moe_route(lg, k, renormalize=bool(renorm))
    torch.cuda.synchronize()
    rid, rw = oracle.route(lg.cpu(), k, renormalize=bool(renorm))
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6


def test_route_ties(dev):
    import moe_layer_topk_amd as moe
    say("route ties")
    E, k = 64, 8
    lg = torch.zeros((6, E))
    lg[1] = torch.round(counter_normal(3, 2, E, "cpu") * 2).float()  # integer ties
    lg[2] = -0.0
    lg[2, ::3] = 0.0
    lg[3] = 1.0
    lg[3, 40:] = 2.0
    lg[4, :] = torch.arange(E).float() % 4  # ties far apart
    lg[5, :] = -1e30
    ids, w = moe.moe_route(lg.to(dev), k)
    torch.cuda.synchronize()
    rid, rw = oracle.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    assert ids.cpu()[0].tolist() == list(range(k))


# ----------------------------------------------------------------- align

def _check_align(got, ref):
    for key in ("expert_counts", "expert_offsets", "sorted_ids", "tile_expert", "num_active"):
        g = got[key].cpu().numpy()[:len(ref[key])]
        assert np.array_equal(g, ref[key]), key
    na = len(ref["active_experts"])
    assert np.array_equal(got["active_experts"].cpu().numpy()[:na], ref["active_experts"])


ALIGN_CASES = [("uniform", 64, 8, 2), ("uniform", 4096, 8, 2), ("zipf", 4096, 8, 2), ("uniform", 2048, 128, 8),
               ("uniform", 512, 64, 8), ("uniform", 1, 8, 2), ("one_expert", 300, 8, 1), ("two_experts", 96, 128, 2),
               ("divisible", 128, 8, 2), ("uniform", 16, 128, 8), ("uniform", 5000, 256, 4),
               # 72000 pairs: more 1024-pair units than workgroups, so workgroups scatter two units and the
               # last ones only write sentinels and tile entries
               ("uniform", 9000, 128, 8), ("zipf", 40000, 8, 2)]


@pytest.mark.parametrize("kind,M,E,k", ALIGN_CASES)
@pytest.mark.parametrize("bm", [1, 16, 32, 64, 128, 256])
def test_align(dev, kind, M, E, k, bm):
    import moe_layer_topk_amd as moe
    say(f"align {kind} M={M} E={E} k={k} bm={bm}")
    if kind == "one_expert":
        ids = np.full((M, k), E - 3, np.int32)
    elif kind == "two_experts":
        ids = np.stack([np.full(M, 5), np.full(M, 77)], 1).astype(np.int32)
    elif kind == "divisible":  # every count a multiple of 16 (and of 64 / 128 for some)
        ids = (np.arange(M * k) // 32 % E).astype(np.int32).reshape(M, k)
    else:
        lg = counter_normal(M, 2, M * E, "cpu").reshape(M, E).float()
        if kind == "zipf":
            lg = lg + torch.log(torch.arange(1, E + 1).double() ** -1.1).float()
        ids, _ = oracle.route(lg, k)
    got = moe.moe_align(torch.from_numpy(ids).to(dev), E, bm)
    torch.cuda.synchronize()
    _check_align(got, oracle.align(ids, E, bm))


# ------------------------------------------------------------ grouped gemm

def _gemm_case(dtype, E, k, H, I, M, seed=0):
    cfg = replace(CONFIGS["tiny_f32"], E=E, topk=k, H=H, I=I, dtype=dtype, router="normal")
    w = layer_weights(cfg, "cpu", seed=seed)
    b = layer_batch(cfg, M, "cpu", seed=seed)
    return cfg, w, b


GEMM_CASES = [("bf16", 8, 2, 256, 256, 40), ("bf16", 16, 4, 512, 384, 100), ("bf16", 4, 2, 128, 128, 300),
              ("fp8", 8, 2, 256, 256, 40), ("fp8", 16, 4, 512, 512, 100), ("f32", 8, 2, 256, 512, 16),
              ("bf16", 128, 8, 256, 128, 16), ("bf16", 8, 2, 1024, 256, 1)]


@pytest.mark.parametrize("dtype,E,k,H,I,M", GEMM_CASES)
@pytest.mark.parametrize("path", ["decode", "prefill", "prefill128"])
def test_grouped_gemm(dev, monkeypatch, dtype, E, k, H, I, M, path):
    import moe_layer_topk_amd as moe
    say(f"gemm {dtype} E={E} k={k} H={H} I={I} M={M} path={path}")
    monkeypatch.setenv("MOE_GEMM_PATH", path.replace("128", ""))
    cfg, w, b = _gemm_case(dtype, E, k, H, I, M)
    rid, _ = oracle.route(b["logits"], k)
    ids = torch.from_numpy(rid).to(dev)
    bm = {"prefill": 64, "prefill128": 128}.get(path, 16)
    al = moe.moe_align(ids, E, bm)
    P = M * k
    pairs = np.arange(P)
    sc = lambda t: None if t is None else t.to(dev)  # noqa: E731
    # GATE_UP
    act, amax = moe.moe_grouped_gemm(moe.MOE_GEMM_GATE_UP_SILU, b["x"].to(dev), w["w1"].to(dev), al, M, k,
                                     a_scale=sc(b["x_scale"]), w_scale=sc(w["w1_scale"]))
    torch.cuda.synchronize()
    ref = oracle.pairs_gate_up(dtype, b["x"], b["x_scale"], rid, w["w1"], w["w1_scale"], pairs)
    err = rel_err(act, ref)
    say(f"  gate_up rel err {err:.2e}")
    assert err <= TOL[dtype]
    if dtype == "fp8":
        assert abs(float(amax) - float(act.float().abs().max())) == 0.0
    # DOWN on a generated intermediate (bf16 rows; float32 for the f32 and e4m3 paths)
    if dtype in ("f32", "fp8"):
        a_in = normal_f32(seed=5, stream=S_ACT, shape=(P, I), std=0.1, device=dev)
    else:
        a_in = normal_bf16(seed=5, stream=S_ACT, shape=(P, I), std=0.1, device=dev)
    a_amax = a_in.abs().max().reshape(1) if dtype == "fp8" else None
    y, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, a_in, w["w2"].to(dev), al, M, k, a_scale=a_amax,
                                w_scale=sc(w["w2_scale"]))
    torch.cuda.synchronize()
    yref = oracle.pairs_down(dtype, a_in.cpu(), rid, w["w2"], w["w2_scale"], pairs,
                             act_amax_value=float(a_amax) if a_amax is not None else 0.0)
    err = rel_err(y, yref)
    say(f"  down rel err {err:.2e}")
    assert err <= TOL[dtype]
    if dtype == "fp8":
        # the codes the down call forms on load, as a tensor: bit-exact against
        # the oracle's encoder of the float32 quotient; the down GEMM over them
        # within the bar of the quantise-on-load one
        q = moe.moe_quant_act(a_in, a_amax)
        s32 = np.float32(float(a_amax)) / np.float32(448.0)
        v = a_in.cpu().numpy().ravel() / s32
        want = np.array([oracle.e4m3_encode(float(t)) for t in v], np.uint8)
        assert np.array_equal(q.view(torch.uint8).cpu().numpy().ravel(), want)
        y8, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN_E4M3_ACT, q, w["w2"].to(dev), al, M, k, a_scale=a_amax,
                                     w_scale=sc(w["w2_scale"]))
        torch.cuda.synchronize()
        err8 = rel_err(y8, yref)
        say(f"  down (e4m3 act) rel err {err8:.2e}")
        assert err8 <= TOL[dtype]


def test_fp8_down_quantise_on_load_equals_codes(dev, monkeypatch):
    """One token tile per expert: the decode ring kernel quantises the float32
    intermediate on load; fed the codes of moe_quant_act instead, the same
    kernel computes the same products in the same order (bitwise equal)."""
    import moe_layer_topk_amd as moe
    monkeypatch.setenv("MOE_GEMM_PATH", "decode")
    for (E, k, H, I, M) in [(16, 2, 512, 768, 8), (64, 8, 1024, 2048, 3), (8, 2, 256, 4096, 1)]:
        say(f"fp8 down on-load vs codes E={E} k={k} H={H} I={I} M={M}")
        cfg, w, b = _gemm_case("fp8", E, k, H, I, M, seed=3)
        rid, _ = oracle.route(b["logits"], k)
        al = moe.moe_align(torch.from_numpy(rid).to(dev), E, 16)
        a_in = normal_f32(seed=7, stream=S_ACT, shape=(M * k, I), std=0.3, device=dev)
        amax = a_in.abs().max().reshape(1)
        y, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, a_in, w["w2"].to(dev), al, M, k, a_scale=amax,
                                    w_scale=w["w2_scale"].to(dev))
        q = moe.moe_quant_act(a_in, amax)
        y8, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN_E4M3_ACT, q, w["w2"].to(dev), al, M, k, a_scale=amax,
                                     w_scale=w["w2_scale"].to(dev))
        torch.cuda.synchronize()
        assert torch.equal(y, y8)
        yref = oracle.pairs_down("fp8", a_in.cpu(), rid, w["w2"], w["w2_scale"], np.arange(M * k),
                                 act_amax_value=float(amax))
        assert rel_err(y, yref) <= TOL["fp8"]


def test_register_kernel_four_groups_two_token_tiles(dev, monkeypatch):
    """The register-operand decode kernel at four row groups and two token
    tiles (128 KiB of LDS for its cross-wavefront reduction): the down GEMM of
    a float32 layer with a short K (I = 512), and a standalone e4m3 DOWN over a
    float32 intermediate (K = 2048), both at 12 pairs per expert on average."""
    import moe_layer_topk_amd as moe
    cfg = replace(CONFIGS["tiny_f32"], E=64, topk=8, H=4096, I=512, router="normal")
    say("register kernel: f32 layer E=64 k=8 H=4096 I=512 M=96")
    check_layer(cfg, 96, dev, tokens=range(0, 96, 7))
    _W.clear()
    monkeypatch.setenv("MOE_GEMM_PATH", "decode")
    E, k, H, I, M = 64, 8, 4096, 2048, 96
    say(f"register kernel: fp8 DOWN on float32 act E={E} k={k} H={H} I={I} M={M}")
    cfg = replace(CONFIGS["fp8_e4m3"], E=E, topk=k, H=H, I=I, router="normal")
    w = layer_weights(cfg, dev, seed=4)  # drawn on the GPU: 64 experts are slow to draw on the host
    b = layer_batch(cfg, M, "cpu", seed=4)
    rid, _ = oracle.route(b["logits"], k)
    al = moe.moe_align(torch.from_numpy(rid).to(dev), E, 16)
    a_in = normal_f32(seed=9, stream=S_ACT, shape=(M * k, I), std=0.3, device=dev)
    amax = a_in.abs().max().reshape(1)
    y, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, a_in, w["w2"], al, M, k, a_scale=amax, w_scale=w["w2_scale"])
    torch.cuda.synchronize()
    pairs = np.arange(0, M * k, 13)
    yref = oracle.pairs_down("fp8", a_in.cpu(), rid, w["w2"].cpu(), w["w2_scale"].cpu(), pairs,
                             act_amax_value=float(amax))
    err = rel_err(y.cpu()[torch.from_numpy(pairs)], yref)
    say(f"  down rel err {err:.2e} over {len(pairs)} pairs")
    assert err <= TOL["fp8"]


def test_quant_act_codes_exhaustive_near_ties(dev):
    """moe_quant_act against the oracle's encoder on values placed at, just
    below and just above every e4m3 rounding midpoint (and the saturation
    edge) for a few scales: the float32 quotient and its rounding decide
    every code exactly as an IEEE division does."""
    import moe_layer_topk_amd as moe
    grid = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    mids = (grid[1:] + grid[:-1]) / 2
    say("quant_act near ties")
    for amax in (1.0, 24.875, 3.3e-3, 448.0 * 7.5):
        s32 = np.float32(amax) / np.float32(448.0)
        base = np.concatenate([grid, mids, [448.0, 460.0, 463.9, 464.0]]).astype(np.float64) * float(s32)
        vals = np.concatenate([base, np.nextafter(base, 0), np.nextafter(base, 1e30)])
        vals = np.concatenate([vals, -vals]).astype(np.float32)
        vals = np.clip(vals, -amax, amax).astype(np.float32)
        vals = np.concatenate([vals, np.zeros((-len(vals)) % 16, np.float32)])
        act = torch.from_numpy(vals).to(dev)
        q = moe.moe_quant_act(act, torch.tensor([amax], dtype=torch.float32, device=dev))
        torch.cuda.synchronize()
        want = np.array([oracle.e4m3_encode(float(np.float32(t) / s32)) for t in vals], np.uint8)
        got = q.view(torch.uint8).cpu().numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(float(vals[i]), int(got[i]), int(want[i])) for i in bad[:5]]


# ----------------------------------------------------------------- combine

@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,k,H", [(1, 2, 4096), (64, 2, 4096), (33, 8, 2048), (5, 16, 128)])
def test_combine(dev, ydt, M, k, H):
    import moe_layer_topk_amd as moe
    say(f"combine {ydt} M={M} k={k} H={H}")
    y = normal_f32(1, S_Y, (M * k, H), 1.0, dev).to(ydt)
    wts = (counter_uniform_int(1, S_WTS, M * k, 1000, dev).float() / 1000.0).reshape(M, k)
    out = moe.moe_combine(y, wts, k, out_dtype=ydt)
    torch.cuda.synchronize()
    ref = oracle.combine(y.cpu(), wts.cpu(), k)
    tol = 1e-2 if ydt == torch.bfloat16 else 1e-5
    assert rel_err(out, ref) <= tol


# ------------------------------------------------------------------ layer

_W = {}


def weights(cfg, dev):
    if cfg not in _W:
        _W.clear()
        w = layer_weights(cfg, dev)
        host = {k: (v.cpu() if v is not None else None) for k, v in w.items()}
        _W[cfg] = (w, host)
    return _W[cfg]


def run_fused(cfg, b, w, dev, topk_ids=None, topk_weights=None):
    import moe_layer_topk_amd as moe
    return moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, x_scale=b["x_scale"],
                         w1_scale=w["w1_scale"], w2_scale=w["w2_scale"], topk_ids=topk_ids,
                         topk_weights=topk_weights)


def check_layer(cfg, M, dev, tokens=None, act_amax=None, batch=None):
    w, wh = weights(cfg, dev)
    b = layer_batch(cfg, M, dev) if batch is None else batch
    ids = torch.empty((M, cfg.topk), dtype=torch.int32, device=dev)
    wts = torch.empty((M, cfg.topk), dtype=torch.float32, device=dev)
    out = run_fused(cfg, b, w, dev, topk_ids=ids, topk_weights=wts)
    torch.cuda.synchronize()
    bh = {k: (v.cpu() if v is not None else None) for k, v in b.items()}
    rid, rw = oracle.route(bh["logits"], cfg.topk)
    assert np.array_equal(ids.cpu().numpy(), rid)
    # routing weights of the layer's own routing step (one launch with the
    # alignment for a few tokens, a separate route kernel otherwise)
    assert np.abs(wts.cpu().numpy() - rw).max() <= 1e-6
    tok = np.arange(M) if tokens is None else np.asarray(tokens)
    amax = act_amax
    if cfg.dtype == "fp8" and amax is None:
        amax = oracle.act_amax("fp8", bh["x"], bh["x_scale"], bh["logits"], wh["w1"], wh["w1_scale"], cfg.topk)
    ref = oracle.moe_layer(cfg.dtype, bh["x"], bh["x_scale"], bh["logits"], wh["w1"], wh["w1_scale"], wh["w2"],
                           wh["w2_scale"], cfg.topk, tokens=tok, act_amax_value=amax)
    err = rel_err(out.cpu()[torch.from_numpy(tok)], ref)
    say(f"  {cfg.name} M={M}: rel err {err:.3e} over {len(tok)} tokens")
    assert err <= TOL[cfg.dtype]
    return out


# 128 experts at 3-6 tokens: batch sizes where the decode GEMMs' row-group
# counts follow the active experts expected for the batch (one gate/up
# group; two down groups at 3 and 4 tokens, four at 5 and 6)
LAYER_CASES = [("tiny_f32", 16), ("mixtral_decode_bf16", 1), ("mixtral_decode_bf16", 8),
               ("finegrained_bf16", 1), ("finegrained_bf16", 3), ("finegrained_bf16", 4), ("finegrained_bf16", 5),
               ("finegrained_bf16", 6), ("finegrained_bf16", 16), ("fp8_e4m3", 1), ("fp8_e4m3", 8)]


@pytest.mark.parametrize("name,M", LAYER_CASES)
def test_fused_layer(dev, name, M):
    say(f"fused {name} M={M}")
    check_layer(CONFIGS[name], M, dev)


def test_fused_layer_full_decode_batch(dev):
    say("fused mixtral_decode_bf16 M=64 (every token)")
    check_layer(CONFIGS["mixtral_decode_bf16"], 64, dev)


@pytest.mark.parametrize("M", [256, 2048])
def test_fused_finegrained_full_sizes(dev, M):
    say(f"fused finegrained_bf16 M={M} (every token)")
    check_layer(CONFIGS["finegrained_bf16"], M, dev)


def tile_tokens(logits, E, k, block_m, rows=(0, 5, 13, 37, 70, 101, 127)):
    """Tokens whose pairs reach every row tile of the tile kernels' grid: for
    each block_m-row tile of the alignment, the pairs at the listed row
    offsets (both wavefront rows, both lane halves, several accumulator
    registers) and at the tile's last real row, which covers every expert's
    last, partial tile."""
    rid, _ = oracle.route(logits, k)
    al = oracle.align(rid, E, block_m)
    tok = set()
    for e in range(E):
        c, start = int(al["expert_counts"][e]), int(al["expert_offsets"][e])
        for t0 in range(0, c, block_m):
            real = min(block_m, c - t0)
            for r in [x for x in rows if x < real] + [real - 1]:
                tok.add(int(al["sorted_ids"][start + t0 + r]) // k)
    return np.array(sorted(tok))


def test_fused_mixtral_m32(dev):
    say("fused mixtral_decode_bf16 M=32")
    check_layer(CONFIGS["mixtral_decode_bf16"], 32, dev)


@pytest.mark.parametrize("M", [32, 512])
def test_fused_fp8_full_sizes(dev, M):
    """The fp8 workload at its full sizes; the batch-wide intermediate amax the
    oracle needs comes from tests/golden/fp8_act_amax.json (written by the
    oracle), after checking that the seeded inputs are the ones it used."""
    import json
    say(f"fused fp8_e4m3 M={M} (golden amax)")
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_act_amax.json")))
    cfg = CONFIGS["fp8_e4m3"]
    w, _ = weights(cfg, dev)
    # the stored statistic was computed from a CPU draw of the batch; drawing it
    # on the CPU here too keeps the quantised input bit-identical to that draw
    b = {k: (v.to(dev) if v is not None else None) for k, v in layer_batch(cfg, M, "cpu").items()}
    fp = gold["fingerprint"]
    assert float(b["x_scale"][0]) == fp[str(M)]["x_scale"]
    assert int(b["x"].view(torch.uint8).long().sum()) == fp[str(M)]["x_code_sum"]
    # weight draws on the GPU may differ from the CPU draw in a last bit of a value
    np.testing.assert_allclose([float(v) for v in w["w1_scale"][:8]], fp["w1_scale"], rtol=1e-6)
    np.testing.assert_allclose([float(v) for v in w["w2_scale"][:8]], fp["w2_scale"], rtol=1e-6)
    # 32 tokens: all of them; 512 tokens: every 128-row tile of the grid (rows
    # in both wavefront halves and the last real row of each tile)
    tok = None if M <= 32 else tile_tokens(b["logits"].cpu(), cfg.E, cfg.topk, 128, rows=(0, 70))
    check_layer(cfg, M, dev, tokens=tok, act_amax=gold["amax"][str(M)], batch=b)


def test_paths_agree_eq2_identity(dev, monkeypatch):
    """Swap-AB (decode) and non-swapped (prefill) kernels compute the same layer."""
    cfg = replace(CONFIGS["finegrained_bf16"], E=16, H=512, I=256)
    say("paths agree")
    w, _ = weights(cfg, dev)
    b = layer_batch(cfg, 200, dev)
    outs = {}
    for path in ("decode", "prefill"):
        monkeypatch.setenv("MOE_GEMM_PATH", path)
        outs[path] = run_fused(cfg, b, w, dev).float()
    torch.cuda.synchronize()
    d = (outs["decode"] - outs["prefill"]).abs().max().item()
    assert d <= 1e-2 * outs["decode"].abs().max().item()


@pytest.mark.parametrize("E,k,H,I,M", [(16, 8, 512, 256, 200), (8, 2, 1024, 512, 700), (4, 1, 256, 128, 1000),
                                        (128, 8, 512, 256, 400), (8, 2, 1024, 512, 160), (8, 2, 512, 256, 200)])
def test_fused_prefill_shapes(dev, E, k, H, I, M):
    """bf16 shapes with more than 24 pairs per expert take the LDS-ring tile
    kernel: 64-row tiles up to 48 pairs per expert (the 400- and 160-token
    cases, 25 and 40 on average), 128-row tiles above."""
    cfg = replace(CONFIGS["finegrained_bf16"], E=E, topk=k, H=H, I=I, router="zipf")
    say(f"fused prefill E={E} k={k} H={H} I={I} M={M}")
    check_layer(cfg, M, dev, tokens=np.arange(0, M, 7))


# extreme and degenerate layer shapes: the most experts and slots the ABI
# takes, a single expert (a dense SwiGLU FFN), top-k equal to E (every expert
# active), two experts sharing every token (prefill tiles holding both), and
# rows shorter than one 256-byte step per wavefront
EDGE_LAYERS = [("bf16", 256, 16, 256, 256, 33), ("bf16", 1, 1, 128, 128, 5), ("f32", 1, 1, 128, 128, 5),
               ("bf16", 8, 8, 128, 128, 1), ("bf16", 2, 2, 256, 128, 300), ("fp8", 256, 16, 256, 256, 20),
               ("fp8", 4, 4, 256, 256, 3)]


@pytest.mark.parametrize("dtype,E,k,H,I,M", EDGE_LAYERS)
def test_fused_edge_shapes(dev, dtype, E, k, H, I, M):
    base = {"f32": "tiny_f32", "bf16": "finegrained_bf16", "fp8": "fp8_e4m3"}[dtype]
    cfg = replace(CONFIGS[base], E=E, topk=k, H=H, I=I, router="normal")
    say(f"fused edge {dtype} E={E} k={k} H={H} I={I} M={M}")
    check_layer(cfg, M, dev)


def test_fused_layer_full_prefill(dev):
    """The 4096-token prefill layer: compared tokens chosen so that every
    128-row tile of the Zipf-skewed grid holds compared pairs."""
    cfg = CONFIGS["mixtral_prefill_bf16"]
    b = layer_batch(cfg, 4096, dev)
    tok = tile_tokens(b["logits"].cpu(), cfg.E, cfg.topk, 128)
    say(f"fused mixtral_prefill_bf16 M=4096 ({len(tok)} tokens covering every row tile)")
    check_layer(cfg, 4096, dev, tokens=tok, batch=b)


def test_fused_prefill_deterministic(dev):
    cfg = replace(CONFIGS["mixtral_prefill_bf16"], H=1024, I=1024)
    say("determinism (tile kernels)")
    w, _ = weights(cfg, dev)
    b = layer_batch(cfg, 600, dev)
    o1 = run_fused(cfg, b, w, dev).clone()
    o2 = run_fused(cfg, b, w, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("M", [8, 300])
def test_fp8_scale_product_invariance_gpu(dev, M):
    """(2 s_x, s_w1 / 2) leaves every product scale, hence the intermediate,
    its amax and the output, bit for bit unchanged; scaling s_w2 by 4 scales
    the output by 4 exactly (bf16 rounding commutes with powers of two)."""
    cfg = replace(CONFIGS["fp8_e4m3"], E=16, H=512, I=512)
    say(f"fp8 scale-product invariance M={M}")
    w, _ = weights(cfg, dev)
    b = layer_batch(cfg, M, dev)
    o1 = run_fused(cfg, b, w, dev).clone()
    b2 = dict(b, x_scale=b["x_scale"] * 2)
    w2 = dict(w, w1_scale=w["w1_scale"] / 2)
    o2 = run_fused(cfg, b2, w2, dev).clone()
    w4 = dict(w, w2_scale=w["w2_scale"] * 4)
    o4 = run_fused(cfg, b, w4, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(o4.float(), o1.float() * 4)


# the decode DOWN GEMM with the combine inside (bf16, about one token tile per
# expert): Mixtral and 128-expert shapes, a skewed batch whose first expert
# takes 32 pairs (two token tiles in one workgroup's sequence), H = 2048 (8
# output columns per workgroup) and H = 4096 (16)
DOWN_COMBINE = [("mixtral_decode_bf16", {}, 1, None), ("mixtral_decode_bf16", {}, 3, None),
                ("finegrained_bf16", {}, 1, None), ("finegrained_bf16", {}, 16, None),
                ("finegrained_bf16", {"E": 64, "topk": 2}, 32, 0), ("finegrained_bf16", {"H": 4096, "I": 512}, 5, None)]


@pytest.mark.parametrize("name,shape,M,skew", DOWN_COMBINE)
def test_down_combine_bitwise_equals_separate(dev, monkeypatch, name, shape, M, skew):
    """The fused layer's DOWN-with-combine kernel (opt-in) against the per-step
    path (DOWN GEMM into y, then moe_combine) on the same intermediate: the
    same bits; and the layer against the oracle."""
    import moe_layer_topk_amd as moe
    monkeypatch.setenv("MOE_DOWN_COMBINE", "1")
    cfg = replace(CONFIGS[name], **shape)
    say(f"down+combine {cfg.name} {shape} M={M} skew={skew}")
    w, wh = weights(cfg, dev)
    b = layer_batch(cfg, M, dev, seed=11)
    if skew is not None:
        b["logits"][:, skew] += 50.0  # every token's first choice
    k, E = cfg.topk, cfg.E
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    wts = torch.empty((M, k), dtype=torch.float32, device=dev)
    out = moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], k, topk_ids=ids, topk_weights=wts)
    al = moe.moe_align(ids, E, 16)
    act, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_GATE_UP_SILU, b["x"], w["w1"], al, M, k)
    y, _ = moe.moe_grouped_gemm(moe.MOE_GEMM_DOWN, act, w["w2"], al, M, k)
    ref = moe.moe_combine(y, wts, k)
    torch.cuda.synchronize()
    if skew is not None:
        assert int((ids[:, 0] == skew).sum()) == M
    assert torch.equal(out, ref), (out.float() - ref.float()).abs().max().item()
    check_layer(cfg, M, dev, batch=b)


def test_fused_deterministic(dev):
    cfg = CONFIGS["finegrained_bf16"]
    say("determinism")
    w, _ = weights(cfg, dev)
    b = layer_batch(cfg, 16, dev)
    o1 = run_fused(cfg, b, w, dev).clone()
    o2 = run_fused(cfg, b, w, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_token_permutation(dev):
    cfg = replace(CONFIGS["finegrained_bf16"], E=16, H=256, I=128)
    say("permutation")
    w, _ = weights(cfg, dev)
    b = layer_batch(cfg, 50, dev)
    perm = torch.randperm(50, generator=torch.Generator().manual_seed(0)).to(dev)
    o1 = run_fused(cfg, b, w, dev)
    bp = dict(b, x=b["x"][perm].contiguous(), logits=b["logits"][perm].contiguous())
    o2 = run_fused(cfg, bp, w, dev)
    torch.cuda.synchronize()
    assert (o1[perm].float() - o2.float()).abs().max().item() <= 1e-2 * o1.float().abs().max().item()


def test_empty_batch(dev):
    import moe_layer_topk_amd as moe
    cfg = replace(CONFIGS["finegrained_bf16"], E=16, H=256, I=128)
    w, _ = weights(cfg, dev)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    out = moe.fused_moe(x, torch.empty((0, 16), device=dev), w["w1"], w["w2"], cfg.topk)
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


def test_fused_no_renormalize(dev):
    """renormalize = 0: weights are the full softmax at the selected experts."""
    import moe_layer_topk_amd as moe
    cfg = replace(CONFIGS["finegrained_bf16"], E=16, H=256, I=128)
    say("fused renormalize=0")
    w, wh = weights(cfg, dev)
    b = layer_batch(cfg, 24, dev)
    out = moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, renormalize=False)
    torch.cuda.synchronize()
    bh = {k: (v.cpu() if v is not None else None) for k, v in b.items()}
    ref = oracle.moe_layer("bf16", bh["x"], None, bh["logits"], wh["w1"], None, wh["w2"], None, cfg.topk,
                           renormalize=False)
    assert rel_err(out.cpu(), ref) <= TOL["bf16"]


@pytest.mark.parametrize("name,M", [("finegrained_bf16", 4), ("fp8_e4m3", 8), ("mixtral_prefill_bf16", 300),
                                    ("finegrained_bf16", 1), ("fp8_e4m3", 1)])
def test_graph_replay(dev, name, M):
    """fused_moe captured in a HIP graph: every replay, with eager work and
    synchronisations in between, equals the eager result bit for bit (one
    token: the self-routed GEMMs, e4m3 with its amax partials in a workspace
    filled with junk before every replay)."""
    import moe_layer_topk_amd as moe
    cfg = CONFIGS[name]
    if name == "fp8_e4m3":
        cfg = replace(cfg, E=16, H=512, I=512)
    elif name == "mixtral_prefill_bf16":
        cfg = replace(cfg, H=1024, I=1024)  # 75 pairs per expert: the tile kernels
    say(f"graph replay {cfg.name} M={M}")
    w, _ = weights(cfg, dev)
    b = layer_batch(cfg, M, dev)
    dt = moe.moe_dtype(w["w1"])
    ws = torch.empty(moe.fused_moe_workspace_size(dt, M, cfg.E, cfg.topk, cfg.H, cfg.I), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((M, cfg.H), dtype=torch.bfloat16, device=dev)

    def call():
        moe.fused_moe(b["x"], b["logits"], w["w1"], w["w2"], cfg.topk, x_scale=b["x_scale"], w1_scale=w["w1_scale"],
                      w2_scale=w["w2_scale"], workspace=ws, out=out)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        ws.fill_(0xA5)  # the workspace contents on entry must not matter
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del junk

"""Pins for the CPU oracle, each against something other than the oracle itself.

- route ids: numpy stable argsort (independent sort; lower index first on ties)
- route weights: full softmax then renormalise (closed form), sum-to-one,
  k=1 -> exactly 1, k=E -> the full softmax
- align: numpy stable argsort of expert ids plus the padding invariants
- whole layer: brute-force dense evaluation of every expert on every token,
  masked by the routing weights (numpy float64)
- E=1, k=1: the dense SwiGLU FFN through torch CPU matmuls
- token order: permutation invariance
- e4m3 codec: torch's float8_e4m3fn (exhaustive decode; encode after clamping)
- fp8 scaling: scale-product invariance and a brute force that quantises the
  intermediate with torch's cast
"""
import math

import numpy as np
import pytest
import torch

import oracle


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_lib):
    return oracle_lib


def np_route(logits, k, renorm=True):
    lg = np.asarray(logits, np.float64)
    ids = np.argsort(-np.asarray(logits, np.float32), axis=1, kind="stable")[:, :k].astype(np.int32)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


def silu(z):
    return z / (1.0 + np.exp(-z))


def dense_masked(x, w1, w2, logits, k, renorm=True, act_fn=None):
    """Every expert on every token, outputs weighted by a top-k mask."""
    M, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    ids, w = np_route(logits, k, renorm)
    mask = np.zeros((M, E))
    for t in range(M):
        for j in range(k):
            mask[t, ids[t, j]] = w[t, j]
    out = np.zeros((M, H))
    for e in range(E):
        h = x @ w1[e].T
        a = silu(h[:, :I]) * h[:, I:]
        if act_fn is not None:
            a = act_fn(a)
        out += mask[:, e:e + 1] * (a @ w2[e].T)
    return out


# ------------------------------------------------------------------ route

@pytest.mark.parametrize("M,E,k", [(1, 8, 2), (37, 8, 2), (64, 128, 8), (20, 64, 8), (9, 5, 5), (13, 3, 1)])
def test_route_matches_stable_argsort(M, E, k):
    rng = np.random.default_rng(M * 1000 + E + k)
    lg = rng.standard_normal((M, E)).astype(np.float32)
    ids, w = oracle.route(lg, k)
    rid, rw = np_route(lg, k)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=1e-13, atol=1e-15)


def test_route_ties_lowest_index():
    E, k = 16, 4
    lg = np.zeros((3, E), np.float32)
    lg[1] = np.round(np.random.default_rng(1).standard_normal(E) * 2)  # many integer ties
    lg[2, :] = -0.0
    lg[2, ::2] = 0.0  # +0 and -0 compare equal
    ids, w = oracle.route(lg, k)
    assert ids[0].tolist() == [0, 1, 2, 3]
    assert ids[2].tolist() == [0, 1, 2, 3]
    rid, _ = np_route(lg, k)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w[0], 0.25, rtol=0, atol=1e-15)


def test_route_weights_identities():
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((50, 12)).astype(np.float32) * 3
    _, w = oracle.route(lg, 5)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)  # slot order is descending weight
    _, w1 = oracle.route(lg, 1)
    assert np.all(w1 == 1.0)
    ids, wf = oracle.route(lg, 12)
    p = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(wf, np.take_along_axis(p, ids, 1), rtol=1e-13)
    # renormalise=0: the selected entries of the full softmax
    ids, wn = oracle.route(lg, 3, renormalize=False)
    np.testing.assert_allclose(wn, np.take_along_axis(p, ids, 1), rtol=1e-13)
    assert np.all(wn.sum(axis=1) < 1.0)


def test_route_rejects_nonfinite():
    lg = np.zeros((2, 4), np.float32)
    lg[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.route(lg, 2)


# ------------------------------------------------------------------ align

def np_align(ids, E, bm):
    flat = ids.reshape(-1)
    P = flat.size
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    padded = (counts + bm - 1) // bm * bm
    offsets = np.concatenate([[0], np.cumsum(padded)])
    segs = np.split(order, np.cumsum(counts)[:-1])
    return counts, offsets, segs, P


@pytest.mark.parametrize("bm", [1, 16, 32, 64, 128])
@pytest.mark.parametrize("M,E,k,skew", [(64, 8, 2, 0), (300, 8, 2, 2), (16, 128, 8, 0), (50, 64, 8, 1),
                                        (1, 8, 2, 0), (7, 3, 3, 0)])
def test_align_matches_numpy(M, E, k, skew, bm):
    rng = np.random.default_rng(M + E + k + skew)
    lg = rng.standard_normal((M, E)).astype(np.float32)
    if skew:
        lg += (-skew * np.log1p(np.arange(E))).astype(np.float32)
    ids, _ = oracle.route(lg, k)
    a = oracle.align(ids, E, bm)
    counts, offsets, segs, P = np_align(ids, E, bm)
    assert np.array_equal(a["expert_counts"], counts)
    assert np.array_equal(a["expert_offsets"], offsets)
    s = a["sorted_ids"]
    assert len(s) == oracle.align_capacity(M, k, E, bm) and len(s) % bm == 0
    for e in range(E):
        seg = s[offsets[e]:offsets[e + 1]]
        assert np.array_equal(seg[:counts[e]], segs[e])
        assert np.all(seg[counts[e]:] == P)
    assert np.all(s[offsets[E]:] == P)
    # every pair exactly once
    real = s[s < P]
    assert np.array_equal(np.sort(real), np.arange(P))
    te = a["tile_expert"]
    for t in range(len(te)):
        r = t * bm
        exp = np.searchsorted(offsets, r, side="right") - 1 if r < offsets[E] else -1
        assert te[t] == exp
        if exp >= 0:
            assert np.all(ids.reshape(-1)[s[r:r + bm][s[r:r + bm] < P]] == exp)
    act = np.nonzero(counts)[0]
    assert a["num_active"][0] == len(act)
    assert np.array_equal(a["active_experts"][:len(act)], act)
    assert np.all(a["active_experts"][len(act):] == -1)


def test_align_all_to_one_expert_and_zero_counts():
    ids = np.full((40, 1), 5, np.int32)
    a = oracle.align(ids, 8, 16)
    assert a["expert_counts"].tolist() == [0, 0, 0, 0, 0, 40, 0, 0]
    assert a["expert_offsets"].tolist() == [0, 0, 0, 0, 0, 0, 48, 48, 48]
    assert a["sorted_ids"][:40].tolist() == list(range(40))
    assert np.all(a["sorted_ids"][40:] == 40)
    assert a["num_active"][0] == 1 and a["active_experts"][0] == 5


def test_align_capacity_bound():
    for M, k, E, bm in [(1, 2, 8, 16), (64, 2, 8, 128), (2048, 8, 128, 64), (0, 2, 8, 16), (3, 8, 128, 32)]:
        P = M * k
        cap = oracle.align_capacity(M, k, E, bm)
        assert cap % bm == 0 and cap >= P + min(E, P) * (bm - 1)
        assert cap < P + min(E, P) * (bm - 1) + bm


# ------------------------------------------------------------------ layer

def _rand_layer(rng, M, E, H, I, scale=0.3):
    x = rng.standard_normal((M, H)).astype(np.float32)
    w1 = (rng.standard_normal((E, 2 * I, H)) * scale).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * scale).astype(np.float32)
    lg = rng.standard_normal((M, E)).astype(np.float32)
    return x, w1, w2, lg


@pytest.mark.parametrize("seed", range(8))
def test_layer_matches_dense_masked(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.choice([1, 2, 4, 8]))
    k = int(rng.integers(1, E + 1))
    H, I = int(rng.integers(8, 65)), int(rng.integers(8, 65))
    M = int(rng.integers(1, 24))
    renorm = bool(seed % 3)
    x, w1, w2, lg = _rand_layer(rng, M, E, H, I)
    out = oracle.moe_layer("f32", x, None, lg, w1, None, w2, None, k, renormalize=renorm)
    ref = dense_masked(x.astype(np.float64), w1.astype(np.float64), w2.astype(np.float64), lg, k, renorm)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_layer_tiny_config_shape_dense_masked():
    # the tiny fp32 workload's shape (8 experts, top-2, hidden 256, intermediate 512)
    from workloads import CONFIGS, layer_batch, layer_weights
    cfg = CONFIGS["tiny_f32"]
    w = layer_weights(cfg, "cpu")
    b = layer_batch(cfg, 16, "cpu")
    out = oracle.moe_layer("f32", b["x"], None, b["logits"], w["w1"], None, w["w2"], None, cfg.topk)
    ref = dense_masked(b["x"].double().numpy(), w["w1"].double().numpy(), w["w2"].double().numpy(),
                       b["logits"].numpy(), cfg.topk)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_single_expert_is_swiglu_ffn():
    rng = np.random.default_rng(3)
    M, H, I = 11, 48, 40
    x, w1, w2, lg = _rand_layer(rng, M, 1, H, I)
    out = oracle.moe_layer("f32", x, None, lg, w1, None, w2, None, 1)
    xt = torch.from_numpy(x).double()
    wg, wu = torch.from_numpy(w1[0, :I]).double(), torch.from_numpy(w1[0, I:]).double()
    ref = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ torch.from_numpy(w2[0]).double().T
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_token_permutation_invariance_bitwise():
    rng = np.random.default_rng(5)
    M, E, k, H, I = 19, 8, 3, 32, 24
    x, w1, w2, lg = _rand_layer(rng, M, E, H, I)
    out = oracle.moe_layer("f32", x, None, lg, w1, None, w2, None, k)
    perm = rng.permutation(M)
    outp = oracle.moe_layer("f32", x[perm], None, lg[perm], w1, None, w2, None, k)
    assert np.array_equal(outp, out[perm])
    # a token subset computes the same rows
    sub = np.array([4, 0, 17])
    assert np.array_equal(oracle.moe_layer("f32", x, None, lg, w1, None, w2, None, k, tokens=sub), out[sub])


def test_bf16_storage_decodes_exactly():
    rng = np.random.default_rng(9)
    M, E, k, H, I = 6, 4, 2, 16, 8
    x, w1, w2, lg = _rand_layer(rng, M, E, H, I)
    xb, w1b, w2b = (torch.from_numpy(a).to(torch.bfloat16) for a in (x, w1, w2))
    out = oracle.moe_layer("bf16", xb, None, lg, w1b, None, w2b, None, k)
    ref = dense_masked(xb.double().numpy(), w1b.double().numpy(), w2b.double().numpy(), lg, k)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- steps

def test_pair_steps_and_combine_compose_to_layer():
    rng = np.random.default_rng(11)
    M, E, k, H, I = 9, 6, 2, 24, 16
    x, w1, w2, lg = _rand_layer(rng, M, E, H, I)
    ids, w = oracle.route(lg, k)
    pairs = np.arange(M * k)
    act = oracle.pairs_gate_up("f32", x, None, ids, w1, None, pairs)
    h = np.einsum("ph,pnh->pn", np.repeat(x.astype(np.float64), k, 0), w1[ids.reshape(-1)].astype(np.float64))
    np.testing.assert_allclose(act, silu(h[:, :I]) * h[:, I:], rtol=1e-12, atol=1e-14)
    y = oracle.pairs_down("f32", torch.from_numpy(act.astype(np.float32)), ids, w2, None, pairs)
    yr = np.einsum("pi,phi->ph", act.astype(np.float32).astype(np.float64), w2[ids.reshape(-1)].astype(np.float64))
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-14)
    out = oracle.combine(torch.from_numpy(y.astype(np.float32)), w.astype(np.float32), k)
    ref = np.einsum("tj,tjh->th", w.astype(np.float32).astype(np.float64),
                    y.astype(np.float32).astype(np.float64).reshape(M, k, H))
    np.testing.assert_allclose(out, ref, rtol=1e-13)


# ------------------------------------------------------------------ e4m3

def test_e4m3_decode_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]), c
    assert oracle.e4m3_decode(0x7E) == 448.0 and oracle.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_vs_torch_clamped():
    rng = np.random.default_rng(0)
    grid = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])  # non-negative finite codes
    mids = (grid[1:] + grid[:-1]) / 2
    vals = np.concatenate([
        grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.standard_normal(20000) * 50, rng.standard_normal(5000) * 1e-3,
        rng.uniform(-600, 600, 5000), [0.0, 448.0, 449.0, 464.0, 465.0, 480.0, 1e9, 2.0 ** -10, 2.0 ** -11],
    ])
    vals = np.concatenate([vals, -vals]).astype(np.float32)  # both sides see float32 inputs
    ref = torch.from_numpy(vals).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(vals[i], got[i], ref[i]) for i in bad[:5]]
    assert oracle.e4m3_encode(float("nan")) == 0x7F


# ------------------------------------------------------------------- fp8

def _fp8_case(seed, M=7, E=4, k=2, H=32, I=16):
    from workloads.gen import _quant_e4m3_per_tensor
    rng = np.random.default_rng(seed)
    x, w1, w2, lg = _rand_layer(rng, M, E, H, I, scale=0.05)
    xq, sx = _quant_e4m3_per_tensor(torch.from_numpy(x))
    q1, q2, s1, s2 = [], [], [], []
    for e in range(E):
        a, s = _quant_e4m3_per_tensor(torch.from_numpy(w1[e]))
        q1.append(a), s1.append(s)
        a, s = _quant_e4m3_per_tensor(torch.from_numpy(w2[e]))
        q2.append(a), s2.append(s)
    return xq, sx, lg, torch.stack(q1), torch.cat(s1), torch.stack(q2), torch.cat(s2), k


def test_fp8_scale_product_invariance_bitwise():
    xq, sx, lg, w1, s1, w2, s2, k = _fp8_case(21)
    out = oracle.moe_layer("fp8", xq, sx, lg, w1, s1, w2, s2, k)
    out2 = oracle.moe_layer("fp8", xq, sx * 2, lg, w1, s1 / 2, w2, s2, k)
    assert np.array_equal(out, out2)
    # scaling the down weights scales the output exactly
    out3 = oracle.moe_layer("fp8", xq, sx, lg, w1, s1, w2, s2 * 4, k)
    assert np.array_equal(out3, out * 4)


def test_fp8_layer_matches_brute_force_with_torch_codec():
    xq, sx, lg, w1, s1, w2, s2, k = _fp8_case(22)
    x = xq.double().numpy() * float(sx)
    w1d = w1.double().numpy() * s1.double().numpy()[:, None, None]
    w2d = w2.double().numpy() * s2.double().numpy()[:, None, None]
    E, twoI, H = w1d.shape
    I = twoI // 2
    # amax over every pair's float64 intermediate
    ids, _ = np_route(lg, k)
    amax = 0.0
    for t in range(x.shape[0]):
        for j in range(k):
            h = w1d[ids[t, j]] @ x[t]
            amax = max(amax, np.abs(silu(h[:I]) * h[I:]).max())
    assert abs(oracle.act_amax("fp8", xq, sx, lg, w1, s1, k) - amax) <= 1e-12 * amax
    s = np.float32(amax) / np.float32(448.0)

    def q(a):
        v = torch.from_numpy((a.astype(np.float32) / s).astype(np.float32)).clamp(-448, 448)
        return v.to(torch.float8_e4m3fn).double().numpy() * float(s)

    ref = dense_masked(x, w1d, w2d, lg, k, act_fn=q)
    out = oracle.moe_layer("fp8", xq, sx, lg, w1, s1, w2, s2, k, act_amax_value=amax)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_fp8_golden_amax_single_token_recomputes():
    """The stored batch amax of the fp8 workload at M=1 is the oracle's (only the
    8 experts the token is routed to are generated here)."""
    import json
    import os
    from workloads import CONFIGS, layer_batch, layer_weights
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_act_amax.json")))
    cfg = CONFIGS["fp8_e4m3"]
    b = layer_batch(cfg, 1, "cpu")
    assert float(b["x_scale"][0]) == gold["fingerprint"]["1"]["x_scale"]
    ids, _ = oracle.route(b["logits"], cfg.topk)
    w = layer_weights(cfg, "cpu", experts=sorted(set(ids.reshape(-1).tolist())))
    am = oracle.act_amax("fp8", b["x"], b["x_scale"], b["logits"], w["w1"], w["w1_scale"], cfg.topk)
    assert am == gold["amax"]["1"]


# ---------------------------------------------------------------- router

def test_router_logits_vs_numpy_matmul():
    """oracle.router_logits against numpy's float64 matmul of the widened
    inputs, for float32, bfloat16 and e4m3 (times its scale) activations."""
    from workloads.gen import _quant_e4m3_per_tensor
    rng = np.random.default_rng(41)
    M, E, H = 9, 12, 96
    x = rng.standard_normal((M, H)).astype(np.float32)
    wg = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    ref = x.astype(np.float64) @ wg.astype(np.float64).T
    np.testing.assert_allclose(oracle.router_logits("f32", x, None, wg), ref, rtol=1e-12, atol=1e-14)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    refb = xb.double().numpy() @ wg.astype(np.float64).T
    np.testing.assert_allclose(oracle.router_logits("bf16", xb, None, wg), refb, rtol=1e-12, atol=1e-14)
    xq, sx = _quant_e4m3_per_tensor(torch.from_numpy(x))
    refq = (xq.double().numpy() * float(sx)) @ wg.astype(np.float64).T
    np.testing.assert_allclose(oracle.router_logits("fp8", xq, sx, wg), refq, rtol=1e-12, atol=1e-14)
    # a one-hot router row picks that activation column
    wg1 = np.zeros((E, H), np.float32)
    wg1[3, 17] = 1.0
    assert np.array_equal(oracle.router_logits("f32", x, None, wg1)[:, 3], x[:, 17].astype(np.float64))


# ------------------------------------------------- int4 weights (W4A16)

def _unpack_int4(codes, gscale):
    """Independent decoder of the packed int4 layout: the 4 bytes covering 8
    consecutive k hold (k0, k0+2), (k0+4, k0+6), (k0+1, k0+3), (k0+5, k0+7)
    as (low, high) nibbles; value = (u - 8) * scale[k // 128][n]."""
    c = np.asarray(codes, np.uint8)
    N, K = c.shape[0], c.shape[1] * 2
    b = c.reshape(N, K // 8, 4)
    u = np.empty((N, K // 8, 8), np.int64)
    u[..., 0], u[..., 2] = b[..., 0] & 15, b[..., 0] >> 4
    u[..., 4], u[..., 6] = b[..., 1] & 15, b[..., 1] >> 4
    u[..., 1], u[..., 3] = b[..., 2] & 15, b[..., 2] >> 4
    u[..., 5], u[..., 7] = b[..., 3] & 15, b[..., 3] >> 4
    s = np.asarray(gscale, np.float64).T  # [N][K/128]
    return (u.reshape(N, K) - 8) * np.repeat(s, 128, axis=1)


def test_int4_packing_round_trip_and_error_bound():
    """The generator's codes decode (independent unpacker and the oracle's
    element accessor agree) to within half a scale step of the float32 input,
    and a group's largest |value| is exactly 7 steps."""
    from workloads import quant_int4_groups
    rng = np.random.default_rng(51)
    v = torch.from_numpy((rng.standard_normal((6, 384)) * 0.02).astype(np.float32))
    v[2, 128:256] = 0.0  # an all-zero group: scale 1, codes 8
    codes, gs = quant_int4_groups(v)
    dq = _unpack_int4(codes.numpy(), gs.numpy())
    step = np.repeat(gs.numpy().T.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(dq - v.numpy()) <= 0.5 * step * (1 + 1e-6))
    assert np.all(dq[2, 128:256] == 0.0) and gs[1, 2] == 1.0
    g = np.abs(dq).reshape(6, 3, 128).max(axis=2)
    assert np.allclose(g[g > 0] / gs.numpy().T[g > 0], 7.0)
    for n, k in [(0, 0), (0, 1), (1, 7), (3, 8), (5, 383), (4, 200), (2, 130)]:
        assert oracle.int4_weight(codes, gs, n, k) == dq[n, k]


def test_w4a16_layer_matches_dense_masked_brute_force():
    """The W4A16 layer (bf16 activations, int4 weights) against every expert
    on every token with the independently dequantised weights."""
    from workloads import quant_int4_groups
    rng = np.random.default_rng(52)
    M, E, k, H, I = 9, 5, 2, 256, 128
    x = torch.from_numpy(rng.standard_normal((M, H)).astype(np.float32)).to(torch.bfloat16)
    lg = rng.standard_normal((M, E)).astype(np.float32)
    c1, s1, c2, s2, d1, d2 = [], [], [], [], [], []
    for e in range(E):
        a, s = quant_int4_groups(torch.from_numpy((rng.standard_normal((2 * I, H)) * 0.05).astype(np.float32)))
        c1.append(a), s1.append(s), d1.append(_unpack_int4(a.numpy(), s.numpy()))
        a, s = quant_int4_groups(torch.from_numpy((rng.standard_normal((H, I)) * 0.05).astype(np.float32)))
        c2.append(a), s2.append(s), d2.append(_unpack_int4(a.numpy(), s.numpy()))
    out = oracle.moe_layer("w4a16", x, None, lg, torch.stack(c1), torch.stack(s1), torch.stack(c2), torch.stack(s2), k)
    ref = dense_masked(x.double().numpy(), np.stack(d1), np.stack(d2), lg, k)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())

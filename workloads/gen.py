"""Counter-based seeded generator and the MoE workload shapes.

Every value is a pure function of (seed, stream, element index), computed
with exact integer arithmetic followed by a Box-Muller transform in float64,
so a draw made on the CPU and the same draw made on a GPU hold the same
bytes (up to a last-ulp difference of the float64 log/cos, which the storage
rounding to fp32/bf16/e4m3 absorbs except with negligible probability).
Because element i of a tensor depends only on i, a batch of M tokens is the
first M rows of any larger batch drawn with the same seed.

Integer mixing uses the "lowbias32" avalanche function from C. Wellons' hash
prospector (two multiply/xor-shift rounds).  Products are taken modulo 2**32
by splitting the constant into 16-bit halves, so every intermediate stays
below 2**49 in int64 and nothing overflows.

Workload shapes follow the MoE problem statement of the pages: routed token
rows A[M,K] times expert weights B[K,N] (MoE kernel engineering post,
"Swap-AB for WGMMA utilization", Eq. 1), Mixtral-8x7B-like experts
(FusedMoE vs MegaMoE post, sections 2 and 3.2: 8 experts, top-2, hidden 4096,
ffn 14336), an 8192-wide expert N (Swap-AB section) and FP8 tensors with one
scale per tensor (FP8 backend-routing section).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_M32 = 0xFFFFFFFF
_CHUNK_GPU = 1 << 26  # elements per generation chunk on a GPU (bounds temporaries)
_CHUNK_CPU = 1 << 18  # on the host: small enough that the int64 temporaries stay in cache

# stream tags: one independent stream per tensor role
S_X, S_LOGITS, S_WG, S_W1, S_W2, S_ACT, S_Y, S_WTS, S_IDS = range(1, 10)


def _mul32_py(a: int, c: int) -> int:
    return (a * c) & _M32


def _lowbias32_py(x: int) -> int:
    x ^= x >> 16
    x = _mul32_py(x, 0x7FEB352D)
    x ^= x >> 15
    x = _mul32_py(x, 0x846CA68B)
    x ^= x >> 16
    return x


def _mul32(a: torch.Tensor, c: int) -> torch.Tensor:
    """(a * c) mod 2**32 for int64 tensors holding values in [0, 2**32)."""
    lo = a * (c & 0xFFFF)
    hi = ((a * (c >> 16)) & 0xFFFF) << 16
    return (lo + hi) & _M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _key(seed: int, stream: int, word: int) -> int:
    k = _lowbias32_py((seed & _M32) ^ 0x9E3779B9)
    k = _lowbias32_py(k ^ (stream & _M32))
    k = _lowbias32_py(k ^ (word * 0x85EBCA6B & _M32))
    return k


def _words(idx: torch.Tensor, seed: int, stream: int, word: int) -> torch.Tensor:
    k = _key(seed, stream, word)
    h = _lowbias32((idx & _M32) ^ k)
    return _lowbias32(h ^ (idx >> 32) ^ (k >> 1))


def counter_normal(seed: int, stream: int, n: int, device, offset: int = 0) -> torch.Tensor:
    """n standard-normal float64 draws for elements [offset, offset + n)."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    two_pi = 2.0 * math.pi
    inv32 = 1.0 / 4294967296.0
    chunk = _CHUNK_CPU if torch.device(device).type == "cpu" else _CHUNK_GPU
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(offset + s, offset + e, dtype=torch.int64, device=device)
        u1 = (_words(idx, seed, stream, 0) + 1).to(torch.float64) * inv32  # (0, 1]
        u2 = _words(idx, seed, stream, 1).to(torch.float64) * inv32  # [0, 1)
        del idx
        r = torch.sqrt(-2.0 * torch.log(u1))
        out[s:e] = r * torch.cos(two_pi * u2)
    return out


def counter_uniform_int(seed: int, stream: int, n: int, hi: int, device, offset: int = 0) -> torch.Tensor:
    """n integers uniform in [0, hi) (hi < 2**16), as int32."""
    idx = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    return ((_words(idx, seed, stream, 0) >> 8) % hi).to(torch.int32)


def normal_f32(seed, stream, shape, std, device, offset=0) -> torch.Tensor:
    n = math.prod(shape)
    z = counter_normal(seed, stream, n, device, offset)
    if std != 1.0:
        z = z * std
    return z.to(torch.float32).reshape(shape)


def normal_bf16(seed, stream, shape, std, device, offset=0) -> torch.Tensor:
    # float64 -> float32 -> bfloat16, each step round-to-nearest-even
    return normal_f32(seed, stream, shape, std, device, offset).to(torch.bfloat16)


def fill_normal(dst: torch.Tensor, seed: int, stream: int, std: float, offset: int = 0) -> torch.Tensor:
    """normal_f32 / normal_bf16 of dst's shape written into dst (float32 or
    bfloat16, contiguous) chunk by chunk: the same bytes, with a few large
    launches and no whole-tensor float64 temporary."""
    flat = dst.view(-1)
    n = flat.numel()
    chunk = _CHUNK_CPU if dst.device.type == "cpu" else _CHUNK_GPU
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        z = counter_normal(seed, stream, e - s, dst.device, offset + s)
        if std != 1.0:
            z = z * std
        flat[s:e] = z.to(torch.float32).to(dst.dtype)
    return dst


def _quant_e4m3_per_tensor(v: torch.Tensor):
    """Store a float32 tensor as OCP e4m3 with one float32 scale s = amax/448.

    s and 1/s are computed on the host in IEEE float32 (numpy), and the codes
    are torch's float8_e4m3fn cast (round to nearest even) of v * (1/s), so a
    CPU and a GPU draw give the same bytes (a division by a scalar is not
    rounded the same way on both).  The clamp keeps values that would round
    past 448 finite.
    """
    import numpy as np
    amax = np.float32(v.abs().max().item())
    s = amax / np.float32(448.0) if amax > 0 else np.float32(1.0)
    inv = np.float32(1.0) / s
    q = (v * float(inv)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q, torch.tensor([float(s)], dtype=torch.float32, device=v.device)


def quant_int4_groups(v: torch.Tensor):
    """Weight-only int4 storage of a float32 matrix v [N][K] (K a multiple of
    128): per row and 128-wide group of k, scale = amax / 7 (float32; 1 for an
    all-zero group) and code u = 8 + round-half-even(v / scale) clamped to
    [1, 15].  Returns (codes uint8 [N][K/2], scales float32 [K/128][N]) in the
    library's packing: the codes of 8 consecutive k fill one little-endian
    32-bit word, k0+2i at bits 4i and k0+2i+1 at bits 16+4i."""
    N, K = v.shape
    g = v.reshape(N, K // 128, 128)
    amax = g.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / 7.0, torch.ones_like(amax))
    u = (torch.round(g / s[:, :, None]).clamp(-7, 7) + 8).to(torch.uint8).reshape(N, K // 8, 8)
    b0 = u[..., 0] | (u[..., 2] << 4)
    b1 = u[..., 4] | (u[..., 6] << 4)
    b2 = u[..., 1] | (u[..., 3] << 4)
    b3 = u[..., 5] | (u[..., 7] << 4)
    codes = torch.stack([b0, b1, b2, b3], dim=2).reshape(N, K // 2)
    return codes, s.t().contiguous()


@dataclass(frozen=True)
class LayerConfig:
    name: str
    E: int
    topk: int
    H: int
    I: int
    dtype: str  # "f32" | "bf16" | "fp8" | "w4a16" (int4 weights, bf16 activations)
    Ms: tuple
    router: str  # "x_wg" | "normal" | "zipf"
    weight_std: float = 0.02
    zipf_s: float = 1.1
    desc: str = field(default="", compare=False)


CONFIGS = {
    c.name: c
    for c in [
        LayerConfig("tiny_f32", 8, 2, 256, 512, "f32", (16,), "x_wg",
                    desc="tiny fp32 layer, router logits x.Wg"),
        LayerConfig("mixtral_decode_bf16", 8, 2, 4096, 14336, "bf16", (1, 8, 32, 64), "normal",
                    desc="Mixtral-8x7B-shaped layer, bf16 decode batches"),
        LayerConfig("mixtral_prefill_bf16", 8, 2, 4096, 14336, "bf16", (4096,), "zipf",
                    desc="Mixtral-8x7B-shaped layer, bf16 prefill with Zipf(1.1)-skewed routing"),
        LayerConfig("finegrained_bf16", 128, 8, 2048, 768, "bf16", (1, 16, 256, 2048), "normal",
                    desc="fine-grained 128-expert top-8 layer, bf16"),
        LayerConfig("fp8_e4m3", 64, 8, 4096, 8192, "fp8", (1, 32, 512), "normal",
                    desc="per-tensor-scaled OCP e4m3 layer, bf16 output"),
        LayerConfig("mixtral_decode_w4a16", 8, 2, 4096, 14336, "w4a16", (1, 8, 32, 64), "normal",
                    desc="Mixtral-8x7B-shaped layer, weight-only int4 (128-wide groups), bf16 activations"),
        LayerConfig("finegrained_w4a16", 128, 8, 2048, 768, "w4a16", (1, 16), "normal",
                    desc="fine-grained 128-expert top-8 layer, weight-only int4, bf16 activations"),
    ]
}


def layer_weights(cfg: LayerConfig, device, seed: int = 0, experts=None) -> dict:
    """Expert weights, K-contiguous: w1[E][2I][H] (gate rows then up rows), w2[E][H][I].

    For fp8, each expert matrix carries one float32 scale (w1_scale[E], w2_scale[E]).
    `experts` restricts generation to a subset (others are left zero) for
    memory-bounded host-side work; default is all experts.
    """
    E, H, I = cfg.E, cfg.H, cfg.I
    n1, n2 = 2 * I * H, H * I
    sel = range(E) if experts is None else experts
    if cfg.dtype == "w4a16":
        # the bf16 layer's float32 draws, stored as int4 codes and group scales
        w1 = torch.full((E, 2 * I, H // 2), 0x88, dtype=torch.uint8, device=device)
        w2 = torch.full((E, H, I // 2), 0x88, dtype=torch.uint8, device=device)
        s1 = torch.ones((E, H // 128, 2 * I), dtype=torch.float32, device=device)
        s2 = torch.ones((E, I // 128, H), dtype=torch.float32, device=device)
        for e in sel:
            v = normal_f32(seed, S_W1, (2 * I, H), cfg.weight_std, device, offset=e * n1)
            w1[e], s1[e] = quant_int4_groups(v)
            v = normal_f32(seed, S_W2, (H, I), cfg.weight_std, device, offset=e * n2)
            w2[e], s2[e] = quant_int4_groups(v)
            del v
        return {"w1": w1, "w2": w2, "w1_scale": s1, "w2_scale": s2}
    if cfg.dtype == "fp8":
        w1 = torch.zeros((E, 2 * I, H), dtype=torch.float8_e4m3fn, device=device)
        w2 = torch.zeros((E, H, I), dtype=torch.float8_e4m3fn, device=device)
        s1 = torch.ones(E, dtype=torch.float32, device=device)
        s2 = torch.ones(E, dtype=torch.float32, device=device)
        for e in sel:
            v = normal_f32(seed, S_W1, (2 * I, H), cfg.weight_std, device, offset=e * n1)
            w1[e], s1[e:e + 1] = _quant_e4m3_per_tensor(v)
            v = normal_f32(seed, S_W2, (H, I), cfg.weight_std, device, offset=e * n2)
            w2[e], s2[e:e + 1] = _quant_e4m3_per_tensor(v)
            del v
        return {"w1": w1, "w2": w2, "w1_scale": s1, "w2_scale": s2}
    mk = normal_bf16 if cfg.dtype == "bf16" else normal_f32
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if experts is None:
        # expert e's element i is element e * n + i of one stream: all experts in one fill
        w1 = fill_normal(torch.empty((E, 2 * I, H), dtype=dt, device=device), seed, S_W1, cfg.weight_std)
        w2 = fill_normal(torch.empty((E, H, I), dtype=dt, device=device), seed, S_W2, cfg.weight_std)
        return {"w1": w1, "w2": w2, "w1_scale": None, "w2_scale": None}
    w1 = torch.zeros((E, 2 * I, H), dtype=dt, device=device)
    w2 = torch.zeros((E, H, I), dtype=dt, device=device)
    for e in sel:
        w1[e] = mk(seed, S_W1, (2 * I, H), cfg.weight_std, device, offset=e * n1)
        w2[e] = mk(seed, S_W2, (H, I), cfg.weight_std, device, offset=e * n2)
    return {"w1": w1, "w2": w2, "w1_scale": None, "w2_scale": None}


def zipf_log_prior(E: int, s: float) -> list:
    """ln p_e with p_e proportional to (e+1)^-s, expert 0 the most likely."""
    z = sum((e + 1) ** -s for e in range(E))
    return [math.log((e + 1) ** -s / z) for e in range(E)]


def layer_batch(cfg: LayerConfig, M: int, device, seed: int = 0) -> dict:
    """Token activations x[M,H] and router logits[M,E] (float32) for one batch."""
    E, H = cfg.E, cfg.H
    out = {}
    if cfg.dtype == "fp8":
        xf = normal_f32(seed, S_X, (M, H), 1.0, device)
        if M > 0:
            out["x"], out["x_scale"] = _quant_e4m3_per_tensor(xf)
        else:
            out["x"] = xf.to(torch.float8_e4m3fn)
            out["x_scale"] = torch.ones(1, dtype=torch.float32, device=device)
    elif cfg.dtype in ("bf16", "w4a16"):
        out["x"], out["x_scale"] = normal_bf16(seed, S_X, (M, H), 1.0, device), None
    else:
        out["x"], out["x_scale"] = normal_f32(seed, S_X, (M, H), 1.0, device), None

    if cfg.router == "x_wg":
        # router projection done here, on the host, in float64 and rounded to
        # float32 once; the layer consumes the logits as given
        wg = normal_f32(seed, S_WG, (H, E), cfg.weight_std, "cpu")
        xs = out["x"].to("cpu", torch.float64)
        out["logits"] = (xs @ wg.to(torch.float64)).to(torch.float32).to(device)
    elif cfg.router == "zipf":
        z = counter_normal(seed, S_LOGITS, M * E, device).reshape(M, E)
        prior = torch.tensor(zipf_log_prior(E, cfg.zipf_s), dtype=torch.float64, device=device)
        out["logits"] = (z + prior).to(torch.float32)
    else:
        out["logits"] = counter_normal(seed, S_LOGITS, M * E, device).reshape(M, E).to(torch.float32)
    return out

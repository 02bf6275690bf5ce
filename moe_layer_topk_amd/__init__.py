"""Fused top-k Mixture-of-Experts layer for MI355X (gfx950).

A thin binding over libmoe.so: every function here only allocates output
tensors with torch, marshals pointers and calls the C entry point of the
same name on torch's current HIP stream.  All arithmetic runs in the HIP
kernels; there is no CPU or framework fallback (a missing library raises).

Steps of the layer (FusedMoE vs MegaMoE post, sections 2 and 3.1):
moe_route -> moe_align -> moe_grouped_gemm (gate/up + SiLU-and-mul, then
down) -> moe_combine, or all of them in one call with fused_moe.  For e4m3
weights the intermediate is float32 and the down call quantises it on load;
moe_quant_act gives the same codes as a tensor.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (  # noqa: F401
    MOE_ERR_SCRATCH,
    MOE_W4A16,
    MOE_BF16,
    MOE_F32,
    MOE_FP8_E4M3,
    MOE_GEMM_DOWN,
    MOE_GEMM_DOWN_E4M3_ACT,
    MOE_GEMM_GATE_UP_SILU,
    AlignBufs,
    MoeError,
    check,
    lib,
)

# weight storage -> layer dtype (uint8 weights are packed int4 codes, W4A16)
_DTYPES = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float8_e4m3fn: MOE_FP8_E4M3, torch.uint8: MOE_W4A16}
_INTER = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_FP8_E4M3: torch.bfloat16,
          MOE_W4A16: torch.bfloat16}  # y and out
_ACT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_FP8_E4M3: torch.float32,
        MOE_W4A16: torch.bfloat16}  # the intermediate


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("moe_layer_topk_amd computes on the GPU only; got a CPU tensor")
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def moe_dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def moe_route(logits: torch.Tensor, topk: int, renormalize: bool = True, topk_ids=None, topk_weights=None):
    """Top-k ids (int32 [M,k]) and weights (float32 [M,k]) from float32 logits [M,E]."""
    M, E = logits.shape
    ids = topk_ids if topk_ids is not None else torch.empty((M, topk), dtype=torch.int32, device=logits.device)
    wts = topk_weights if topk_weights is not None else torch.empty((M, topk), dtype=torch.float32,
                                                                    device=logits.device)
    check(lib().moe_route(_p(logits), M, E, topk, int(renormalize), _p(ids), _p(wts), _stream(logits)),
          "moe_route")
    return ids, wts


def moe_align_capacity(M: int, topk: int, E: int, block_m: int) -> int:
    return lib().moe_align_capacity(M, topk, E, block_m)


def moe_align(topk_ids: torch.Tensor, E: int, block_m: int) -> dict:
    """Index system of the sorted pairs (see moe_align_bufs in include/moe.h)."""
    M, topk = topk_ids.shape
    cap = moe_align_capacity(M, topk, E, block_m)
    dev = topk_ids.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = {
        "sorted_ids": torch.empty(max(cap, 1), **i32),
        "tile_expert": torch.empty(max(cap // block_m, 1), **i32),
        "expert_counts": torch.empty(E, **i32),
        "expert_offsets": torch.empty(E + 1, **i32),
        "active_experts": torch.empty(max(min(E, M * topk), 1), **i32),
        "num_active": torch.empty(1, **i32),
        "block_m": block_m,
    }
    check(lib().moe_align(_p(topk_ids), M, topk, E, block_m, align_struct(out), _stream(topk_ids)), "moe_align")
    return out


def align_struct(al: dict) -> AlignBufs:
    return AlignBufs(*(al[n].data_ptr() for n in
                       ("sorted_ids", "tile_expert", "expert_counts", "expert_offsets", "active_experts",
                        "num_active")))


def moe_grouped_gemm(kind: int, a: torch.Tensor, w: torch.Tensor, al: dict, M: int, topk: int,
                     a_scale=None, w_scale=None, c=None, c_amax=None):
    """GATE_UP: act[P, N/2] = silu(gate) * up;  DOWN: y[P, N].  Returns (c, c_amax)."""
    E, N, K = w.shape
    dt = moe_dtype(w)
    if dt == MOE_W4A16:
        K *= 2  # two 4-bit codes per byte
    P = M * topk
    cols = N // 2 if kind == MOE_GEMM_GATE_UP_SILU else N
    if kind != MOE_GEMM_GATE_UP_SILU and (kind == MOE_GEMM_DOWN_E4M3_ACT) != (a.dtype == torch.float8_e4m3fn):
        raise ValueError("MOE_GEMM_DOWN_E4M3_ACT takes e4m3 act codes and e4m3 weights; DOWN takes the act")
    if kind != MOE_GEMM_GATE_UP_SILU and kind != MOE_GEMM_DOWN_E4M3_ACT and a.dtype != _ACT[dt]:
        raise ValueError(f"DOWN with {w.dtype} weights takes a {_ACT[dt]} intermediate, got {a.dtype}")
    if c is None:
        c = torch.empty((P, cols), dtype=_ACT[dt] if kind == MOE_GEMM_GATE_UP_SILU else _INTER[dt], device=w.device)
    if dt == MOE_FP8_E4M3 and kind == MOE_GEMM_GATE_UP_SILU and c_amax is None:
        c_amax = torch.empty(1, dtype=torch.float32, device=w.device)
    bufs = align_struct(al)
    check(lib().moe_grouped_gemm(kind, dt, _p(a), _p(a_scale), _p(w), _p(w_scale), ctypes.byref(bufs), M, topk,
                                 E, N, K, al["block_m"], _p(c), _p(c_amax), _stream(w)), "moe_grouped_gemm")
    return c, c_amax


def moe_quant_act(act: torch.Tensor, amax: torch.Tensor, out=None):
    """e4m3 codes (torch.float8_e4m3fn, same shape) of the float32 intermediate with scale amax/448."""
    if act.dtype != torch.float32:
        raise ValueError("moe_quant_act takes the float32 intermediate")
    q = out if out is not None else torch.empty(act.shape, dtype=torch.float8_e4m3fn, device=act.device)
    check(lib().moe_quant_act(_p(act), _p(amax), act.numel(), _p(q), _stream(act)), "moe_quant_act")
    return q


def moe_combine(y: torch.Tensor, topk_weights: torch.Tensor, topk: int, out_dtype=None, out=None):
    P, H = y.shape
    M = P // topk
    odt = y.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, H), dtype=odt, device=y.device)
    check(lib().moe_combine(moe_dtype(y), _p(y), _p(topk_weights), M, topk, H, moe_dtype(out), _p(out),
                            _stream(y)), "moe_combine")
    return out


def fused_moe_workspace_size(dtype: int, M: int, E: int, topk: int, H: int, I: int) -> int:
    return lib().fused_moe_workspace_size(dtype, M, E, topk, H, I)


def fused_moe(x, router_logits, w1, w2, topk: int, renormalize: bool = True, x_scale=None, w1_scale=None,
              w2_scale=None, workspace=None, out=None, topk_ids=None, topk_weights=None):
    """The whole layer; returns out[M,H] (float32 for fp32 weights, bfloat16 otherwise)."""
    M, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    dt = moe_dtype(w1)
    need = fused_moe_workspace_size(dt, M, E, topk, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=_INTER[dt], device=x.device)
    check(lib().fused_moe(dt, _p(x), _p(x_scale), _p(router_logits), _p(w1), _p(w1_scale), _p(w2), _p(w2_scale),
                          M, E, topk, H, I, int(renormalize), _p(out), _p(topk_ids), _p(topk_weights),
                          _p(workspace), workspace.numel(), _stream(x)), "fused_moe")
    return out


def fused_moe_noalloc(x, router_logits, w1, w2, topk: int, renormalize: bool = True, x_scale=None, w1_scale=None,
                      w2_scale=None, out=None, topk_ids=None, topk_weights=None):
    """fused_moe with the library's static device scratch as its workspace
    (no workspace argument; calls overlapping on one GPU race)."""
    M, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    dt = moe_dtype(w1)
    if out is None:
        out = torch.empty((M, H), dtype=_INTER[dt], device=x.device)
    check(lib().fused_moe_noalloc(dt, _p(x), _p(x_scale), _p(router_logits), _p(w1), _p(w1_scale), _p(w2),
                                  _p(w2_scale), M, E, topk, H, I, int(renormalize), _p(out), _p(topk_ids),
                                  _p(topk_weights), _stream(x)), "fused_moe_noalloc")
    return out


def moe_router_logits(x, router_w, x_scale=None, out=None):
    """Router scores float32 [M, E] = x . router_w^T (router_w float32 [E, H])."""
    M, H = x.shape
    E = router_w.shape[0]
    if router_w.dtype != torch.float32:
        raise ValueError("router weights are float32")
    lg = out if out is not None else torch.empty((M, E), dtype=torch.float32, device=x.device)
    check(lib().moe_router_logits(moe_dtype(x), _p(x), _p(x_scale), _p(router_w), M, H, E, _p(lg), _stream(x)),
          "moe_router_logits")
    return lg


def fused_moe_router(x, router_w, w1, w2, topk: int, renormalize: bool = True, x_scale=None, w1_scale=None,
                     w2_scale=None, workspace=None, out=None, logits=None, topk_ids=None, topk_weights=None):
    """The whole layer from the hidden states: router scores on the GPU (written
    to `logits`, float32 [M, E]), then route -> align -> experts -> combine.
    Returns (out, logits)."""
    M, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    dt = moe_dtype(w1)
    need = fused_moe_workspace_size(dt, M, E, topk, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=_INTER[dt], device=x.device)
    if logits is None:
        logits = torch.empty((M, E), dtype=torch.float32, device=x.device)
    check(lib().fused_moe_router(dt, _p(x), _p(x_scale), _p(router_w), _p(logits), _p(w1), _p(w1_scale), _p(w2),
                                 _p(w2_scale), M, E, topk, H, I, int(renormalize), _p(out), _p(topk_ids),
                                 _p(topk_weights), _p(workspace), workspace.numel(), _stream(x)), "fused_moe_router")
    return out, logits

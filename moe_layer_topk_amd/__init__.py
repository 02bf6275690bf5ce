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
    MOE_ERR_UNSUPPORTED,
    MOE_W4A16,
    MOE_BF16,
    MOE_F32,
    MOE_FP8_E4M3,
    MOE_GEMM_DOWN,
    MOE_GEMM_DOWN_E4M3_ACT,
    MOE_GEMM_GATE_UP_SILU,
    AlignBufs,
    ExpertWeights,
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


class ExpertCache:
    """Expert streaming (the MoE inference post, FusedMoE vs MegaMoE, sections
    4.1-4.3): the experts' weights stay in pinned host memory and a GPU pool of
    `capacity` slots holds the ones in use.  Calling the cache runs the layer
    (fused_moe_cached): route, copy in the missing experts (least recently
    used slot first), then the fused layer over the slots.  prefetch() copies
    experts ahead of a call on the cache's own copy stream.

    w1, w2 (and the scales of fp8 or W4A16 weights) are the layer's weights
    in fused_moe's layout, on the host; they are copied once into pinned
    memory unless already pinned."""

    def __init__(self, w1, w2, capacity: int, w1_scale=None, w2_scale=None, device=None, copy_stream=None):
        self.dtype = moe_dtype(w1)
        self.E, twoI = w1.shape[0], w1.shape[1]
        self.I, self.H, self.capacity = twoI // 2, w2.shape[1], capacity
        device = torch.device("cuda" if device is None else device)
        self.device = device if device.index is not None else torch.device("cuda", torch.cuda.current_device())
        parts = (w1, w2, w1_scale, w2_scale)
        if any(t is not None and t.is_cuda for t in parts):
            raise ValueError("ExpertCache takes the experts' weights on the host")
        self.host = [None if t is None else (t.contiguous() if t.is_pinned() else t.contiguous().pin_memory())
                     for t in parts]
        self.slots = [None if t is None else torch.empty((capacity,) + tuple(t.shape[1:]), dtype=t.dtype,
                                                         device=self.device) for t in parts]
        # default priority: copies overlap compute through events, not priorities
        self.copy_stream = copy_stream if copy_stream is not None else torch.cuda.Stream(self.device)
        self._host_ids = torch.empty(0, dtype=torch.int32, pin_memory=True)
        self._ws = None
        h = ctypes.c_void_p()
        check(lib().moe_cache_create(self.dtype, self.E, self.H, self.I, capacity, ExpertWeights(*map(_p, self.host)),
                                     ExpertWeights(*map(_p, self.slots)), ctypes.c_void_p(self.copy_stream.cuda_stream),
                                     ctypes.byref(h)), "moe_cache_create")
        self._h = h

    def prefetch(self, experts) -> None:
        ids = torch.as_tensor(list(experts), dtype=torch.int32)
        check(lib().moe_cache_prefetch(self._h, _p(ids), ids.numel()), "moe_cache_prefetch")

    def stats(self) -> dict:
        v = [ctypes.c_int64() for _ in range(4)]
        check(lib().moe_cache_stats(self._h, *map(ctypes.byref, v)), "moe_cache_stats")
        return dict(zip(("hits", "misses", "prefetched", "h2d_bytes"), (x.value for x in v)))

    def __call__(self, x, router_logits, topk: int, renormalize: bool = True, x_scale=None, workspace=None,
                 out=None, topk_ids=None, topk_weights=None):
        """The layer over the cache; returns out[M,H] as fused_moe does."""
        M = x.shape[0]
        if self._host_ids.numel() < M * topk:
            # the previous call's copy from the old buffer may still be queued
            torch.cuda.current_stream(x.device).synchronize()
            self._host_ids = torch.empty(M * topk, dtype=torch.int32, pin_memory=True)
        if workspace is None:
            need = max(fused_moe_workspace_size(self.dtype, M, self.capacity, topk, self.H, self.I), 1)
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(need, dtype=torch.uint8, device=x.device)
            workspace = self._ws
        if out is None:
            out = torch.empty((M, self.H), dtype=_INTER[self.dtype], device=x.device)
        check(lib().fused_moe_cached(self._h, _p(x), _p(x_scale), _p(router_logits), M, topk, int(renormalize),
                                     _p(out), _p(topk_ids), _p(topk_weights), _p(self._host_ids), _p(workspace),
                                     workspace.numel(), _stream(x)), "fused_moe_cached")
        return out

    def close(self) -> None:
        if getattr(self, "_h", None):
            check(lib().moe_cache_destroy(self._h), "moe_cache_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

"""ctypes loader for libmoe.so (the C ABI declared in include/moe.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

(MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_ALIGNMENT, MOE_ERR_HIP,
 MOE_ERR_SCRATCH) = range(8)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_W4A16 = 0, 1, 2, 3
MOE_GEMM_GATE_UP_SILU, MOE_GEMM_DOWN, MOE_GEMM_DOWN_E4M3_ACT = 0, 1, 2


class AlignBufs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("sorted_ids", "tile_expert", "expert_counts", "expert_offsets", "active_experts", "num_active")]


class ExpertWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w2", "w1_scale", "w2_scale")]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lib = None

# exported symbol -> (restype, argtypes)
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "moe_route": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_align_capacity": (_I64, [_I32, _I32, _I32, _I32]),
    "moe_align": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, AlignBufs, _P]),
    "moe_grouped_gemm": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, ctypes.POINTER(AlignBufs),
                                        _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_quant_act": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "moe_combine": (ctypes.c_int, [ctypes.c_int, _P, _P, _I32, _I32, _I32, ctypes.c_int, _P, _P]),
    "fused_moe_workspace_size": (_SZ, [ctypes.c_int, _I32, _I32, _I32, _I32, _I32]),
    "fused_moe": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                 _P, _P, _P, _P, _SZ, _P]),
    "moe_router_logits": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "fused_moe_router": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                        _I32, _P, _P, _P, _P, _SZ, _P]),
    "fused_moe_noalloc": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                         _I32, _P, _P, _P, _P]),
    "fused_moe_noalloc_scratch_bytes": (_SZ, []),
    "moe_cache_create": (ctypes.c_int, [ctypes.c_int, _I32, _I32, _I32, _I32, ExpertWeights, ExpertWeights, _P,
                                        ctypes.POINTER(_P)]),
    "moe_cache_destroy": (ctypes.c_int, [_P]),
    "moe_cache_prefetch": (ctypes.c_int, [_P, _P, _I32]),
    "moe_cache_stats": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "fused_moe_cached": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
}


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m moe_layer_topk_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().moe_status_str(s).decode()


def check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, what)

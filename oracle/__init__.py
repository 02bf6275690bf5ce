"""CPU oracle for the fused top-k MoE layer (Python side).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the benchmark's CPU-baseline leg, never by the product path.  The arithmetic
lives in moe_oracle.c (float64, one token at a time); this module only
marshals arrays into it.  It shares nothing with the HIP library.

Each function follows the pages as cited in moe_oracle.c: routing and
weighted sum (FusedMoE vs MegaMoE post, sections 2 and 3.1), the sort and
index system (section 3.1, steps 1-2), the per-expert contraction
(MoE kernel engineering post, Eq. 1) and per-tensor FP8 scaling (its FP8
backend-routing section).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

OR_F32, OR_BF16, OR_FP8, OR_W4A16 = 0, 1, 2, 3
_DT = {"f32": OR_F32, "bf16": OR_BF16, "fp8": OR_FP8, "w4a16": OR_W4A16}


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc: -O3, OpenMP, no -ffast-math and no FMA
    contraction (every product and sum rounds as written).  The target is
    x86-64-v3 (AVX2/FMA) rather than -march=native: the library is built once
    and also runs on other hosts, whose CPU may lack what this one has."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp",
             "-fno-fast-math", "-std=c11",
             "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sig = {
            "oracle_bf16_decode": (dbl, [ctypes.c_uint16]),
            "oracle_e4m3_decode": (dbl, [ctypes.c_uint8]),
            "oracle_e4m3_encode": (ctypes.c_uint8, [dbl]),
            "oracle_int4_weight": (dbl, [P, P, i64, i64, i64, i64]),
            "oracle_num_threads": (i32, []),
            "oracle_route": (i32, [P, i64, i32, i32, i32, P, P]),
            "oracle_align_capacity": (i64, [i64, i32, i32, i32]),
            "oracle_align": (i32, [P, i64, i32, i32, i32, i64, P, P, P, P, P, P]),
            "oracle_act_amax": (i32, [i32, P, P, P, P, P, i64, i32, i32, i64, i64, i32, P]),
            "oracle_act_amax_per_token": (i32, [i32, P, P, P, P, P, i64, i32, i32, i64, i64, i32, P]),
            "oracle_moe": (i32, [i32, P, P, P, P, P, P, P, i64, i32, i32, i64, i64, i32, dbl, P, i64, P]),
            "oracle_pairs_gate_up": (i32, [i32, P, P, P, i64, i32, P, P, i32, i64, i64, P, i64, P]),
            "oracle_pairs_down": (i32, [i32, i32, P, dbl, P, i64, P, P, i32, i64, i64, P, i64, P]),
            "oracle_combine": (i32, [i32, P, P, i64, i32, i64, P]),
            "oracle_router_logits": (i32, [i32, P, P, P, i64, i32, i64, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


# ----------------------------------------------------------------- helpers

def _np(a):
    """torch tensor or ndarray -> C-contiguous host ndarray of its storage bytes."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            t = a.detach().to("cpu").contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype == torch.float8_e4m3fn:
                return t.view(torch.uint8).numpy()
            return t.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return lib().oracle_num_threads()


# ---------------------------------------------------------------- codecs

def bf16_decode(bits: int) -> float:
    return lib().oracle_bf16_decode(bits)


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(float(v))


# ----------------------------------------------------------------- steps

def route(logits, topk: int, renormalize: bool = True):
    """-> (ids int32 [M,k], weights float64 [M,k])."""
    lg = np.ascontiguousarray(_np(logits), dtype=np.float32)
    M, E = lg.shape
    ids = np.empty((M, topk), np.int32)
    w = np.empty((M, topk), np.float64)
    _check(lib().oracle_route(_ptr(lg), M, E, topk, int(renormalize), _ptr(ids), _ptr(w)), "route")
    return ids, w


def router_logits(dtype, x, x_scale, wg):
    """float64 [M, E] = x . wg^T (wg float32 [E, H]; x stored as dtype, times x_scale)."""
    xn = _np(x)
    wgn = np.ascontiguousarray(_np(wg), np.float32)
    M, H = xn.shape
    E = wgn.shape[0]
    out = np.empty((M, E), np.float64)
    _check(lib().oracle_router_logits(_DT[dtype], _ptr(xn), _ptr(_f32(x_scale)), _ptr(wgn), M, E, H, _ptr(out)),
           "router_logits")
    return out


def align_capacity(M: int, topk: int, E: int, block_m: int) -> int:
    return lib().oracle_align_capacity(M, topk, E, block_m)


def align(ids, E: int, block_m: int) -> dict:
    """Stable per-pair counting sort by expert with block_m padding."""
    ids = np.ascontiguousarray(_np(ids), dtype=np.int32)
    M, k = ids.shape
    cap = align_capacity(M, k, E, block_m)
    nact = min(E, M * k)
    out = {
        "expert_counts": np.empty(E, np.int32),
        "expert_offsets": np.empty(E + 1, np.int32),
        "sorted_ids": np.empty(cap, np.int32),
        "tile_expert": np.empty(cap // block_m, np.int32),
        "active_experts": np.empty(max(nact, 1), np.int32)[:nact],
        "num_active": np.zeros(1, np.int32),
    }
    _check(lib().oracle_align(_ptr(ids), M, k, E, block_m, cap, _ptr(out["expert_counts"]),
                              _ptr(out["expert_offsets"]), _ptr(out["sorted_ids"]),
                              _ptr(out["tile_expert"]), _ptr(out["active_experts"]),
                              _ptr(out["num_active"])), "align")
    return out


def _f32(a):
    return None if a is None else np.ascontiguousarray(_np(a), dtype=np.float32).reshape(-1)


def act_amax(dtype, x, x_scale, logits, w1, w1_scale, topk, renormalize=True) -> float:
    xn, lg, w1n = _np(x), np.ascontiguousarray(_np(logits), np.float32), _np(w1)
    M, H = xn.shape
    E, twoI, _ = w1n.shape
    out = np.zeros(1, np.float64)
    _check(lib().oracle_act_amax(_DT[dtype], _ptr(xn), _ptr(_f32(x_scale)), _ptr(lg), _ptr(w1n),
                                 _ptr(_f32(w1_scale)), M, E, topk, H, twoI // 2, int(renormalize),
                                 _ptr(out)), "act_amax")
    return float(out[0])


def act_amax_per_token(dtype, x, x_scale, logits, w1, w1_scale, topk, renormalize=True):
    """float64 [M]: largest |intermediate| over each token's pairs."""
    xn, lg, w1n = _np(x), np.ascontiguousarray(_np(logits), np.float32), _np(w1)
    M, H = xn.shape
    E, twoI, _ = w1n.shape
    out = np.zeros(M, np.float64)
    _check(lib().oracle_act_amax_per_token(_DT[dtype], _ptr(xn), _ptr(_f32(x_scale)), _ptr(lg), _ptr(w1n),
                                           _ptr(_f32(w1_scale)), M, E, topk, H, twoI // 2, int(renormalize),
                                           _ptr(out)), "act_amax_per_token")
    return out


def moe_layer(dtype, x, x_scale, logits, w1, w1_scale, w2, w2_scale, topk, renormalize=True,
              tokens=None, act_amax_value=None):
    """Layer output in float64 for the listed tokens (all tokens by default)."""
    xn, lg, w1n, w2n = _np(x), np.ascontiguousarray(_np(logits), np.float32), _np(w1), _np(w2)
    M, H = xn.shape
    E, twoI, _ = w1n.shape
    I = twoI // 2
    tok = np.arange(M, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    if dtype == "fp8" and act_amax_value is None:
        act_amax_value = act_amax(dtype, x, x_scale, logits, w1, w1_scale, topk, renormalize)
    out = np.empty((len(tok), H), np.float64)
    _check(lib().oracle_moe(_DT[dtype], _ptr(xn), _ptr(_f32(x_scale)), _ptr(lg), _ptr(w1n),
                            _ptr(_f32(w1_scale)), _ptr(w2n), _ptr(_f32(w2_scale)), M, E, topk, H, I,
                            int(renormalize), float(act_amax_value or 0.0), _ptr(tok), len(tok),
                            _ptr(out)), "moe")
    return out


def int4_weight(codes, gscale, n, k):
    """W[n][k] of one expert's packed int4 matrix codes [N][K/2] with group scales [K/128][N]."""
    cn = np.ascontiguousarray(_np(codes), np.uint8)
    gs = np.ascontiguousarray(_np(gscale), np.float32)
    N, K = cn.shape[0], cn.shape[1] * 2
    return lib().oracle_int4_weight(_ptr(cn), _ptr(gs), N, K, n, k)


def pairs_gate_up(dtype, x, x_scale, ids, w1, w1_scale, pairs):
    """act rows (float64 [n, I]) for the listed pairs p (token p//k, expert ids.flat[p])."""
    xn, w1n = _np(x), _np(w1)
    idn = np.ascontiguousarray(_np(ids), np.int32)
    M, k = idn.shape
    E, twoI = w1n.shape[:2]
    H = xn.shape[1]
    pr = np.ascontiguousarray(pairs, np.int64)
    act = np.empty((len(pr), twoI // 2), np.float64)
    _check(lib().oracle_pairs_gate_up(_DT[dtype], _ptr(xn), _ptr(_f32(x_scale)), _ptr(idn), M, k,
                                      _ptr(w1n), _ptr(_f32(w1_scale)), E, H, twoI // 2, _ptr(pr),
                                      len(pr), _ptr(act)), "pairs_gate_up")
    return act


def pairs_down(dtype, act, ids, w2, w2_scale, pairs, act_amax_value=0.0):
    """y rows (float64 [n, H]) for the listed pairs from stored act rows (f32 or bf16)."""
    import torch
    adt = OR_BF16 if (isinstance(act, torch.Tensor) and act.dtype == torch.bfloat16) else OR_F32
    an, w2n = _np(act), _np(w2)
    idn = np.ascontiguousarray(_np(ids), np.int32).reshape(-1)
    E, H = w2n.shape[:2]
    I = an.shape[1]
    pr = np.ascontiguousarray(pairs, np.int64)
    y = np.empty((len(pr), H), np.float64)
    _check(lib().oracle_pairs_down(_DT[dtype], adt, _ptr(an), float(act_amax_value), _ptr(idn),
                                   len(idn), _ptr(w2n), _ptr(_f32(w2_scale)), E, H, I, _ptr(pr),
                                   len(pr), _ptr(y)), "pairs_down")
    return y


def combine(y, weights, topk):
    import torch
    ydt = OR_BF16 if (isinstance(y, torch.Tensor) and y.dtype == torch.bfloat16) else OR_F32
    yn = _np(y)
    wn = np.ascontiguousarray(_np(weights), np.float32)
    P, H = yn.shape
    M = P // topk
    out = np.empty((M, H), np.float64)
    _check(lib().oracle_combine(ydt, _ptr(yn), _ptr(wn), M, topk, H, _ptr(out)), "combine")
    return out

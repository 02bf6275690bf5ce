"""The C ABI on the host: the library loads, exports what include/moe.h
declares, and rejects bad arguments before touching HIP (no GPU needed)."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from moe_layer_topk_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from moe_layer_topk_amd import build
        build.build()
    return _lib.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, re.M))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert {"moe_route", "moe_align", "moe_grouped_gemm", "moe_combine", "fused_moe", "moe_align_capacity",
            "fused_moe_workspace_size", "moe_status_str"} <= names
    for n in names:
        assert hasattr(L, n), n
    from moe_layer_topk_amd._lib import SIGNATURES
    assert set(SIGNATURES) == names


def test_status_strings(L):
    for s in range(8):
        assert L.moe_status_str(s)
    assert L.moe_status_str(0) == b"ok"


def test_align_capacity_matches_oracle(L):
    for M, k, E, bm in [(1, 2, 8, 16), (64, 2, 8, 16), (4096, 2, 8, 128), (2048, 8, 128, 64), (512, 8, 64, 128),
                        (0, 2, 8, 16), (3, 8, 128, 1), (7, 3, 5, 256)]:
        assert L.moe_align_capacity(M, k, E, bm) == oracle.align_capacity(M, k, E, bm)
    assert L.moe_align_capacity(-1, 2, 8, 16) == -1
    assert L.moe_align_capacity(4, 2, 8, 0) == -1


NULL = None
FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first
ODD = ctypes.c_void_p(0x10004)


def test_route_validation(L):
    assert L.moe_route(FAKE, -1, 8, 2, 1, FAKE, FAKE, NULL) == 2
    assert L.moe_route(FAKE, 4, 8, 9, 1, FAKE, FAKE, NULL) == 2
    assert L.moe_route(FAKE, 4, 8, 0, 1, FAKE, FAKE, NULL) == 2
    assert L.moe_route(FAKE, 4, 0, 1, 1, FAKE, FAKE, NULL) == 2
    assert L.moe_route(FAKE, 4, 300, 2, 1, FAKE, FAKE, NULL) == 3
    assert L.moe_route(FAKE, 4, 64, 17, 1, FAKE, FAKE, NULL) == 3
    assert L.moe_route(NULL, 4, 8, 2, 1, FAKE, FAKE, NULL) == 1
    assert L.moe_route(FAKE, 4, 8, 2, 1, NULL, FAKE, NULL) == 1
    assert L.moe_route(ODD, 4, 8, 2, 1, FAKE, FAKE, NULL) == 5
    assert L.moe_route(NULL, 0, 8, 2, 1, NULL, NULL, NULL) == 0  # M = 0: no-op


def test_align_validation(L):
    from moe_layer_topk_amd._lib import AlignBufs
    ok = AlignBufs(*(0x10000,) * 6)
    assert L.moe_align(FAKE, 4, 2, 8, 24, ok, NULL) == 3
    assert L.moe_align(FAKE, 4, 9, 8, 16, ok, NULL) == 2
    assert L.moe_align(NULL, 4, 2, 8, 16, ok, NULL) == 1
    bad = AlignBufs(0x10000, 0, 0x10000, 0x10000, 0x10000, 0x10000)
    assert L.moe_align(FAKE, 4, 2, 8, 16, bad, NULL) == 1
    odd = AlignBufs(0x10000, 0x10004, 0x10000, 0x10000, 0x10000, 0x10000)
    assert L.moe_align(FAKE, 4, 2, 8, 16, odd, NULL) == 5
    assert L.moe_align(NULL, 0, 2, 8, 16, AlignBufs(), NULL) == 0


def test_gemm_validation(L):
    from moe_layer_topk_amd._lib import AlignBufs
    al = AlignBufs(*(0x10000,) * 6)
    bal = ctypes.byref(al)
    g = L.moe_grouped_gemm
    assert g(5, 1, FAKE, NULL, FAKE, NULL, bal, 4, 2, 8, 1024, 256, 16, FAKE, NULL, NULL) == 3
    assert g(0, 7, FAKE, NULL, FAKE, NULL, bal, 4, 2, 8, 1024, 256, 16, FAKE, NULL, NULL) == 3
    assert g(0, 1, FAKE, NULL, FAKE, NULL, bal, 4, 2, 8, 1000, 256, 16, FAKE, NULL, NULL) == 2
    assert g(0, 1, FAKE, NULL, FAKE, NULL, bal, 4, 2, 8, 384, 256, 16, FAKE, NULL, NULL) == 2  # I = 192
    assert g(1, 1, FAKE, NULL, FAKE, NULL, bal, 4, 2, 8, 384, 200, 16, FAKE, NULL, NULL) == 2
    assert g(1, 1, FAKE, NULL, FAKE, NULL, bal, 4, 2, 8, 384, 256, 48, FAKE, NULL, NULL) == 3
    assert g(1, 1, FAKE, FAKE, FAKE, NULL, bal, 4, 2, 8, 384, 256, 16, FAKE, NULL, NULL) == 3  # scale on bf16
    assert g(1, 1, NULL, NULL, FAKE, NULL, bal, 4, 2, 8, 384, 256, 16, FAKE, NULL, NULL) == 1
    assert g(1, 1, FAKE, NULL, FAKE, NULL, None, 4, 2, 8, 384, 256, 16, FAKE, NULL, NULL) == 1
    assert g(1, 2, FAKE, NULL, FAKE, FAKE, bal, 4, 2, 8, 384, 256, 16, FAKE, NULL, NULL) == 1  # fp8 needs a_scale
    assert g(0, 2, FAKE, FAKE, FAKE, FAKE, bal, 4, 2, 8, 512, 256, 16, FAKE, NULL, NULL) == 1  # fp8 needs amax
    assert g(1, 1, ODD, NULL, FAKE, NULL, bal, 4, 2, 8, 384, 256, 16, FAKE, NULL, NULL) == 5
    assert g(1, 1, NULL, NULL, NULL, NULL, None, 0, 2, 8, 384, 256, 16, NULL, NULL, NULL) == 0


def test_combine_validation(L):
    c = L.moe_combine
    assert c(2, FAKE, FAKE, 4, 2, 256, 1, FAKE, NULL) == 3
    assert c(1, FAKE, FAKE, 4, 2, 252, 1, FAKE, NULL) == 2
    assert c(1, FAKE, FAKE, 4, 0, 256, 1, FAKE, NULL) == 2
    assert c(1, NULL, FAKE, 4, 2, 256, 1, FAKE, NULL) == 1
    assert c(1, FAKE, FAKE, 4, 2, 256, 1, ODD, NULL) == 5
    assert c(1, NULL, NULL, 0, 2, 256, 1, NULL, NULL) == 0


def test_fused_validation_and_workspace(L):
    f = L.fused_moe
    sz = L.fused_moe_workspace_size(1, 64, 8, 2, 4096, 14336)
    P = 128
    assert sz >= P * 14336 * 2 + P * 4096 * 2  # act and y rows at least
    assert L.fused_moe_workspace_size(1, 0, 8, 2, 4096, 14336) == 0
    assert L.fused_moe_workspace_size(2, 32, 64, 8, 4096, 8192) > 0
    args = [FAKE, NULL, FAKE, FAKE, NULL, FAKE, NULL]
    assert f(1, *args, 64, 8, 2, 4096, 14336, 1, FAKE, NULL, NULL, FAKE, sz - 1, NULL) == 4
    assert f(1, *args, 64, 8, 2, 4000, 14336, 1, FAKE, NULL, NULL, FAKE, sz, NULL) == 2
    assert f(1, *args, 64, 8, 9, 4096, 14336, 1, FAKE, NULL, NULL, FAKE, sz, NULL) == 2
    assert f(1, *args, 64, 8, 2, 4096, 14336, 1, NULL, NULL, NULL, FAKE, sz, NULL) == 1
    assert f(1, *args, 64, 8, 2, 4096, 14336, 1, FAKE, NULL, NULL, ctypes.c_void_p(0x10010), sz, NULL) == 5
    fp8 = [FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert f(2, *fp8, 4, 64, 8, 4096, 8192, 1, FAKE, NULL, NULL, FAKE, 1 << 40, NULL) == 1  # x_scale missing
    assert f(1, *fp8, 4, 64, 8, 4096, 8192, 1, FAKE, NULL, NULL, FAKE, 1 << 40, NULL) == 3  # scales on bf16
    assert f(1, *args, 0, 8, 2, 4096, 14336, 1, FAKE, NULL, NULL, FAKE, 0, NULL) == 0


def test_binding_refuses_cpu_tensors():
    import torch

    import moe_layer_topk_amd as moe
    with pytest.raises(ValueError):
        moe.moe_route(torch.zeros(4, 8), 2)


def test_quant_act_and_e4m3_down_validation(L):
    q = L.moe_quant_act
    assert q(FAKE, FAKE, 17, FAKE, NULL) == 2  # n not a multiple of 16
    assert q(FAKE, FAKE, -16, FAKE, NULL) == 2
    assert q(NULL, FAKE, 32, FAKE, NULL) == 1
    assert q(FAKE, NULL, 32, FAKE, NULL) == 1
    assert q(FAKE, FAKE, 32, ODD, NULL) == 5
    assert q(NULL, NULL, 0, NULL, NULL) == 0  # n = 0: no-op
    from moe_layer_topk_amd._lib import AlignBufs
    bal = ctypes.byref(AlignBufs(*(0x10000,) * 6))
    g = L.moe_grouped_gemm
    # the e4m3-intermediate DOWN kind exists for e4m3 weights only
    assert g(2, 1, FAKE, NULL, FAKE, NULL, bal, 4, 2, 8, 512, 256, 16, FAKE, NULL, NULL) == 3
    assert g(2, 2, FAKE, NULL, FAKE, FAKE, bal, 4, 2, 8, 512, 256, 16, FAKE, NULL, NULL) == 1  # needs the amax


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_fused_noalloc_validation(L):
    """fused_moe_noalloc checks its arguments like fused_moe and rejects sizes
    beyond its static scratch before any HIP call."""
    from moe_layer_topk_amd._lib import MOE_ERR_SCRATCH
    assert L.fused_moe_noalloc_scratch_bytes() == 64 << 20
    args = lambda dt, M, E, k, H, I: (dt, FAKE, None, FAKE, FAKE, None, FAKE, None, M, E, k, H, I, 1, FAKE, None,  # noqa
                                      None, NULL)
    # the 4096-token Mixtral-shaped bf16 layer needs ~280 MB of workspace
    assert L.fused_moe_workspace_size(1, 4096, 8, 2, 4096, 14336) > (64 << 20)
    assert L.fused_moe_noalloc(*args(1, 4096, 8, 2, 4096, 14336)) == MOE_ERR_SCRATCH
    assert L.fused_moe_noalloc(*args(1, 4, 8, 9, 256, 256)) == 2
    assert L.fused_moe_noalloc(*args(5, 4, 8, 2, 256, 256)) == 3
    assert L.fused_moe_noalloc(1, NULL, None, FAKE, FAKE, None, FAKE, None, 4, 8, 2, 256, 256, 1, FAKE, None, None,
                               NULL) == 1
    assert L.fused_moe_noalloc(1, ODD, None, FAKE, FAKE, None, FAKE, None, 4, 8, 2, 256, 256, 1, FAKE, None, None,
                               NULL) == 5
    assert L.fused_moe_noalloc(*args(1, 0, 8, 2, 256, 256)) == 0  # M = 0: no-op
    # every decode batch (up to 64 tokens) of every layer shape fits
    for dt, E, k, H, I in [(1, 8, 2, 4096, 14336), (1, 128, 8, 2048, 768), (2, 64, 8, 4096, 8192)]:
        assert L.fused_moe_workspace_size(dt, 64, E, k, H, I) <= (64 << 20)


def test_expert_cache_validation(L):
    """moe_cache_create rejects bad arguments before creating any HIP object;
    the other cache calls reject a NULL cache."""
    from moe_layer_topk_amd._lib import ExpertWeights
    out = ctypes.c_void_p()
    plain = ExpertWeights(FAKE, FAKE, None, None)
    scaled = ExpertWeights(FAKE, FAKE, FAKE, FAKE)
    create = L.moe_cache_create
    assert create(1, 8, 256, 256, 4, plain, plain, NULL, None) == 1  # no output handle
    assert create(1, 8, 256, 256, 9, plain, plain, NULL, ctypes.byref(out)) == 2  # capacity > E
    assert create(1, 8, 256, 256, 0, plain, plain, NULL, ctypes.byref(out)) == 2
    assert create(1, 8, 200, 256, 4, plain, plain, NULL, ctypes.byref(out)) == 2  # H % 128
    assert create(2, 8, 384, 256, 4, scaled, scaled, NULL, ctypes.byref(out)) == 2  # fp8: H % 256
    assert create(1, 300, 256, 256, 4, plain, plain, NULL, ctypes.byref(out)) == 3  # E > 256
    assert create(7, 8, 256, 256, 4, plain, plain, NULL, ctypes.byref(out)) == 3  # unknown dtype
    assert create(1, 8, 256, 256, 4, scaled, scaled, NULL, ctypes.byref(out)) == 3  # scales for bf16
    assert create(2, 8, 256, 256, 4, plain, plain, NULL, ctypes.byref(out)) == 1  # fp8 without scales
    assert create(3, 8, 256, 256, 4, scaled, ExpertWeights(ODD, FAKE, FAKE, FAKE), NULL,
                  ctypes.byref(out)) == 5  # misaligned slots
    assert out.value is None
    assert L.moe_cache_prefetch(NULL, NULL, 0) == 1
    assert L.moe_cache_stats(NULL, None, None, None, None) == 1
    assert L.fused_moe_cached(NULL, FAKE, None, FAKE, 1, 2, 1, FAKE, None, None, FAKE, FAKE, 1 << 20, NULL) == 1
    assert L.moe_cache_destroy(NULL) == 0

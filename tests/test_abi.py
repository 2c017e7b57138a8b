"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and validates arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from megatron_tensor_layer_amd import tplayer as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_layer.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tp.LIB_PATH), reason="libtplayer.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(tp.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = tp.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    # the exported symbols are plain C names (no C++ mangling)
    nm = os.popen(f"nm -D --defined-only {tp.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", nm, re.M), name


@pytest.mark.parametrize("args,expect", [
    ((64, 4, 32, 2, 4, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_OK),
    ((12288, 96, 2048, 1, 8, 7, tp.TP_BF16, tp.TP_MLP), tp.TP_OK),
    ((25600, 160, 2048, 1, 8, 3, tp.TP_BF16, tp.TP_ATTN), tp.TP_OK),
    ((2304, 24, 2048, 4, 1, 0, tp.TP_BF16, tp.TP_ATTN), tp.TP_OK),
    ((64, 4, 32, 2, 3, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_EINVAL),      # a % t != 0: heads must stay whole
    ((64, 5, 32, 2, 1, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_EINVAL),      # h % a != 0
    ((64, 4, 32, 2, 4, 4, tp.TP_FP32, tp.TP_ATTN), tp.TP_EINVAL),      # rank out of range
    ((64, 4, 32, 2, 4, -1, tp.TP_FP32, tp.TP_ATTN), tp.TP_EINVAL),
    ((64, 4, 0, 2, 4, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_EINVAL),
    ((64, 4, 32, 2, 4, 0, 7, tp.TP_ATTN), tp.TP_EINVAL),
    ((64, 4, 32, 2, 4, 0, tp.TP_FP32, 2), tp.TP_EINVAL),
    ((64, 4, 24, 2, 4, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_EUNSUPPORTED),  # s % 16
    ((96, 4, 32, 2, 4, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_EUNSUPPORTED),  # d = 24
    ((128, 8, 32, 2, 8, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_OK),           # d = 16, h/t = 16
    # every matrix below 2^31 elements (32-bit byte offsets in the tile loaders)
    ((32768, 256, 2048, 1, 1, 0, tp.TP_BF16, tp.TP_MLP), tp.TP_EUNSUPPORTED),   # W1 shard 32768 x 131072
    ((32768, 256, 2048, 1, 4, 0, tp.TP_BF16, tp.TP_MLP), tp.TP_OK),             # W1 shard 32768 x 32768
    ((16384, 128, 2048, 64, 8, 0, tp.TP_BF16, tp.TP_ATTN), tp.TP_EUNSUPPORTED),  # X: 131072 x 16384 = 2^31
    ((16384, 128, 2048, 32, 8, 0, tp.TP_BF16, tp.TP_ATTN), tp.TP_OK),            # X: 2^30
    ((4096, 32, 8192, 2, 8, 0, tp.TP_BF16, tp.TP_MLP), tp.TP_OK),
    ((4096, 32, 8192, 16, 1, 0, tp.TP_BF16, tp.TP_MLP), tp.TP_EUNSUPPORTED),    # U: 131072 x 16384
    # one [s, s] score matrix on the materialised path (fp32, or d = 48); none on the fused bf16 path
    ((1024, 8, 47104, 1, 1, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_EUNSUPPORTED),   # 47104^2 > 2^31
    ((1024, 8, 46336, 1, 1, 0, tp.TP_FP32, tp.TP_ATTN), tp.TP_OK),             # 46336^2 < 2^31
    ((1024, 8, 47104, 1, 1, 0, tp.TP_BF16, tp.TP_ATTN), tp.TP_OK),             # d = 128: fused, no s x s
    ((768, 16, 47104, 1, 1, 0, tp.TP_BF16, tp.TP_ATTN), tp.TP_EUNSUPPORTED),   # d = 48: materialised
])
def test_check_args(args, expect):
    assert tp.tp_check_args(*args) == expect


def test_saved_and_workspace_sizes():
    h, a, s, b, t = 12288, 96, 2048, 1, 8
    T, ar, hr = s * b, a // t, h // t
    # bf16 with d = 128 runs the fused flash kernels: the attention block keeps
    # QKV, the Q/K rounding residuals, C in bf16 and fp32 and one log-sum-exp
    # per query, and neither it nor its workspace holds any s x s matrix
    sa = tp.tp_saved_bytes(h, a, s, b, t, tp.TP_BF16, tp.TP_ATTN)
    assert sa >= 2 * (T * 3 * hr + T * 2 * hr + T * hr) + 4 * T * hr + 4 * b * ar * s
    assert sa < 2 * b * ar * s * s
    assert tp.tp_workspace_bytes(h, a, s, b, t, tp.TP_BF16, tp.TP_ATTN) < 4 * b * ar * s * s  # no fp32 scores
    sm = tp.tp_saved_bytes(h, a, s, b, t, tp.TP_BF16, tp.TP_MLP)
    assert sm >= 2 * 2 * T * 4 * h // t
    # fp32, and bf16 with a head width the flash kernels are not built for
    # (d = 48), materialise P (saved) and the fp32 scores (workspace)
    for dt, es, a2 in ((tp.TP_FP32, 4, a), (tp.TP_BF16, 2, 256)):
        ar2 = a2 // t
        sa2 = tp.tp_saved_bytes(h, a2, s, b, t, dt, tp.TP_ATTN)
        assert sa2 >= es * (T * 3 * hr + b * ar2 * s * s + T * hr)
        assert tp.tp_workspace_bytes(h, a2, s, b, t, dt, tp.TP_ATTN) >= 4 * b * ar2 * s * s
    assert tp.tp_saved_bytes(h, a, s, b, 5, tp.TP_BF16, tp.TP_ATTN) == 0  # a % t != 0 -> 0


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_fwd_rejects_null_misaligned_and_small_workspace_on_host():
    L = tp.lib()
    dims = (64, 4, 32, 2, 4, 0, tp.TP_FP32, tp.TP_ATTN)
    ok = tp.TPBlockWeights(0x10000, 0x20000, 0x30000, 0x40000)
    none = ctypes.c_void_p(None)
    a = _fake(0x100000)
    ws_need = tp.tp_workspace_bytes(64, 4, 32, 2, 4, tp.TP_FP32, tp.TP_ATTN)
    # NULL input
    assert L.tp_layer_fwd(*dims, none, ctypes.byref(ok), a, a, a, ws_need, none) == tp.TP_ENULL
    # NULL weight pointer
    bad = tp.TPBlockWeights(0x10000, None, 0x30000, 0x40000)
    assert L.tp_layer_fwd(*dims, a, ctypes.byref(bad), a, a, a, ws_need, none) == tp.TP_ENULL
    # misaligned
    assert L.tp_layer_fwd(*dims, _fake(0x100004), ctypes.byref(ok), a, a, a, ws_need, none) == tp.TP_EALIGN
    # workspace too small
    assert L.tp_layer_fwd(*dims, a, ctypes.byref(ok), a, a, a, ws_need - 1, none) == tp.TP_EWORKSPACE
    # invalid dims come first
    assert L.tp_layer_fwd(64, 4, 32, 2, 3, 0, tp.TP_FP32, tp.TP_ATTN, none, None, none, none, none, 0,
                          none) == tp.TP_EINVAL


def test_bwd_rejects_null_grads_on_host():
    L = tp.lib()
    dims = (64, 4, 32, 2, 4, 1, tp.TP_FP32, tp.TP_MLP)
    ok = tp.TPBlockWeights(0x10000, 0x20000, 0x30000, 0x40000)
    g = tp.TPBlockGrads(0x50000, 0x60000, None, 0x80000)
    a = _fake(0x100000)
    ws = tp.tp_workspace_bytes(64, 4, 32, 2, 4, tp.TP_FP32, tp.TP_MLP)
    assert L.tp_layer_bwd(*dims, a, ctypes.byref(ok), a, a, a, ctypes.byref(g), a, ws, None) == tp.TP_ENULL


def test_reduce_and_gemm_validation_on_host():
    L = tp.lib()
    a = _fake(0x100000)
    none = ctypes.c_void_p(None)
    assert L.tp_reduce_partials(tp.TP_BF16, 4, 12, 2, a, none, none, a, None) == tp.TP_EINVAL   # cols % 8
    assert L.tp_reduce_partials(tp.TP_BF16, 4, 16, 2, none, none, none, a, None) == tp.TP_ENULL
    assert L.tp_reduce_partials(tp.TP_BF16, 4, 16, 2, _fake(0x100002), none, none, a, None) == tp.TP_EALIGN
    assert L.tp_reduce_partials(tp.TP_BF16, 4, 16, 2, a, _fake(0x100008), none, a, None) == tp.TP_EALIGN
    assert L.tp_gemm(tp.TP_BF16, 20, 16, 16, 1.0, a, 16, 1, a, 16, 1, None, a, 16, None, 0, None) == tp.TP_EUNSUPPORTED
    assert L.tp_gemm(tp.TP_BF16, 16, 16, 32, 1.0, a, 16, 1, a, 32, 1, None, a, 16, None, 0, None) == tp.TP_EINVAL
    # operands and output below 2^31 elements: rows x leading dimension
    big = 1 << 16
    assert L.tp_gemm(tp.TP_BF16, big, 64, 32768, 1.0, a, 32768, 1, a, 64, 0, None, a, 64, None, 0,
                     None) == tp.TP_EUNSUPPORTED                                  # A [65536, 32768]
    assert L.tp_gemm(tp.TP_BF16, 64, big, 32768, 1.0, a, 32768, 1, a, 32768, 1, None, a, big, None, 0,
                     None) == tp.TP_EUNSUPPORTED                                  # B [65536, 32768]
    assert L.tp_gemm(tp.TP_BF16, 64, 64, big, 1.0, a, 32768, 0, a, 64, 0, None, a, 64, None, 0,
                     None) == tp.TP_EUNSUPPORTED                                  # A stored [K=65536, 32768]
    assert L.tp_gemm(tp.TP_BF16, big, 32768, 64, 1.0, a, 64, 1, a, 32768, 0, None, a, 32768, None, 0,
                     None) == tp.TP_EUNSUPPORTED                                  # C [65536, 32768]
    # stream-K over the partial wave behind a whole one needs fp32 fragment slots (384 tiles: 128 tiles in
    # 2 pieces each): workspace checked before any launch
    M, N, K = 2048, 12288, 6144
    need = tp.tp_gemm_workspace_bytes(tp.TP_BF16, M, N, K)
    assert need >= 128 * 2 * 256 * 256 * 4
    # fewer than 160 tiles (and at least 128) run as one partial wave of whole tiles and need none
    assert tp.tp_gemm_workspace_bytes(tp.TP_BF16, 2048, 4608, 12288) == 0
    assert L.tp_gemm(tp.TP_BF16, M, N, K, 1.0, a, K, 1, a, N, 0, None, a, N, a, need - 256, None) == tp.TP_EWORKSPACE
    assert L.tp_gemm(tp.TP_BF16, M, N, K, 1.0, a, K, 1, a, N, 0, None, a, N, none, need, None) == tp.TP_ENULL
    # small problems need none; fp32 never does
    assert tp.tp_gemm_workspace_bytes(tp.TP_BF16, 256, 256, 256) == 0
    assert tp.tp_gemm_workspace_bytes(tp.TP_FP32, M, N, K) == 0
    assert tp.tp_gemm_workspace_bytes(tp.TP_BF16, 0, N, K) == 0


def test_profiler_without_gpu_work():
    tp.tp_prof_enable(True)
    assert tp.tp_prof_read() == {}
    tp.tp_prof_enable(False)


def test_noalloc_validation_on_host():
    """tp_layer_bwd_noalloc checks its arguments and the scratch it needs
    before any HIP call."""
    L = tp.lib()
    assert tp.tp_noalloc_scratch_bytes() == 256 << 20
    W = tp.TPBlockWeights(0x10000, 0x20000, 0x30000, 0x40000)
    G = tp.TPBlockGrads(0x50000, 0x60000, 0x70000, 0x80000)
    a = _fake(0x100000)
    # invalid dims first
    assert L.tp_layer_bwd_noalloc(64, 4, 32, 2, 3, 0, tp.TP_FP32, tp.TP_ATTN, a, ctypes.byref(W), a, a, a,
                                  ctypes.byref(G), None) == tp.TP_EINVAL
    # the 1.7B attention block needs more workspace than the static scratch holds
    assert tp.tp_workspace_bytes(2304, 24, 2048, 4, 1, tp.TP_BF16, tp.TP_ATTN) > tp.tp_noalloc_scratch_bytes()
    assert L.tp_layer_bwd_noalloc(2304, 24, 2048, 4, 1, 0, tp.TP_BF16, tp.TP_ATTN, a, ctypes.byref(W), a, a, a,
                                  ctypes.byref(G), None) == tp.TP_ESCRATCH
    # every benchmark shape of the 175B, 18B and 1T layers fits
    for h, a_, s, b, t in ((12288, 96, 2048, 1, 8), (6144, 48, 2048, 2, 8), (25600, 160, 2048, 1, 8)):
        for blk in (tp.TP_ATTN, tp.TP_MLP):
            assert tp.tp_workspace_bytes(h, a_, s, b, t, tp.TP_BF16, blk) <= tp.tp_noalloc_scratch_bytes()


def test_strerror():
    for code in (tp.TP_OK, tp.TP_EINVAL, tp.TP_EUNSUPPORTED, tp.TP_ENULL, tp.TP_EALIGN, tp.TP_EWORKSPACE, tp.TP_EHIP,
                 tp.TP_ESCRATCH):
        assert len(tp.strerror(code)) > 0
    assert "unknown" in tp.strerror(-99)


def test_layernorm_validation_on_host():
    L = tp.lib()
    a = _fake(0x100000)
    none = ctypes.c_void_p(None)
    BF, F32 = tp.TP_BF16, tp.TP_FP32
    f = L.tp_layernorm_fwd
    # dtype, sizes, eps
    assert f(7, 4, 64, 1e-5, a, none, none, a, a, none, a, a, None) == tp.TP_EINVAL
    assert f(BF, -1, 64, 1e-5, a, none, none, a, a, none, a, a, None) == tp.TP_EINVAL
    assert f(BF, 4, 0, 1e-5, a, none, none, a, a, none, a, a, None) == tp.TP_EINVAL
    assert f(BF, 4, 60, 1e-5, a, none, none, a, a, none, a, a, None) == tp.TP_EUNSUPPORTED  # h % 8
    assert f(BF, 4, 32776, 1e-5, a, none, none, a, a, none, a, a, None) == tp.TP_EUNSUPPORTED
    assert f(F32, 4, 16392, 1e-5, a, none, none, a, a, none, a, a, None) == tp.TP_EUNSUPPORTED
    assert f(BF, 4, 64, -1.0, a, none, none, a, a, none, a, a, None) == tp.TP_EINVAL
    assert f(BF, 4, 64, float("nan"), a, none, none, a, a, none, a, a, None) == tp.TP_EINVAL
    # required pointers: with gamma, beta + y + stats; without gamma, sum_out
    assert f(BF, 4, 64, 1e-5, none, none, none, a, a, none, a, a, None) == tp.TP_ENULL
    assert f(BF, 4, 64, 1e-5, a, none, none, a, none, none, a, a, None) == tp.TP_ENULL
    assert f(BF, 4, 64, 1e-5, a, none, none, a, a, none, a, none, None) == tp.TP_ENULL
    assert f(BF, 4, 64, 1e-5, a, a, a, none, none, none, none, none, None) == tp.TP_ENULL
    # alignment: 16 bytes, stats 8
    assert f(BF, 4, 64, 1e-5, _fake(0x100008), none, none, a, a, none, a, a, None) == tp.TP_EALIGN
    assert f(BF, 4, 64, 1e-5, a, none, none, a, a, none, a, _fake(0x100004), None) == tp.TP_EALIGN
    # zero rows: nothing to do, no pointer needed
    assert f(BF, 0, 64, 1e-5, none, none, none, none, none, none, none, none, None) == tp.TP_OK
    b = L.tp_layernorm_bwd
    assert b(BF, 4, 64, a, a, a, a, none, a, a, none, None) == tp.TP_ENULL            # dgamma without dbeta
    assert b(BF, 4, 64, none, a, a, a, none, a, none, none, None) == tp.TP_ENULL      # no dy
    assert b(BF, 4, 64, a, a, a, none, none, a, none, none, None) == tp.TP_ENULL      # no gamma
    assert b(BF, 4, 64, a, a, _fake(0x100004), a, none, a, none, none, None) == tp.TP_EALIGN
    assert b(BF, 4, 64, a, a, a, a, _fake(0x100002), a, none, none, None) == tp.TP_EALIGN
    assert b(BF, 4, 61, a, a, a, a, none, a, none, none, None) == tp.TP_EUNSUPPORTED
    assert b(BF, 0, 64, none, none, none, none, none, none, none, none, None) == tp.TP_OK


def test_recompute_validation_on_host():
    L = tp.lib()
    dims = (64, 4, 32, 2, 4, 1, tp.TP_FP32, tp.TP_MLP)
    ok = tp.TPBlockWeights(0x10000, 0x20000, 0x30000, 0x40000)
    g = tp.TPBlockGrads(0x50000, 0x60000, 0x70000, 0x80000)
    a = _fake(0x100000)
    none = ctypes.c_void_p(None)
    ws = tp.tp_workspace_bytes(64, 4, 32, 2, 4, tp.TP_FP32, tp.TP_MLP)
    f = L.tp_layer_bwd_recompute
    assert f(*dims, a, ctypes.byref(ok), a, a, ctypes.byref(g), none, a, ws, None) == tp.TP_ENULL     # scratch
    assert f(*dims, a, ctypes.byref(ok), a, a, ctypes.byref(g), _fake(0x100008), a, ws, None) == tp.TP_EALIGN
    assert f(*dims, a, ctypes.byref(ok), a, a, ctypes.byref(g), a, a, ws - 1, None) == tp.TP_EWORKSPACE
    assert f(64, 4, 32, 2, 3, 0, tp.TP_FP32, tp.TP_MLP, a, ctypes.byref(ok), a, a, ctypes.byref(g), a, a, ws,
             None) == tp.TP_EINVAL

"""Thin ctypes binding of libtplayer (include/tp_layer.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
of the library.  Tensors are torch tensors on the GPU (PyTorch provides
device memory and streams); pointers, sizes and the current HIP stream are
passed through unchanged.  If the library has not been built, every entry
point raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

TP_BF16, TP_FP32 = 0, 1
TP_ATTN, TP_MLP = 0, 1

TP_OK = 0
TP_EINVAL, TP_EUNSUPPORTED, TP_ENULL, TP_EALIGN, TP_EWORKSPACE, TP_EHIP = -1, -2, -3, -4, -5, -6
TP_ESCRATCH = -7

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtplayer.so")

# every symbol include/tp_layer.h declares
EXPORTS = ("tp_check_args", "tp_saved_bytes", "tp_workspace_bytes", "tp_layer_fwd", "tp_layer_bwd",
           "tp_reduce_partials", "tp_layer_bwd_recompute", "tp_layernorm_fwd", "tp_layernorm_bwd",
           "tp_gemm_workspace_bytes", "tp_gemm", "tp_prof_enable", "tp_prof_read", "tp_strerror",
           "tp_noalloc_scratch_bytes", "tp_layer_bwd_noalloc")

_lib = None


class TPBlockWeights(ctypes.Structure):
    _fields_ = [("w_in", ctypes.c_void_p), ("b_in", ctypes.c_void_p),
                ("w_out", ctypes.c_void_p), ("b_out", ctypes.c_void_p)]


class TPBlockGrads(ctypes.Structure):
    _fields_ = [("dw_in", ctypes.c_void_p), ("db_in", ctypes.c_void_p),
                ("dw_out", ctypes.c_void_p), ("db_out", ctypes.c_void_p)]


class TPProfEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("launches", ctypes.c_int), ("ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class TPError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def lib():
    """Load libtplayer.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m megatron_tensor_layer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i, sz, vp, f32, lng = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_long
    dims = [i] * 8
    L.tp_check_args.argtypes, L.tp_check_args.restype = dims, i
    L.tp_saved_bytes.argtypes, L.tp_saved_bytes.restype = [i] * 7, sz
    L.tp_workspace_bytes.argtypes, L.tp_workspace_bytes.restype = [i] * 7, sz
    L.tp_layer_fwd.argtypes = dims + [vp, ctypes.POINTER(TPBlockWeights), vp, vp, vp, sz, vp]
    L.tp_layer_fwd.restype = i
    L.tp_layer_bwd.argtypes = dims + [vp, ctypes.POINTER(TPBlockWeights), vp, vp, vp,
                                      ctypes.POINTER(TPBlockGrads), vp, sz, vp]
    L.tp_layer_bwd.restype = i
    L.tp_noalloc_scratch_bytes.argtypes, L.tp_noalloc_scratch_bytes.restype = [], sz
    L.tp_layer_bwd_noalloc.argtypes = dims + [vp, ctypes.POINTER(TPBlockWeights), vp, vp, vp,
                                              ctypes.POINTER(TPBlockGrads), vp]
    L.tp_layer_bwd_noalloc.restype = i
    L.tp_reduce_partials.argtypes = [i, lng, lng, i, vp, vp, vp, vp, vp]
    L.tp_reduce_partials.restype = i
    L.tp_layer_bwd_recompute.argtypes = dims + [vp, ctypes.POINTER(TPBlockWeights), vp, vp,
                                                ctypes.POINTER(TPBlockGrads), vp, vp, sz, vp]
    L.tp_layer_bwd_recompute.restype = i
    L.tp_layernorm_fwd.argtypes = [i, lng, lng, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.tp_layernorm_fwd.restype = i
    L.tp_layernorm_bwd.argtypes = [i, lng, lng, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.tp_layernorm_bwd.restype = i
    L.tp_prof_enable.argtypes, L.tp_prof_enable.restype = [i], i
    L.tp_prof_read.argtypes, L.tp_prof_read.restype = [ctypes.POINTER(TPProfEntry), i], i
    L.tp_gemm_workspace_bytes.argtypes = [i, i, i, i]
    L.tp_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.tp_gemm.argtypes = [i, i, i, i, f32, vp, lng, i, vp, lng, i, vp, vp, lng, vp, ctypes.c_size_t, vp]
    L.tp_gemm.restype = i
    L.tp_strerror.argtypes, L.tp_strerror.restype = [i], ctypes.c_char_p
    _lib = L
    return L


def strerror(code: int) -> str:
    return lib().tp_strerror(code).decode()


def _check(code, where):
    if code != TP_OK:
        raise TPError(code, where)


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def torch_dtype(dtype: int):
    return torch.bfloat16 if dtype == TP_BF16 else torch.float32


def _expect(t, numel, dt, name):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dt or t.numel() != numel:
        raise ValueError(f"{name}: expected a contiguous {dt} CUDA tensor of {numel} elements, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


# ---------------------------------------------------------------------------
# entry points, same names as the C ABI
# ---------------------------------------------------------------------------

def tp_check_args(h, a, s, b, t, rank, dtype, block) -> int:
    return lib().tp_check_args(h, a, s, b, t, rank, dtype, block)


def tp_saved_bytes(h, a, s, b, t, dtype, block) -> int:
    return lib().tp_saved_bytes(h, a, s, b, t, dtype, block)


def tp_workspace_bytes(h, a, s, b, t, dtype, block) -> int:
    return lib().tp_workspace_bytes(h, a, s, b, t, dtype, block)


def block_shapes(h, t, block):
    """(w_in, b_in, w_out, b_out) shapes of one rank's block weights."""
    n = 3 * h // t if block == TP_ATTN else 4 * h // t
    k = h // t if block == TP_ATTN else 4 * h // t
    return (h, n), (n,), (k, h), (h,)


def tp_layer_fwd(h, a, s, b, t, rank, dtype, block, x, w, y_partial, saved, workspace, stream=None):
    """w = (w_in, b_in, w_out, b_out) tensors; see tp_block_weights."""
    dt = torch_dtype(dtype)
    T = s * b
    shapes = block_shapes(h, t, block)
    for name, tens, shp in zip(("w_in", "b_in", "w_out", "b_out"), w, shapes):
        _expect(tens, int(torch.Size(shp).numel()), dt, name)
    _expect(x, T * h, dt, "x")
    _expect(y_partial, T * h, dt, "y_partial")
    W = TPBlockWeights(*[t_.data_ptr() for t_ in w])
    rc = lib().tp_layer_fwd(h, a, s, b, t, rank, dtype, block, _ptr(x), ctypes.byref(W), _ptr(y_partial),
                            _ptr(saved), _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream))
    _check(rc, "tp_layer_fwd")


def tp_layer_bwd(h, a, s, b, t, rank, dtype, block, x, w, saved, dy, dx_partial, g, workspace, stream=None):
    """g = (dw_in, db_in, dw_out, db_out) output tensors; see tp_block_grads."""
    dt = torch_dtype(dtype)
    T = s * b
    shapes = block_shapes(h, t, block)
    for name, tens, shp in zip(("w_in", "b_in", "w_out", "b_out"), w, shapes):
        _expect(tens, int(torch.Size(shp).numel()), dt, name)
    for name, tens, shp in zip(("dw_in", "db_in", "dw_out", "db_out"), g, shapes):
        _expect(tens, int(torch.Size(shp).numel()), dt, name)
    _expect(x, T * h, dt, "x")
    _expect(dy, T * h, dt, "dy")
    _expect(dx_partial, T * h, dt, "dx_partial")
    W = TPBlockWeights(*[t_.data_ptr() for t_ in w])
    G = TPBlockGrads(*[t_.data_ptr() for t_ in g])
    rc = lib().tp_layer_bwd(h, a, s, b, t, rank, dtype, block, _ptr(x), ctypes.byref(W), _ptr(saved), _ptr(dy),
                            _ptr(dx_partial), ctypes.byref(G), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "tp_layer_bwd")


def tp_noalloc_scratch_bytes():
    return int(lib().tp_noalloc_scratch_bytes())


def tp_layer_bwd_noalloc(h, a, s, b, t, rank, dtype, block, x, w, saved, dy, dx_partial, g, stream=None):
    """tp_layer_bwd on the library's own device scratch (no workspace argument)."""
    dt = torch_dtype(dtype)
    T = s * b
    shapes = block_shapes(h, t, block)
    for name, tens, shp in zip(("w_in", "b_in", "w_out", "b_out"), w, shapes):
        _expect(tens, int(torch.Size(shp).numel()), dt, name)
    for name, tens, shp in zip(("dw_in", "db_in", "dw_out", "db_out"), g, shapes):
        _expect(tens, int(torch.Size(shp).numel()), dt, name)
    _expect(x, T * h, dt, "x")
    _expect(dy, T * h, dt, "dy")
    _expect(dx_partial, T * h, dt, "dx_partial")
    W = TPBlockWeights(*[t_.data_ptr() for t_ in w])
    G = TPBlockGrads(*[t_.data_ptr() for t_ in g])
    rc = lib().tp_layer_bwd_noalloc(h, a, s, b, t, rank, dtype, block, _ptr(x), ctypes.byref(W), _ptr(saved),
                                    _ptr(dy), _ptr(dx_partial), ctypes.byref(G), _stream(stream))
    _check(rc, "tp_layer_bwd_noalloc")


def tp_reduce_partials(dtype, partials, out, bias=None, residual=None, stream=None):
    """out = sum over ranks of partials [t, rows, cols] (+ bias [cols]) (+ residual [rows, cols])."""
    t = partials.shape[0]
    rows, cols = out.shape
    dt = torch_dtype(dtype)
    _expect(partials, t * rows * cols, dt, "partials")
    _expect(out, rows * cols, dt, "out")
    _expect(bias, cols, dt, "bias")
    _expect(residual, rows * cols, dt, "residual")
    _check(lib().tp_reduce_partials(dtype, rows, cols, t, _ptr(partials), _ptr(bias), _ptr(residual), _ptr(out),
                                    _stream(stream)), "tp_reduce_partials")


def tp_layer_bwd_recompute(h, a, s, b, t, rank, dtype, block, x, w, dy, dx_partial, g, scratch, workspace,
                           stream=None):
    """tp_layer_bwd that re-runs the forward into `scratch` (tp_saved_bytes) first."""
    dt = torch_dtype(dtype)
    T = s * b
    shapes = block_shapes(h, t, block)
    for name, tens, shp in zip(("w_in", "b_in", "w_out", "b_out"), w, shapes):
        _expect(tens, int(torch.Size(shp).numel()), dt, name)
    for name, tens, shp in zip(("dw_in", "db_in", "dw_out", "db_out"), g, shapes):
        _expect(tens, int(torch.Size(shp).numel()), dt, name)
    _expect(x, T * h, dt, "x")
    _expect(dy, T * h, dt, "dy")
    _expect(dx_partial, T * h, dt, "dx_partial")
    if scratch.numel() * scratch.element_size() < tp_saved_bytes(h, a, s, b, t, dtype, block):
        raise ValueError("scratch: smaller than tp_saved_bytes")
    W = TPBlockWeights(*[t_.data_ptr() for t_ in w])
    G = TPBlockGrads(*[t_.data_ptr() for t_ in g])
    rc = lib().tp_layer_bwd_recompute(h, a, s, b, t, rank, dtype, block, _ptr(x), ctypes.byref(W), _ptr(dy),
                                      _ptr(dx_partial), ctypes.byref(G), _ptr(scratch), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "tp_layer_bwd_recompute")


def tp_layernorm_fwd(dtype, x, gamma=None, beta=None, y=None, stats=None, bias=None, residual=None, sum_out=None,
                     eps=1e-5, stream=None):
    """v = x + residual + bias (into sum_out); y = LayerNorm(v) gamma + beta, stats [rows, 2] fp32."""
    rows, h = x.shape
    dt = torch_dtype(dtype)
    _expect(x, rows * h, dt, "x")
    for name, tens, n in (("bias", bias, h), ("residual", residual, rows * h), ("gamma", gamma, h),
                          ("beta", beta, h), ("sum_out", sum_out, rows * h), ("y", y, rows * h)):
        _expect(tens, n, dt, name)
    _expect(stats, rows * 2, torch.float32, "stats")
    _check(lib().tp_layernorm_fwd(dtype, rows, h, eps, _ptr(x), _ptr(bias), _ptr(residual), _ptr(gamma), _ptr(beta),
                                  _ptr(sum_out), _ptr(y), _ptr(stats), _stream(stream)), "tp_layernorm_fwd")


def tp_layernorm_bwd(dtype, dy, v, stats, gamma, dx, dresid=None, dgamma=None, dbeta=None, stream=None):
    """dx = LayerNorm backward of dy (+ dresid); dgamma, dbeta = sums over the rows."""
    rows, h = dy.shape
    dt = torch_dtype(dtype)
    for name, tens, n in (("dy", dy, rows * h), ("v", v, rows * h), ("gamma", gamma, h), ("dx", dx, rows * h),
                          ("dresid", dresid, rows * h), ("dgamma", dgamma, h), ("dbeta", dbeta, h)):
        _expect(tens, n, dt, name)
    _expect(stats, rows * 2, torch.float32, "stats")
    _check(lib().tp_layernorm_bwd(dtype, rows, h, _ptr(dy), _ptr(v), _ptr(stats), _ptr(gamma), _ptr(dresid),
                                  _ptr(dx), _ptr(dgamma), _ptr(dbeta), _stream(stream)), "tp_layernorm_bwd")


def tp_prof_enable(on: bool):
    _check(lib().tp_prof_enable(int(bool(on))), "tp_prof_enable")


def tp_prof_read():
    """{role: {"launches", "ms", "flops", "bytes"}} summed since tp_prof_enable(True)."""
    buf = (TPProfEntry * 64)()
    n = lib().tp_prof_read(buf, 64)
    if n < 0:
        raise TPError(n, "tp_prof_read")
    return {buf[i].name.decode(): {"launches": buf[i].launches, "ms": buf[i].ms, "flops": buf[i].flops,
                                   "bytes": buf[i].bytes} for i in range(min(n, 64))}


def tp_gemm_workspace_bytes(dtype, M, N, K):
    return int(lib().tp_gemm_workspace_bytes(dtype, M, N, K))


def tp_gemm(dtype, M, N, K, alpha, A, lda, a_kmajor, B, ldb, b_kmajor, bias, C, ldc, workspace=None, stream=None):
    """C = alpha op(A) op(B) (+ bias). `workspace`: a device tensor of at least
    tp_gemm_workspace_bytes(dtype, M, N, K) bytes, allocated here if None."""
    need = tp_gemm_workspace_bytes(dtype, M, N, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=C.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tp_gemm(dtype, M, N, K, alpha, _ptr(A), lda, int(a_kmajor), _ptr(B), ldb, int(b_kmajor),
                         _ptr(bias), _ptr(C), ldc, _ptr(workspace), nbytes, _stream(stream)), "tp_gemm")

"""Helpers shared by the GPU parity tests: run the layer through the C ABI
and compare with the oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

from megatron_tensor_layer_amd import inputs as I
from megatron_tensor_layer_amd import tplayer as tp
from megatron_tensor_layer_amd.layer import TPLayer, weights_from_parts
from oracle import tp_layer_oracle as O

TOL = {"fp32": 1e-5, "bf16": 1e-2}


def dtype_code(cfg):
    return tp.TP_BF16 if cfg.dtype == "bf16" else tp.TP_FP32


def to_dev(x, cfg):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda", tp.torch_dtype(dtype_code(cfg)))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite values in GPU output"
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def assert_close(name, gpu, ref, tol, report=None):
    e = rel_err(gpu, ref)
    if report is not None:
        report[name] = e
    assert e <= tol, f"{name}: max|err|/max|ref| = {e:.3e} > {tol:.0e}"


def full_layer_gpu(cfg):
    """All t ranks on the GPU, whole layer fwd + bwd. Returns the layer and inputs."""
    dt = dtype_code(cfg)
    weights = [weights_from_parts(I.params_rank(cfg, r), dt) for r in range(cfg.t)]
    layer = TPLayer(cfg.h, cfg.a, cfg.s, cfg.b, cfg.t, dt, weights)
    X = I.activation(cfg, "X")
    dY = I.activation(cfg, "dY")
    Xd, dYd = to_dev(X, cfg), to_dev(dY, cfg)
    layer.forward(Xd)
    layer.backward(dYd)
    torch.cuda.synchronize()
    return layer, X, dY


def full_layer_oracle(cfg, X, dY):
    p = I.params_full(cfg)
    Y, cache = O.layer_forward(X, p, cfg.s, cfg.b, cfg.a)
    g = O.layer_backward(cache, p, dY, cfg.s, cfg.b, cfg.a)
    return p, Y, cache, g


def compare_full_layer(cfg, layer, Y, cache, g, tol, report=None):
    t, h = cfg.t, cfg.h
    assert_close("H", to_np(layer.H), cache["H"], tol, report)
    assert_close("Y", to_np(layer.Y), Y, tol, report)
    assert_close("dH", to_np(layer.dH), g["dH"], tol, report)
    assert_close("dX", to_np(layer.dX), g["dX"], tol, report)
    c = lambda r: O.col_range(h, r, t)          # noqa: E731
    f = lambda r: O.col_range(4 * h, r, t)      # noqa: E731
    ref_qkv = lambda r: np.concatenate([g["dWq"][:, c(r)], g["dWk"][:, c(r)], g["dWv"][:, c(r)]], axis=1)  # noqa
    ref_bqkv = lambda r: np.concatenate([g["dbq"][c(r)], g["dbk"][c(r)], g["dbv"][c(r)]])  # noqa
    dw_qkv = np.concatenate([to_np(layer.grads[r]["attn"][0]) for r in range(t)], axis=1)
    assert_close("dWqkv", dw_qkv, np.concatenate([ref_qkv(r) for r in range(t)], axis=1), tol, report)
    db_qkv = np.concatenate([to_np(layer.grads[r]["attn"][1]) for r in range(t)])
    assert_close("dbqkv", db_qkv, np.concatenate([ref_bqkv(r) for r in range(t)]), tol, report)
    dwo = np.concatenate([to_np(layer.grads[r]["attn"][2]) for r in range(t)], axis=0)
    assert_close("dWo", dwo, g["dWo"], tol, report)
    dw1 = np.concatenate([to_np(layer.grads[r]["mlp"][0]) for r in range(t)], axis=1)
    assert_close("dW1", dw1, g["dW1"], tol, report)
    db1 = np.concatenate([to_np(layer.grads[r]["mlp"][1]) for r in range(t)])
    assert_close("db1", db1, g["db1"], tol, report)
    dw2 = np.concatenate([to_np(layer.grads[r]["mlp"][2]) for r in range(t)], axis=0)
    assert_close("dW2", dw2, g["dW2"], tol, report)
    for r in range(t):  # replicas: identical on every rank
        assert_close(f"dbo[r={r}]", to_np(layer.grads[r]["attn"][3]), g["dbo"], tol, report)
        assert_close(f"db2[r={r}]", to_np(layer.grads[r]["mlp"][3]), g["db2"], tol, report)

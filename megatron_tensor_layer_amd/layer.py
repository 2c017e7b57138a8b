"""Runs the t tensor-parallel ranks of one GPT layer one after another on a
single GPU through the C ABI, with the stand-in all-reduce (tp_reduce_partials)
where the collectives would sit:

    for r: tp_layer_fwd(ATTN, r, X)  -> partial_r ;  H  = X + bo + sum_r partial_r   (g)
    for r: tp_layer_fwd(MLP,  r, H)  -> partial_r ;  Y  = H + b2 + sum_r partial_r   (g)
    for r: tp_layer_bwd(MLP,  r, dY) -> dH_r      ;  dH = dY + sum_r dH_r           (f)
    for r: tp_layer_bwd(ATTN, r, dH) -> dX_r      ;  dX = dH + sum_r dX_r           (f)

The bias + residual add after each sum is fused into the reduction kernel.

Only buffers are allocated here (torch); every computation is a library call.
"""

from __future__ import annotations

import torch

from . import tplayer as tp


class TPLayer:
    """All t ranks of one layer, resident on one GPU.

    weights[r] = {"attn": (w_in, b_in, w_out, b_out), "mlp": (w_in, b_in, w_out, b_out)}
    with the shapes of tp_block_weights (rank-local shards, replicated biases whole).
    """

    def __init__(self, h, a, s, b, t, dtype, weights, device="cuda"):
        rc = tp.tp_check_args(h, a, s, b, t, 0, dtype, tp.TP_ATTN)
        if rc != tp.TP_OK:
            raise tp.TPError(rc, "TPLayer")
        self.h, self.a, self.s, self.b, self.t, self.dtype = h, a, s, b, t, dtype
        self.dims = (h, a, s, b, t)
        self.T = s * b
        dt = tp.torch_dtype(dtype)
        self.tdtype = dt
        self.weights = weights
        ws = max(tp.tp_workspace_bytes(h, a, s, b, t, dtype, blk) for blk in (tp.TP_ATTN, tp.TP_MLP))
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.saved = {blk: [torch.empty(tp.tp_saved_bytes(h, a, s, b, t, dtype, blk), dtype=torch.uint8,
                                        device=device) for _ in range(t)]
                      for blk in (tp.TP_ATTN, tp.TP_MLP)}
        self.partials = torch.empty((t, self.T, h), dtype=dt, device=device)
        self.H = torch.empty((self.T, h), dtype=dt, device=device)
        self.Y = torch.empty((self.T, h), dtype=dt, device=device)
        self.dH = torch.empty((self.T, h), dtype=dt, device=device)
        self.dX = torch.empty((self.T, h), dtype=dt, device=device)
        self.grads = []
        for r in range(t):
            g = {}
            for name, blk in (("attn", tp.TP_ATTN), ("mlp", tp.TP_MLP)):
                g[name] = tuple(torch.empty(shp, dtype=dt, device=device) for shp in tp.block_shapes(h, t, blk))
            self.grads.append(g)
        self.X = None

    # -- single rank / block calls -------------------------------------------
    def block_fwd(self, blk, r, x, out):
        name = "attn" if blk == tp.TP_ATTN else "mlp"
        tp.tp_layer_fwd(*self.dims, r, self.dtype, blk, x, self.weights[r][name], out, self.saved[blk][r],
                        self.workspace)

    def block_bwd(self, blk, r, x, dy, dx_out):
        name = "attn" if blk == tp.TP_ATTN else "mlp"
        tp.tp_layer_bwd(*self.dims, r, self.dtype, blk, x, self.weights[r][name], self.saved[blk][r], dy,
                        dx_out, self.grads[r][name], self.workspace)

    def reduce(self, out, bias=None, residual=None):
        tp.tp_reduce_partials(self.dtype, self.partials, out, bias=bias, residual=residual)

    # -- whole layer -----------------------------------------------------------
    def forward(self, X, reduce=True):
        self.X = X
        for r in range(self.t):
            self.block_fwd(tp.TP_ATTN, r, X, self.partials[r])
        if reduce:
            self.reduce(self.H, self.weights[0]["attn"][3], X)
        for r in range(self.t):
            self.block_fwd(tp.TP_MLP, r, self.H, self.partials[r])
        if reduce:
            self.reduce(self.Y, self.weights[0]["mlp"][3], self.H)
        return self.Y

    def backward(self, dY, reduce=True):
        for r in range(self.t):
            self.block_bwd(tp.TP_MLP, r, self.H, dY, self.partials[r])
        if reduce:
            self.reduce(self.dH, None, dY)
        for r in range(self.t):
            self.block_bwd(tp.TP_ATTN, r, self.X, self.dH, self.partials[r])
        if reduce:
            self.reduce(self.dX, None, self.dH)
        return self.dX


def weights_from_parts(parts, dtype, device="cuda"):
    """Rank weights in the ABI layout from per-rank parameter parts (numpy
    float32 arrays named Wq, Wk, Wv, bq, bk, bv, Wo, bo, W1, b1, W2, b2):
    the QKV shard is [Wq_r | Wk_r | Wv_r] side by side."""
    import numpy as np

    dt = tp.torch_dtype(dtype)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device=device, dtype=dt)

    w_qkv = np.concatenate([parts["Wq"], parts["Wk"], parts["Wv"]], axis=1)
    b_qkv = np.concatenate([parts["bq"], parts["bk"], parts["bv"]])
    return {"attn": (dev(w_qkv), dev(b_qkv), dev(parts["Wo"]), dev(parts["bo"])),
            "mlp": (dev(parts["W1"]), dev(parts["b1"]), dev(parts["W2"]), dev(parts["b2"]))}

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

    def __init__(self, h, a, s, b, t, dtype, weights, device="cuda", recompute=False):
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
        self.recompute = recompute
        if recompute:
            # full recomputation: nothing is kept between a block's forward and
            # its backward, which re-runs the forward into one shared scratch
            n = max(tp.tp_saved_bytes(h, a, s, b, t, dtype, blk) for blk in (tp.TP_ATTN, tp.TP_MLP))
            self.scratch = torch.empty(n, dtype=torch.uint8, device=device)
            self.saved = {blk: [self.scratch] * t for blk in (tp.TP_ATTN, tp.TP_MLP)}
        else:
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
        if self.recompute:
            tp.tp_layer_bwd_recompute(*self.dims, r, self.dtype, blk, x, self.weights[r][name], dy, dx_out,
                                      self.grads[r][name], self.scratch, self.workspace)
        else:
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


class SPLayer(TPLayer):
    """The pre-norm GPT layer (LayerNorm before each block) with sequence
    parallelism: rank r owns rows [r T/t, (r+1) T/t) of every [T, h]
    activation (the positions [r s/t, (r+1) s/t) of each sequence) for the
    LayerNorms, the output biases and the residual adds; the blocks run as in
    TPLayer on the gathered rows.  On one GPU the ranks write their slices of
    one [T, h] buffer, which is then the all-gather's result, and the
    reduce-scatter is the stand-in sum (tp_reduce_partials) read slice by
    slice:

      fwd  for r: a_r = LN1(x_r)                                   (rank)
           for r: tp_layer_fwd(ATTN, r, A)     -> partial_r        (rank)
           R = sum_r partial_r                                     (stand-in)
           for r: h_r = R_r + bo + x_r;  b_r = LN2(h_r)            (rank)
           for r: tp_layer_fwd(MLP, r, B)      -> partial_r        (rank)
           R = sum_r partial_r                                     (stand-in)
           for r: y_r = R_r + b2 + h_r                             (rank)
      bwd  for r: tp_layer_bwd(MLP, r, B, dY)  -> partial_r        (rank)
           R = sum_r partial_r                                     (stand-in)
           for r: dh_r = LN2'(R_r) + dy_r;  dg2_r, dbe2_r          (rank)
           for r: tp_layer_bwd(ATTN, r, A, dH) -> partial_r        (rank)
           R = sum_r partial_r                                     (stand-in)
           for r: dx_r = LN1'(R_r) + dh_r;  dg1_r, dbe1_r          (rank)
           dg = sum_r dg_r for the four LayerNorm parameters       (stand-in)

    ln = (g1, be1, g2, be2) device tensors [h], replicated."""

    def __init__(self, h, a, s, b, t, dtype, weights, ln, device="cuda", eps=1e-5, recompute=False):
        super().__init__(h, a, s, b, t, dtype, weights, device=device, recompute=recompute)
        if s % t != 0:
            raise ValueError(f"sequence parallelism needs s % t == 0 (s={s}, t={t})")
        dt = self.tdtype
        T = self.T
        self.n = T // t
        self.eps = eps
        self.ln = ln
        self.A = torch.empty((T, h), dtype=dt, device=device)
        self.B = torch.empty((T, h), dtype=dt, device=device)
        self.R = torch.empty((T, h), dtype=dt, device=device)
        self.stats1 = torch.empty((T, 2), dtype=torch.float32, device=device)
        self.stats2 = torch.empty((T, 2), dtype=torch.float32, device=device)
        self.ln_part = torch.empty((4, t, 1, h), dtype=dt, device=device)   # dg1, dbe1, dg2, dbe2 per rank
        self.ln_grads = torch.empty((4, 1, h), dtype=dt, device=device)

    def rows(self, r):
        return slice(r * self.n, (r + 1) * self.n)

    # -- rank calls of the sequence-parallel region -----------------------------
    def ln1_fwd(self, r, X):
        sl = self.rows(r)
        tp.tp_layernorm_fwd(self.dtype, X[sl], gamma=self.ln[0], beta=self.ln[1], y=self.A[sl],
                            stats=self.stats1[sl], eps=self.eps)

    def add_ln2_fwd(self, r, X):
        sl = self.rows(r)
        tp.tp_layernorm_fwd(self.dtype, self.R[sl], bias=self.weights[r]["attn"][3], residual=X[sl],
                            gamma=self.ln[2], beta=self.ln[3], sum_out=self.H[sl], y=self.B[sl],
                            stats=self.stats2[sl], eps=self.eps)

    def add_out_fwd(self, r):
        sl = self.rows(r)
        tp.tp_layernorm_fwd(self.dtype, self.R[sl], bias=self.weights[r]["mlp"][3], residual=self.H[sl],
                            sum_out=self.Y[sl])

    def ln2_bwd(self, r, dY):
        sl = self.rows(r)
        tp.tp_layernorm_bwd(self.dtype, self.R[sl], self.H[sl], self.stats2[sl], self.ln[2], self.dH[sl],
                            dresid=dY[sl], dgamma=self.ln_part[2, r, 0], dbeta=self.ln_part[3, r, 0])

    def ln1_bwd(self, r, X):
        sl = self.rows(r)
        tp.tp_layernorm_bwd(self.dtype, self.R[sl], X[sl], self.stats1[sl], self.ln[0], self.dX[sl],
                            dresid=self.dH[sl], dgamma=self.ln_part[0, r, 0], dbeta=self.ln_part[1, r, 0])

    def reduce_sum(self):
        tp.tp_reduce_partials(self.dtype, self.partials, self.R)

    def reduce_ln_grads(self):
        for i in range(4):
            tp.tp_reduce_partials(self.dtype, self.ln_part[i], self.ln_grads[i])

    # -- whole layer ------------------------------------------------------------
    def forward(self, X, reduce=True):
        self.X = X
        for r in range(self.t):
            self.ln1_fwd(r, X)
        for r in range(self.t):
            self.block_fwd(tp.TP_ATTN, r, self.A, self.partials[r])
        self.reduce_sum()
        for r in range(self.t):
            self.add_ln2_fwd(r, X)
        for r in range(self.t):
            self.block_fwd(tp.TP_MLP, r, self.B, self.partials[r])
        self.reduce_sum()
        for r in range(self.t):
            self.add_out_fwd(r)
        return self.Y

    def backward(self, dY, reduce=True):
        for r in range(self.t):
            self.block_bwd(tp.TP_MLP, r, self.B, dY, self.partials[r])
        self.reduce_sum()
        for r in range(self.t):
            self.ln2_bwd(r, dY)
        for r in range(self.t):
            self.block_bwd(tp.TP_ATTN, r, self.A, self.dH, self.partials[r])
        self.reduce_sum()
        for r in range(self.t):
            self.ln1_bwd(r, self.X)
        self.reduce_ln_grads()
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

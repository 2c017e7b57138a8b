"""Plain fp64 CPU oracle of one Megatron-style GPT Transformer layer and its
tensor-parallel (TP) per-rank view.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never imports it; the product path must never call it.

What it computes
----------------
The hot-path form of the unsharded layer is the attention block followed by
the MLP block, causal, dropout-free, with a residual add after each block and
no LayerNorm:

    Q = X Wq + bq,  K = X Wk + bk,  V = X Wv + bv
    per sequence beta and head j:  S = Q_bj K_bj^T / sqrt(d),
        S[i, k] = -inf for k > i,  P = row-softmax(S),  C_bj = P V_bj
    H = X + C Wo + bo
    U = H W1 + b1,  Z = GELU(U),  Y = H + Z W2 + b2

Activations are token-major [s, b, h] flattened to [s*b, h] with row index
sigma*b + beta; weights are W[d_in, d_out] with Y = X W.  The backward pass is
the hand-derived chain rule of the same definitions.

Sources (the pages this follows):
  * "Efficient Large-Scale Language Model Training on GPU Clusters Using
    Megatron-LM" (paper-graph summary), section 3, "Tensor Model Parallelism:
    The Megatron Partitioning": MLP Y = GeLU(XA), output YB; A split by
    columns, B by rows, one all-reduce after B; Q/K/V split by columns (whole
    heads), output projection split by rows; the conjugate f / g operators.
    Same section, "Computation Optimizations": the [s, b, a, h] layout, the
    causal mask applied implicitly inside the softmax, the fused bias+GeLU and
    bias+dropout+add (here without dropout).
  * "parallelism" blog post, "Tensor parallelism: split every matrix": the
    worked MLP example (ReLU) and its backward; the backward of a copied input
    is a sum; weight gradients need no communication; heads stay whole.
    Same page, "First: the three collectives": all-reduce is an element-wise
    sum over ranks.
  * "Distributed training" (ML interview book), section 2.6: column- and
    row-parallel definitions with row-major Y = XW; section 3.2: head-parallel
    attention with scale 1/sqrt(d_head) and contiguous column / row shards.

Readings where the pages are silent (each is listed in the design notes):
GELU is the exact erf form; biases exist on all four linears; the causal
mask lets query i see keys k <= i; the softmax scale is 1/sqrt(d_head); the
QKV shard of rank r is the contiguous column range c_r of each of Wq, Wk, Wv;
replicated terms (the output bias and the residual) are added once, after
the all-reduce of the partials, as the fused bias+dropout+add of the
paper-graph page's "Computation Optimizations" (here without dropout).

A second form of the layer adds the two LayerNorms of the GPT layer in
front of the blocks (pre-norm) and runs it with sequence parallelism: each
rank applies the LayerNorms, the biases after the row-parallel products and
the residual adds to its own contiguous slice of the sequence, the all-reduce
becomes a reduce-scatter along the sequence before that region and an
all-gather after it:

    A = LN1(X),  H = X + attn(A) Wo + bo,  B = LN2(H),  Y = H + MLP(B) + b2
    LN(x) = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta   per token,
        mean and (biased) variance over the token's h features, eps = 1e-5

Sources: "parallelism" blog post, "Sequence parallelism: the parts TP leaves
behind" (LayerNorm, dropout and the residual add split by tokens; the
all-reduce as reduce-scatter plus all-gather; LayerNorm on the rank's tokens,
then all-gather, the sharded products, reduce-scatter, then the residual),
and the same page's hybrid-parallelism walk-through (the gradients of the
replicated LayerNorm weights are partial per rank and are summed over the
tensor-parallel group); "Distributed training" (ML interview book), section
2.2 (two LayerNorms per layer, each storing its input; sequence parallelism
shards them along s).  The pages do not write LayerNorm out: the textbook
definition above is used, with biased variance and eps = 1e-5 (readings).

Parity pins live in tests/test_oracle_pins.py: the blog's worked MLP values,
closed forms of GELU and the softmax, brute-force loops on tiny inputs,
causal special cases, the sharded-equals-unsharded invariant and central
finite differences for every gradient.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64

PARAM_NAMES = ("Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo", "bo", "W1", "b1", "W2", "b2")


# ---------------------------------------------------------------------------
# element-wise pieces
# ---------------------------------------------------------------------------

def gelu(x):
    """Exact GELU, x * Phi(x), Phi the standard normal CDF (erf form).

    The paper-graph page names only "GeLU"; the interview book's listing uses
    PyTorch's default GELU, which is the erf form.
    """
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def gelu_grad(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x)."""
    x = np.asarray(x, dtype=F64)
    cdf = 0.5 * (1.0 + _erf(x / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return cdf + x * pdf


def relu(x):
    """Used only by the blog's worked example."""
    return np.maximum(np.asarray(x, dtype=F64), 0.0)


def relu_grad(x):
    """ReLU'(0) = 0: the blog's backward zeroes the entry whose input was 0."""
    return (np.asarray(x, dtype=F64) > 0.0).astype(F64)


_ACT = {"gelu": (gelu, gelu_grad), "relu": (relu, relu_grad)}


def softmax_rows(S):
    """Row-wise softmax with the usual max subtraction; -inf entries give 0."""
    S = np.asarray(S, dtype=F64)
    m = np.max(S, axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def all_reduce_sum(partials):
    """The stand-in for the all-reduce: element-wise sum over ranks, in rank order."""
    out = np.zeros_like(np.asarray(partials[0], dtype=F64))
    for p in partials:
        out = out + np.asarray(p, dtype=F64)
    return out


# ---------------------------------------------------------------------------
# token / head bookkeeping
# ---------------------------------------------------------------------------

def _heads(M, s, b, n_heads):
    """[s*b, n_heads*d] token-major -> [b, n_heads, s, d]."""
    d = M.shape[1] // n_heads
    return M.reshape(s, b, n_heads, d).transpose(1, 2, 0, 3)


def _unheads(M):
    """[b, n_heads, s, d] -> [s*b, n_heads*d] token-major."""
    b, n, s, d = M.shape
    return M.transpose(2, 0, 1, 3).reshape(s * b, n * d)


def causal_mask(s):
    """Boolean [s, s]: True where key k is hidden from query i (k > i)."""
    return np.triu(np.ones((s, s), dtype=bool), k=1)


# ---------------------------------------------------------------------------
# attention core: heads are independent, so one routine serves both the
# unsharded layer (all heads) and a rank (its own heads)
# ---------------------------------------------------------------------------

def attention_core_forward(Q, K, V, s, b, n_heads):
    """Causal scaled dot-product attention over n_heads heads of width d.

    Q, K, V: [s*b, n_heads*d] token-major.  Returns C [s*b, n_heads*d] and P
    [b, n_heads, s, s].
    """
    d = Q.shape[1] // n_heads
    q, k, v = (_heads(np.asarray(M, dtype=F64), s, b, n_heads) for M in (Q, K, V))
    S = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(d)
    S = np.where(causal_mask(s), -np.inf, S)
    P = softmax_rows(S)
    C = np.matmul(P, v)
    return _unheads(C), P


def attention_core_backward(Q, K, V, P, dC, s, b, n_heads):
    """Chain rule through C = P V, P = softmax(S), S = Q K^T / sqrt(d).

    Returns dQ, dK, dV, token-major like Q.
    """
    d = Q.shape[1] // n_heads
    q, k, v, dc = (_heads(np.asarray(M, dtype=F64), s, b, n_heads) for M in (Q, K, V, dC))
    dP = np.matmul(dc, np.swapaxes(v, -1, -2))
    dv = np.matmul(np.swapaxes(P, -1, -2), dc)
    # softmax Jacobian row by row: dS_i = P_i * (dP_i - <P_i, dP_i>)
    dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
    dq = np.matmul(dS, k) / math.sqrt(d)
    dk = np.matmul(np.swapaxes(dS, -1, -2), q) / math.sqrt(d)
    return _unheads(dq), _unheads(dk), _unheads(dv)


# ---------------------------------------------------------------------------
# unsharded layer
# ---------------------------------------------------------------------------

def attention_block_forward(X, p, s, b, n_heads):
    """H = X + C Wo + bo.  Returns H and the cache for the backward pass."""
    X = np.asarray(X, dtype=F64)
    Q = X @ p["Wq"] + p["bq"]
    K = X @ p["Wk"] + p["bk"]
    V = X @ p["Wv"] + p["bv"]
    C, P = attention_core_forward(Q, K, V, s, b, n_heads)
    H = X + C @ p["Wo"] + p["bo"]
    return H, dict(X=X, Q=Q, K=K, V=V, P=P, C=C)


def attention_block_backward(cache, p, dH, s, b, n_heads):
    dH = np.asarray(dH, dtype=F64)
    X, C = cache["X"], cache["C"]
    g = {"dWo": C.T @ dH, "dbo": dH.sum(axis=0)}
    dC = dH @ p["Wo"].T
    dQ, dK, dV = attention_core_backward(cache["Q"], cache["K"], cache["V"], cache["P"], dC, s, b, n_heads)
    g.update(dWq=X.T @ dQ, dWk=X.T @ dK, dWv=X.T @ dV,
             dbq=dQ.sum(axis=0), dbk=dK.sum(axis=0), dbv=dV.sum(axis=0))
    # X feeds the residual and the three projections: its gradient is the sum
    g["dX"] = dH + dQ @ p["Wq"].T + dK @ p["Wk"].T + dV @ p["Wv"].T
    return g


def mlp_branch_forward(H, W1, b1, W2, b2, act="gelu"):
    """Branch output act(H W1 + b1) W2 + b2, without the residual."""
    H = np.asarray(H, dtype=F64)
    U = H @ W1 + b1
    Z = _ACT[act][0](U)
    return Z @ W2 + b2, dict(H=H, U=U, Z=Z)


def mlp_branch_backward(cache, W1, W2, dOut, act="gelu"):
    """Gradients of the branch; dH here excludes the residual path."""
    dOut = np.asarray(dOut, dtype=F64)
    g = {"dW2": cache["Z"].T @ dOut, "db2": dOut.sum(axis=0)}
    dU = (dOut @ W2.T) * _ACT[act][1](cache["U"])
    g.update(dW1=cache["H"].T @ dU, db1=dU.sum(axis=0), dH=dU @ W1.T)
    return g


def mlp_block_forward(H, p, act="gelu"):
    """Y = H + act(H W1 + b1) W2 + b2."""
    out, cache = mlp_branch_forward(H, p["W1"], p["b1"], p["W2"], p["b2"], act)
    return cache["H"] + out, cache


def mlp_block_backward(cache, p, dY, act="gelu"):
    g = mlp_branch_backward(cache, p["W1"], p["W2"], dY, act)
    g["dH"] = np.asarray(dY, dtype=F64) + g["dH"]
    return g


def layer_forward(X, p, s, b, n_heads, act="gelu"):
    H, ca = attention_block_forward(X, p, s, b, n_heads)
    Y, cm = mlp_block_forward(H, p, act)
    return Y, dict(attn=ca, mlp=cm, H=H)


def layer_backward(cache, p, dY, s, b, n_heads, act="gelu"):
    gm = mlp_block_backward(cache["mlp"], p, dY, act)
    ga = attention_block_backward(cache["attn"], p, gm["dH"], s, b, n_heads)
    g = {k: v for k, v in gm.items() if k != "dH"}
    g.update(ga)
    g["dH"] = gm["dH"]
    return g


# ---------------------------------------------------------------------------
# the tensor-parallel method: rank r's share of each block
# ---------------------------------------------------------------------------

def col_range(width, r, t):
    """Contiguous chunk r of t along a split axis of the given width."""
    assert width % t == 0
    w = width // t
    return slice(r * w, (r + 1) * w)


def shard_params(p, r, t):
    """Rank r's slices: Wq/Wk/Wv/bq/bk/bv and W1/b1 by columns, Wo and W2 by
    rows; bo and b2 are replicated on every rank."""
    h = p["Wq"].shape[0]
    ffn = p["W1"].shape[1]
    c, f = col_range(h, r, t), col_range(ffn, r, t)
    return {
        "Wq": p["Wq"][:, c], "Wk": p["Wk"][:, c], "Wv": p["Wv"][:, c],
        "bq": p["bq"][c], "bk": p["bk"][c], "bv": p["bv"][c],
        "Wo": p["Wo"][c, :], "bo": p["bo"],
        "W1": p["W1"][:, f], "b1": p["b1"][f],
        "W2": p["W2"][f, :], "b2": p["b2"],
    }


def attention_rank_forward(X, pr, s, b, heads_r):
    """Rank's partial of the attention block: C_r Wo_r.

    The rank projects X (replicated: f is the identity forward) onto its own
    heads, runs their attention locally, and multiplies by its rows of Wo.
    The output bias and the residual are not part of any rank's partial: they
    are added after the all-reduce (see block_output).
    """
    X = np.asarray(X, dtype=F64)
    Q = X @ pr["Wq"] + pr["bq"]
    K = X @ pr["Wk"] + pr["bk"]
    V = X @ pr["Wv"] + pr["bv"]
    C, P = attention_core_forward(Q, K, V, s, b, heads_r)
    return C @ pr["Wo"], dict(X=X, Q=Q, K=K, V=V, P=P, C=C)


def attention_rank_backward(cache, pr, dH, s, b, heads_r):
    """Rank-local backward of the attention block given the replicated dH
    (g's backward is the identity).  Returns the rank's partial of dL/dX
    through its own heads (summed over ranks by f's backward all-reduce; the
    residual path dH is added once after it, see block_output), its weight and
    bias gradient shards, and dbo (a replica, equal on every rank)."""
    dH = np.asarray(dH, dtype=F64)
    X, C = cache["X"], cache["C"]
    g = {"dWo": C.T @ dH, "dbo": dH.sum(axis=0)}
    dC = dH @ pr["Wo"].T
    dQ, dK, dV = attention_core_backward(cache["Q"], cache["K"], cache["V"], cache["P"], dC, s, b, heads_r)
    g.update(dWq=X.T @ dQ, dWk=X.T @ dK, dWv=X.T @ dV,
             dbq=dQ.sum(axis=0), dbk=dK.sum(axis=0), dbv=dV.sum(axis=0))
    g["dX"] = dQ @ pr["Wq"].T + dK @ pr["Wk"].T + dV @ pr["Wv"].T
    g["dC"] = dC
    return g


def mlp_rank_forward(H, pr, act="gelu"):
    """Rank's partial act(H W1_r + b1_r) W2_r; b2 and the residual are added
    after the all-reduce."""
    return mlp_branch_forward(H, pr["W1"], pr["b1"], pr["W2"], 0.0, act)


def mlp_rank_backward(cache, pr, dY, act="gelu"):
    """Rank's partial of dL/dH through its FC1/FC2 shards (the residual path
    dY is added after the all-reduce), its W1/b1/W2 shards' gradients and db2
    (a replica)."""
    return mlp_branch_backward(cache, pr["W1"], pr["W2"], dY, act)


def block_output(partials, bias=None, residual=None):
    """After the all-reduce: residual + bias + sum of the ranks' partials (the
    fused bias + dropout + residual add, without dropout).  In the backward the
    same routine adds the residual gradient to the summed partials."""
    out = all_reduce_sum(partials)
    if bias is not None:
        out = out + np.asarray(bias, dtype=F64)
    if residual is not None:
        out = out + np.asarray(residual, dtype=F64)
    return out


# ---------------------------------------------------------------------------
# FLOP accounting (paper-graph page, "FLOP Counting and Training Time
# Estimation", Eq. 3 restricted to one layer without recomputation and
# without the logit term)
# ---------------------------------------------------------------------------

def model_flops_per_rank(h, s, b, t):
    """72 b s h^2 (1 + s / 6h) / t: forward (24 b s h^2 (1 + s/6h)) plus a
    backward of twice that, for one layer, shared evenly over t ranks."""
    return 72.0 * b * s * h * h * (1.0 + s / (6.0 * h)) / t


# ---------------------------------------------------------------------------
# LayerNorm and the pre-norm layer with sequence parallelism
# ---------------------------------------------------------------------------

LN_EPS = 1e-5
LN_NAMES = ("g1", "be1", "g2", "be2")  # LN1 weight / bias, LN2 weight / bias


def layer_norm(x, gamma, beta, eps=LN_EPS):
    """Per token (row): normalise over the h features with the mean and the
    biased variance, then scale by gamma and shift by beta.  Returns the
    output and the cache for the backward pass (x_hat and 1/sqrt(var+eps))."""
    x = np.asarray(x, dtype=F64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * gamma + beta, dict(xhat=xhat, rstd=rstd, mean=mean)


def layer_norm_backward(cache, gamma, dy):
    """Chain rule through y = gamma * x_hat + beta, x_hat = (x - mean) rstd:
    with g = dy * gamma, dx = rstd (g - mean(g) - x_hat mean(g x_hat));
    dgamma = sum over tokens of dy x_hat, dbeta = sum over tokens of dy."""
    dy = np.asarray(dy, dtype=F64)
    xhat, rstd = cache["xhat"], cache["rstd"]
    g = dy * gamma
    dx = rstd * (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def attention_branch_forward(A, p, s, b, n_heads):
    """C Wo for the attention block fed with A (no bias, no residual)."""
    A = np.asarray(A, dtype=F64)
    Q = A @ p["Wq"] + p["bq"]
    K = A @ p["Wk"] + p["bk"]
    V = A @ p["Wv"] + p["bv"]
    C, P = attention_core_forward(Q, K, V, s, b, n_heads)
    return C @ p["Wo"], dict(X=A, Q=Q, K=K, V=V, P=P, C=C)


def prenorm_layer_forward(X, p, ln, s, b, n_heads):
    """The unsharded pre-norm layer: A = LN1(X), H = X + attn(A) Wo + bo,
    B = LN2(H), Y = H + MLP(B) + b2 (biases of all four linears, exact GELU)."""
    X = np.asarray(X, dtype=F64)
    A, c1 = layer_norm(X, ln["g1"], ln["be1"])
    att, ca = attention_branch_forward(A, p, s, b, n_heads)
    H = X + att + p["bo"]
    B, c2 = layer_norm(H, ln["g2"], ln["be2"])
    mo, cm = mlp_branch_forward(B, p["W1"], p["b1"], p["W2"], p["b2"])
    Y = H + mo
    return Y, dict(X=X, A=A, H=H, B=B, ln1=c1, ln2=c2, attn=ca, mlp=cm)


def prenorm_layer_backward(cache, p, ln, dY, s, b, n_heads):
    """Gradients of the pre-norm layer for the upstream gradient dY: every
    weight and bias, the four LayerNorm parameters, dH and dX."""
    dY = np.asarray(dY, dtype=F64)
    g = mlp_branch_backward(cache["mlp"], p["W1"], p["W2"], dY)
    dB = g.pop("dH")
    dH_ln, g["dg2"], g["dbe2"] = layer_norm_backward(cache["ln2"], ln["g2"], dB)
    dH = dY + dH_ln                       # residual path + through LN2
    ga = attention_rank_backward(cache["attn"], p, dH, s, b, n_heads)
    dA = ga.pop("dX")
    ga.pop("dC")
    g.update(ga)
    dX_ln, g["dg1"], g["dbe1"] = layer_norm_backward(cache["ln1"], ln["g1"], dA)
    g["dX"] = dH + dX_ln                  # residual path + through LN1
    g["dH"] = dH
    return g


def seq_range(tokens, r, t):
    """Rank r's contiguous slice of the token rows.  Rows are token-major
    (row = sigma * b + beta), so the slice is the positions
    [r s / t, (r + 1) s / t) of every sequence."""
    return col_range(tokens, r, t)


def all_gather_rows(slices):
    """Stand-in for the all-gather along the sequence: rank slices in order."""
    return np.concatenate([np.asarray(x, dtype=F64) for x in slices], axis=0)


def reduce_scatter_rows(partials, r, t):
    """Stand-in for the reduce-scatter along the sequence: rank r's slice of
    the element-wise sum over ranks."""
    tot = all_reduce_sum(partials)
    return tot[seq_range(tot.shape[0], r, t)]


def sp_layer_forward(X, p, ln, s, b, n_heads, t):
    """The pre-norm layer as t sequence- and tensor-parallel ranks compute it.

    Per rank r, with x_r its token slice of X:
      a_r = LN1(x_r);  A = all-gather(a_r);  part_r = attn_r(A) Wo_r
      h_r = reduce-scatter(part)_r + bo + x_r;  b_r = LN2(h_r);  B = all-gather(b_r)
      part_r = MLP_r(B);  y_r = reduce-scatter(part)_r + b2 + h_r
    Returns the rank outputs y_r (their concatenation is Y) and per-rank caches."""
    X = np.asarray(X, dtype=F64)
    T = X.shape[0]
    ar = n_heads // t
    ranks = [dict(pr=shard_params(p, r, t), x=X[seq_range(T, r, t)]) for r in range(t)]
    for rk in ranks:
        rk["a"], rk["ln1"] = layer_norm(rk["x"], ln["g1"], ln["be1"])
    A = all_gather_rows([rk["a"] for rk in ranks])
    parts = []
    for rk in ranks:
        part, rk["attn"] = attention_rank_forward(A, rk["pr"], s, b, ar)
        parts.append(part)
    for r, rk in enumerate(ranks):
        rk["h"] = reduce_scatter_rows(parts, r, t) + p["bo"] + rk["x"]
        rk["b"], rk["ln2"] = layer_norm(rk["h"], ln["g2"], ln["be2"])
    B = all_gather_rows([rk["b"] for rk in ranks])
    parts = []
    for rk in ranks:
        part, rk["mlp"] = mlp_rank_forward(B, rk["pr"])
        parts.append(part)
    ys = [reduce_scatter_rows(parts, r, t) + p["b2"] + rk["h"] for r, rk in enumerate(ranks)]
    return ys, ranks


def sp_layer_backward(ranks, ln, dys, s, b, n_heads, t):
    """Backward of sp_layer_forward for the rank slices dy_r of dY.

    Per rank r:
      dY = all-gather(dy_r);  MLP_r backward -> part_r (and the W1/b1/W2 shards, db2)
      dh_r = LN2 backward of reduce-scatter(part)_r + dy_r   (dg2_r, dbe2_r partial)
      dH = all-gather(dh_r);  attention_r backward -> part_r (QKV/Wo shards, dbo)
      dx_r = LN1 backward of reduce-scatter(part)_r + dh_r   (dg1_r, dbe1_r partial)
    The LayerNorm parameter gradients of a rank cover its own tokens only:
    their sum over ranks is the full gradient.  Returns per-rank dicts."""
    T = sum(np.asarray(d).shape[0] for d in dys)
    ar = n_heads // t
    dY = all_gather_rows(dys)
    out = [dict() for _ in range(t)]
    parts = []
    for r, rk in enumerate(ranks):
        g = mlp_rank_backward(rk["mlp"], rk["pr"], dY)
        parts.append(g.pop("dH"))
        out[r].update(g)
    for r, rk in enumerate(ranks):
        dln, out[r]["dg2"], out[r]["dbe2"] = layer_norm_backward(rk["ln2"], ln["g2"], reduce_scatter_rows(parts, r, t))
        out[r]["dh"] = dln + np.asarray(dys[r], dtype=F64)
    dH = all_gather_rows([o["dh"] for o in out])
    parts = []
    for r, rk in enumerate(ranks):
        g = attention_rank_backward(rk["attn"], rk["pr"], dH, s, b, ar)
        parts.append(g.pop("dX"))
        g.pop("dC")
        out[r].update(g)
    for r, rk in enumerate(ranks):
        dln, out[r]["dg1"], out[r]["dbe1"] = layer_norm_backward(rk["ln1"], ln["g1"], reduce_scatter_rows(parts, r, t))
        out[r]["dx"] = dln + out[r]["dh"]
    assert dY.shape[0] == T
    return out

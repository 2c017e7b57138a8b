"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Tolerance per tensor: max|gpu - ref| / max|ref| <= 1e-5
for the fp32 configuration and <= 1e-2 for bf16."""

import math

import numpy as np
import pytest
import torch

from megatron_tensor_layer_amd import inputs as I
from megatron_tensor_layer_amd import tplayer as tp
from megatron_tensor_layer_amd.layer import weights_from_parts
from oracle import tp_layer_oracle as O

from gpu_helpers import (TOL, assert_close, compare_full_layer, dtype_code, full_layer_gpu, full_layer_oracle,
                         rel_err, to_dev, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(gpu):
    tp.lib()  # fail loudly if the library is missing where a GPU is present
    yield


# ---------------------------------------------------------------------------
# the MFMA GEMM on its own, every operand layout, ragged tiles
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("ak,bk", [(1, 0), (1, 1), (0, 0), (0, 1)])
@pytest.mark.parametrize("M,N,K", [(272, 400, 336), (16, 32, 48), (528, 256, 1040), (528, 528, 256)])
@pytest.mark.parametrize("alpha,with_bias", [(0.5, True), (1.0, False)])  # scaled + bias, and the plain epilogue
def test_gemm_layouts(dtype, ak, bk, M, N, K, alpha, with_bias):
    print(f"gemm {dtype} ak={ak} bk={bk} {M}x{N}x{K} alpha={alpha} bias={with_bias}", flush=True)
    cfg = I.make_config("gemm", 64, 4, 32, 2, 1, dtype)
    rng = np.random.default_rng(M * 7 + N * 3 + K + ak * 2 + bk)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    if dtype == "bf16":
        A, B, bias = I.round_to_bf16(A), I.round_to_bf16(B), I.round_to_bf16(bias)
    ref = alpha * (A.astype(np.float64) @ B.astype(np.float64)) + (bias if with_bias else 0.0)
    Ad = to_dev(A if ak else A.T, cfg)
    Bd = to_dev(B.T if bk else B, cfg)
    C = torch.full((M, N), float("nan"), device="cuda", dtype=tp.torch_dtype(dtype_code(cfg)))
    tp.tp_gemm(dtype_code(cfg), M, N, K, alpha, Ad, K if ak else M, ak, Bd, K if bk else N, bk,
               to_dev(bias, cfg) if with_bias else None, C, N)
    torch.cuda.synchronize()
    # bf16 output rounding (2^-9) plus fp32 accumulation; fp32: accumulation only
    tol = 8e-3 if dtype == "bf16" else 1e-5
    assert rel_err(to_np(C), ref) <= tol


# Launch plans at full size: stream-K over a partial last wave (with and
# without whole waves before it, ragged M and N, 3 and 6 fragments per tile,
# with and without the per-XCD placement of stream-K tiles), whole waves of
# 256 x 192 tiles, and split-K. Rows sampled (first, last, scattered), every column, fp64
# reference from the same bf16 operands; a second call must match bitwise.
@pytest.mark.parametrize("M,N,K,ak,bk,plan", [
    (2064, 4624, 12288, 1, 0, "sk"),   # 171 tiles < one wave: all stream-K (c = 129 of 192 iterations)
    (2064, 4112, 12288, 1, 1, "dp192"),  # 153 tiles of 256 rows: one partial wave of 187 192-row tiles
    (2048, 4608, 12288, 1, 0, "dp192"),  # the 175B QKV shape: 144 -> 198 tiles (3 passes of 64 staged rows)
    (1936, 4112, 12288, 1, 1, "dp192"),  # ragged M in 192-row tiles (1936 = 10 x 192 + 16)
    (1936, 4112, 12288, 0, 1, "dp"),     # M-contiguous A: 256-row tiles only
    (2048, 6144, 2048, 1, 1, "dp"),    # 192 tiles, one partial wave: 256 more 192-row tiles would not fit
    (2048, 12288, 1536, 1, 1, "dp+half"),  # 384 tiles: 256 whole, then columns 8192.. as 256 x 128 tiles
    (2048, 10256, 1536, 1, 1, "dp+half"),  # 328 tiles: 8192 columns whole, 2064 (ragged) in 136 half tiles
    (2048, 12288, 1536, 0, 0, "dp+half"),  # M-contiguous A and N-contiguous B in the half tiles
    (2048, 10256, 1536, 0, 1, "dp+half"),
    (2048, 6144, 12288, 1, 1, "sk"),   # stream-K tiles placed as 2 x 12 blocks per XCD
    (2048, 6128, 12288, 1, 1, "sk"),   # the same placement with a ragged last tile-column
    (2048, 12288, 6144, 1, 1, "sk"),   # a whole wave, then stream-K tiles in 4 x 4 blocks
    (2048, 6144, 12288, 1, 0, "n192"),  # the 175B FC1 shape: one whole wave of 256 x 192 tiles
    (2048, 12288, 6144, 1, 0, "n192"),  # the 175B FC2 shape: two whole waves of 256 x 192 tiles
    (2048, 12288, 1536, 1, 0, "n192"),  # the 175B O projection
    (1024, 12288, 8192, 0, 1, "sk"),   # 4 tile-rows: 2 x 12 blocks per XCD, two blocks down the rows
    (2048, 10240, 4096, 1, 1, "sk"),   # a whole wave, then 64 stream-K tiles in 2 x 4 blocks from column 32
    (2064, 8208, 6144, 0, 0, "sk"),    # 297 tiles: one whole wave + stream-K over 41 tiles (6 fragments each)
    (2064, 8208, 6144, 0, 1, "sk"),
    (1040, 2832, 4096, 1, 0, "split"),  # 60 tiles: split-K
])
def test_gemm_launch_plans_full_size(M, N, K, ak, bk, plan):
    print(f"gemm plan {M}x{N}x{K} ak={ak} bk={bk} ({plan})", flush=True)
    rng = np.random.default_rng(M + N + K + 2 * ak + bk)
    A = I.round_to_bf16(rng.standard_normal((M, K), dtype=np.float32))
    B = I.round_to_bf16(rng.standard_normal((K, N), dtype=np.float32))
    bias = I.round_to_bf16(rng.standard_normal(N, dtype=np.float32))
    bf = torch.bfloat16
    Ad = torch.from_numpy(A if ak else np.ascontiguousarray(A.T)).to("cuda", bf)
    Bd = torch.from_numpy(np.ascontiguousarray(B.T) if bk else B).to("cuda", bf)
    bd = torch.from_numpy(bias).to("cuda", bf)
    # stream-K and split-K keep fp32 partials in the workspace; whole tiles need none
    # (the size is layout-blind: shapes that 256 x 192 tiles fill get the stream-K size)
    if plan != "n192":
        assert (tp.tp_gemm_workspace_bytes(tp.TP_BF16, M, N, K) > 0) == (not plan.startswith("dp"))
    outs = []
    for _ in range(2):
        C = torch.full((M, N), float("nan"), device="cuda", dtype=bf)
        tp.tp_gemm(tp.TP_BF16, M, N, K, 0.5, Ad, K if ak else M, ak, Bd, K if bk else N, bk, bd, C, N)
        outs.append(C)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 16, M - 1], rng.integers(0, M, 59)]))
    ref = 0.5 * (A[rows].astype(np.float64) @ B.astype(np.float64)) + bias
    got = outs[0][torch.from_numpy(rows).cuda()].float().cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= 8e-3


# ---------------------------------------------------------------------------
# whole layer, all ranks, element by element
# ---------------------------------------------------------------------------

SMALL = {
    # the fp32 check configuration: h=64, a=4, s=32, b=2, t=4
    "check_fp32": I.CONFIGS["check_fp32"],
    # bf16, several tiles in every GEMM with ragged tails (T=544, s=272 vs 128/256 tiles)
    "bf16_ragged": I.make_config("bf16_ragged", h=384, a=6, s=272, b=2, t=2, dtype="bf16"),
    # bf16, d = 160 (non power of two head width, as at the 1T shape), t = 2
    "bf16_d160": I.make_config("bf16_d160", h=320, a=2, s=160, b=2, t=2, dtype="bf16"),
    # bf16, d = 96 and t = 1 (as at the 1.7B shape), short-K split-K off
    "bf16_d96": I.make_config("bf16_d96", h=192, a=2, s=128, b=3, t=1, dtype="bf16"),
    # bf16, split-K engaged (few output tiles, K = h >= 2048)
    "bf16_splitk": I.make_config("bf16_splitk", h=2048, a=16, s=256, b=1, t=2, dtype="bf16"),
    # fp32, ragged and several tiles
    "fp32_ragged": I.make_config("fp32_ragged", h=128, a=8, s=80, b=3, t=2, dtype="fp32"),
    # bf16, d = 128, sequence long enough (18 key tiles of 64) that the fused
    # attention cuts the longer causal ranges into chunks and merges them
    "bf16_chunked": I.make_config("bf16_chunked", h=256, a=2, s=1152, b=1, t=2, dtype="bf16"),
    # the same chunk merge at d = 160 (the 1T head width): the last query
    # blocks' 18-tile ranges run as chunks of 8, 8 and 2 tiles
    "bf16_d160_chunked": I.make_config("bf16_d160_chunked", h=320, a=2, s=1152, b=1, t=2, dtype="bf16"),
    # d = 96 with enough (sequence, head) pairs (b * a / t = 128, 8 query
    # blocks each) that every causal range runs whole in one workgroup: up to
    # 16 key tiles of online softmax without a chunk merge, as at the 1.7B shape
    "bf16_d96_long": I.make_config("bf16_d96_long", h=192, a=2, s=1024, b=64, t=1, dtype="bf16"),
    # bf16, d = 64, a sequence shorter than one 64-key tile (s = 16): the fused
    # attention's partial tiles, clamped rows and LSE chunks at their smallest
    "bf16_short": I.make_config("bf16_short", h=128, a=2, s=16, b=3, t=2, dtype="bf16"),
    # bf16 with a head width the fused attention kernels are not built for
    # (d = 48): attention through the materialised s x s GEMM path
    "bf16_d48": I.make_config("bf16_d48", h=192, a=4, s=96, b=2, t=2, dtype="bf16"),
}

# bf16 head widths that run the fused (flash) attention kernels
FLASH_D = (64, 96, 128, 160)


def attention_roles(cfg):
    if cfg.dtype == "bf16" and cfg.d in FLASH_D:
        return {"attn_fwd", "attn_dkv", "attn_dq"}
    return {"scores", "softmax", "pv", "ds", "dv", "dq", "dk"}


@pytest.mark.parametrize("name", list(SMALL))
def test_full_layer_against_oracle(name):
    cfg = SMALL[name]
    print(f"full layer {name}: {cfg}", flush=True)
    layer, X, dY = full_layer_gpu(cfg)
    _, Y, cache, g = full_layer_oracle(cfg, X, dY)
    report = {}
    compare_full_layer(cfg, layer, Y, cache, g, TOL[cfg.dtype], report)
    print({k: f"{v:.2e}" for k, v in report.items()}, flush=True)


def test_rank_partials_against_oracle_per_rank():
    """Each rank's partial outputs and gradients against the oracle's per-rank
    view (fp32 check configuration)."""
    cfg = I.CONFIGS["check_fp32"]
    layer, X, dY = full_layer_gpu(cfg)
    p = I.params_full(cfg)
    ar = cfg.a // cfg.t
    tol = TOL["fp32"]
    # attention partials of every rank from the same X
    for r in range(cfg.t):
        pr = O.shard_params(p, r, cfg.t)
        part, _ = O.attention_rank_forward(X, pr, cfg.s, cfg.b, ar)
        out = torch.empty_like(layer.H)
        layer.block_fwd(tp.TP_ATTN, r, to_dev(X, cfg), out)
        torch.cuda.synchronize()
        assert_close(f"attn partial r={r}", to_np(out), part, tol)
    # MLP partials and their backward from the same (oracle) H
    H = to_np(layer.H)
    for r in range(cfg.t):
        pr = O.shard_params(p, r, cfg.t)
        part, cm = O.mlp_rank_forward(H, pr)
        gm = O.mlp_rank_backward(cm, pr, dY)
        out = torch.empty_like(layer.H)
        layer.block_fwd(tp.TP_MLP, r, layer.H, out)
        dx = torch.empty_like(layer.H)
        layer.block_bwd(tp.TP_MLP, r, layer.H, to_dev(dY, cfg), dx)
        torch.cuda.synchronize()
        assert_close(f"mlp partial r={r}", to_np(out), part, tol)
        assert_close(f"mlp dH partial r={r}", to_np(dx), gm["dH"], tol)


def test_layer_is_deterministic():
    cfg = SMALL["bf16_ragged"]
    a, _, _ = full_layer_gpu(cfg)
    b, _, _ = full_layer_gpu(cfg)
    for x, y in ((a.Y, b.Y), (a.dX, b.dX), (a.grads[1]["attn"][0], b.grads[1]["attn"][0]),
                 (a.grads[0]["mlp"][1], b.grads[0]["mlp"][1])):
        assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# full-size shapes, rank 0, in the launch configuration the benchmark times.
# The attention block is compared over the whole sequence with a dense
# upstream gradient; the MLP is token-wise, so a sample of rows (with dY zero
# elsewhere) is checked exactly.
# ---------------------------------------------------------------------------

FULL = ["gpt_1.7b", "gpt_18b", "gpt_175b", "gpt_1t"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_rank0_attention(name):
    """Rank 0's attention block at full size, every one of the s query rows of
    the forward partial and a dense dH, so every gradient carries the late
    queries' contributions: the online softmax over the longest causal ranges
    (s / 64 key tiles: whole in one workgroup at 1.7B, merged from chunks of 8
    tiles at 18B, 175B and 1T) and the chunk merges of dK, dV and dQ
    ("parallelism" blog, "How the softmax stays exact: the online softmax";
    causal visibility as in its "Context parallelism" section)."""
    cfg = I.CONFIGS[name]
    print(f"full-size attention {name} rank 0, all {cfg.s} query rows, dense dH", flush=True)
    h, a, s, b, t = cfg.h, cfg.a, cfg.s, cfg.b, cfg.t
    dt = dtype_code(cfg)
    parts = I.params_rank(cfg, 0)
    w = weights_from_parts(parts, dt)["attn"]
    X = I.activation(cfg, "X")
    dH = I.activation(cfg, "dY")
    Xd, dHd = to_dev(X, cfg), to_dev(dH, cfg)
    saved = torch.empty(tp.tp_saved_bytes(h, a, s, b, t, dt, tp.TP_ATTN), dtype=torch.uint8, device="cuda")
    ws = torch.empty(tp.tp_workspace_bytes(h, a, s, b, t, dt, tp.TP_ATTN), dtype=torch.uint8, device="cuda")
    y = torch.full_like(Xd, float("nan"))
    dx = torch.full_like(Xd, float("nan"))
    grads = tuple(torch.full(shp, float("nan"), dtype=Xd.dtype, device="cuda")
                  for shp in tp.block_shapes(h, t, tp.TP_ATTN))
    tp.tp_layer_fwd(h, a, s, b, t, 0, dt, tp.TP_ATTN, Xd, w, y, saved, ws)
    tp.tp_layer_bwd(h, a, s, b, t, 0, dt, tp.TP_ATTN, Xd, w, saved, dHd, dx, grads, ws)
    torch.cuda.synchronize()
    yg, dxg = to_np(y), to_np(dx)
    gg = [to_np(g_) for g_ in grads]
    del saved, ws, y, dx, grads, Xd, dHd
    torch.cuda.empty_cache()

    pr = {k: v.astype(np.float64) for k, v in parts.items()}
    del parts
    ar = a // t
    part, cache = O.attention_rank_forward(X, pr, s, b, ar)
    gr = O.attention_rank_backward(cache, pr, dH, s, b, ar)
    del cache
    tol = TOL[cfg.dtype]
    report = {}
    assert_close("partial", yg, part, tol, report)
    assert_close("dX", dxg, gr["dX"], tol, report)
    assert_close("dWqkv", gg[0], np.concatenate([gr["dWq"], gr["dWk"], gr["dWv"]], axis=1), tol, report)
    assert_close("dbqkv", gg[1], np.concatenate([gr["dbq"], gr["dbk"], gr["dbv"]]), tol, report)
    assert_close("dWo", gg[2], gr["dWo"], tol, report)
    assert_close("dbo", gg[3], gr["dbo"], tol, report)
    # the last query rows (the longest causal ranges) on their own
    last = slice((s - 128) * b, s * b)
    assert_close("partial[last 128 queries]", yg[last], part[last], tol, report)
    assert_close("dX[last 128 queries]", dxg[last], gr["dX"][last], tol, report)
    print({k: f"{v:.2e}" for k, v in report.items()}, flush=True)


@pytest.mark.parametrize("name", FULL)
def test_full_size_rank0_mlp(name):
    cfg = I.CONFIGS[name]
    h, a, s, b, t = cfg.h, cfg.a, cfg.s, cfg.b, cfg.t
    T = s * b
    print(f"full-size MLP {name} rank 0", flush=True)
    dt = dtype_code(cfg)
    parts = I.params_rank(cfg, 0)
    w = weights_from_parts(parts, dt)["mlp"]
    Hin = I.activation(cfg, "H")
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, size=61, replace=False)]))
    dY = np.zeros_like(Hin)
    dY[rows] = I.activation(cfg, "dY")[rows]
    Hd, dYd = to_dev(Hin, cfg), to_dev(dY, cfg)
    saved = torch.empty(tp.tp_saved_bytes(h, a, s, b, t, dt, tp.TP_MLP), dtype=torch.uint8, device="cuda")
    ws = torch.empty(tp.tp_workspace_bytes(h, a, s, b, t, dt, tp.TP_MLP), dtype=torch.uint8, device="cuda")
    y = torch.full_like(Hd, float("nan"))
    dx = torch.full_like(Hd, float("nan"))
    grads = tuple(torch.full(shp, float("nan"), dtype=Hd.dtype, device="cuda")
                  for shp in tp.block_shapes(h, t, tp.TP_MLP))
    tp.tp_layer_fwd(h, a, s, b, t, 0, dt, tp.TP_MLP, Hd, w, y, saved, ws)
    tp.tp_layer_bwd(h, a, s, b, t, 0, dt, tp.TP_MLP, Hd, w, saved, dYd, dx, grads, ws)
    torch.cuda.synchronize()

    pr = {k: v.astype(np.float64) for k, v in parts.items()}
    part, cm = O.mlp_rank_forward(Hin[rows], pr)
    gm = O.mlp_rank_backward(cm, pr, dY[rows])
    tol = TOL[cfg.dtype]
    yg = to_np(y)
    assert np.all(np.isfinite(yg))
    assert_close("partial[rows]", yg[rows], part, tol)
    dxg = to_np(dx)
    assert_close("dH[rows]", dxg[rows], gm["dH"], tol)
    others = np.setdiff1d(np.arange(T), rows)
    assert np.all(dxg[others] == 0.0)
    assert_close("dW1", to_np(grads[0]), gm["dW1"], tol)
    assert_close("db1", to_np(grads[1]), gm["db1"], tol)
    assert_close("dW2", to_np(grads[2]), gm["dW2"], tol)
    assert_close("db2", to_np(grads[3]), gm["db2"], tol)


def test_stand_in_reduce_is_the_elementwise_sum():
    """'parallelism' blog, 'First: the three collectives': [1,2,3,4] + [10,20,30,40]."""
    for dt in (tp.TP_BF16, tp.TP_FP32):
        td = tp.torch_dtype(dt)
        parts = torch.tensor([[[1, 2, 3, 4, 0, 0, 0, 0]], [[10, 20, 30, 40, 0, 0, 0, 0]]], dtype=td, device="cuda")
        out = torch.empty((1, 8), dtype=td, device="cuda")
        tp.tp_reduce_partials(dt, parts, out)
        torch.cuda.synchronize()
        assert out.float().cpu().tolist() == [[11, 22, 33, 44, 0, 0, 0, 0]]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_reduce_with_bias_and_residual_matches_block_output(dtype):
    cfg = I.make_config("reduce", 64, 4, 32, 2, 3, dtype)
    rng = np.random.default_rng(9)
    rows, cols, t = 200, 72, 3
    parts = [rng.standard_normal((rows, cols)).astype(np.float32) for _ in range(t)]
    bias = rng.standard_normal(cols).astype(np.float32)
    res = rng.standard_normal((rows, cols)).astype(np.float32)
    if dtype == "bf16":
        parts = [I.round_to_bf16(x) for x in parts]
        bias, res = I.round_to_bf16(bias), I.round_to_bf16(res)
    ref = O.block_output(parts, bias, res)
    out = torch.empty((rows, cols), dtype=tp.torch_dtype(dtype_code(cfg)), device="cuda")
    tp.tp_reduce_partials(dtype_code(cfg), to_dev(np.stack(parts), cfg), out, bias=to_dev(bias, cfg),
                          residual=to_dev(res, cfg))
    torch.cuda.synchronize()
    # fp32 sum, one rounding to the storage type
    assert rel_err(to_np(out), ref) <= (4e-3 if dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_d48"])
def test_profiler_attributes_every_role(name):
    cfg = SMALL[name]
    tp.tp_prof_enable(True)
    full_layer_gpu(cfg)
    tp.tp_prof_enable(False)
    prof = tp.tp_prof_read()
    roles = {"qkv_fwd", "o_fwd", "fc1_fwd", "fc2_fwd", "rowdot", "reduce"}
    roles |= attention_roles(cfg)
    # the fused and the materialised attention never both run
    other = {"attn_fwd", "attn_dkv", "attn_dq", "scores", "softmax", "pv", "ds", "dv", "dq", "dk"} - roles
    assert not (other & set(prof)), other & set(prof)
    # a weight's input- and weight-gradient GEMMs run as one grouped launch
    # when both take whole 64-deep K steps, else as two launches; the grouped
    # launch also forms the bias gradient (column sums of its weight-gradient
    # operand), else a column-sum kernel does
    for w, db in (("fc2", "db2"), ("fc1", "db1"), ("o", "dbo"), ("qkv", "dbqkv")):
        grouped = f"{w}_dgrad+wgrad"
        if grouped in prof:
            roles |= {grouped}
            assert db not in prof, db
        else:
            roles |= {f"{w}_dgrad", f"{w}_wgrad", db}
    assert roles <= set(prof)
    for name in roles - {"reduce"}:
        assert prof[name]["launches"] == cfg.t, name
        assert prof[name]["ms"] > 0
    assert prof["reduce"]["launches"] == 4
    T, h, t = cfg.tokens, cfg.h, cfg.t
    assert prof["fc1_fwd"]["flops"] == pytest.approx(t * 2.0 * T * (4 * h // t) * h)


# ---------------------------------------------------------------------------
# GELU and GELU' epilogues, element by element over a wide input range
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_gelu_epilogues_element_by_element(dtype):
    """Rank 1 of an MLP block whose FC1 weight is zero, so U = b1, and whose
    FC2 weight shard is a partial identity, so the block output holds
    Z = GELU(b1) column by column; with dY = 1/T in every row the FC1 bias
    gradient is sum_tokens dU = GELU'(b1) (a power-of-two scale commutes with
    rounding). b1 spans [-8, 8], tails included. Reference: the oracle's exact
    (erf-form) GELU and GELU' on the same (rounded) b1."""
    from megatron_tensor_layer_amd.layer import TPLayer
    h, a, s, b, t = 256, 2, 64, 2, 2
    T, fr = s * b, 4 * h // t
    code = tp.TP_BF16 if dtype == "bf16" else tp.TP_FP32
    dt = tp.torch_dtype(code)
    b1 = torch.zeros(fr, dtype=dt, device="cuda")
    b1[:h] = torch.linspace(-8.0, 8.0, h, device="cuda")
    w2 = torch.zeros((fr, h), dtype=dt, device="cuda")
    w2[torch.arange(h), torch.arange(h)] = 1.0
    mlp = (torch.zeros((h, fr), dtype=dt, device="cuda"), b1, w2, torch.zeros(h, dtype=dt, device="cuda"))
    attn = tuple(torch.zeros(shp, dtype=dt, device="cuda") for shp in tp.block_shapes(h, t, tp.TP_ATTN))
    layer = TPLayer(h, a, s, b, t, code, [{"attn": attn, "mlp": mlp} for _ in range(t)])
    x = torch.randn((T, h), device="cuda").to(dt)
    out = torch.empty((T, h), dtype=dt, device="cuda")
    layer.block_fwd(tp.TP_MLP, 1, x, out)
    dy = torch.full((T, h), 1.0 / T, dtype=dt, device="cuda")
    dx = torch.empty_like(out)
    layer.block_bwd(tp.TP_MLP, 1, x, dy, dx)
    torch.cuda.synchronize()
    u = to_np(b1[:h])
    # the device's Phi is within 3e-7 of the exact one (times |x| <= 8 in GELU);
    # bf16 adds one rounding of the output (2^-8 relative); fp32 adds the fixed-
    # order fp32 sum of the 128 token rows in the bias gradient
    rel, floor = (2.0 ** -8, 4e-7 * 8) if dtype == "bf16" else (1e-5, 4e-7 * 8)
    z = to_np(out)
    ref_z = O.gelu(u)
    assert np.all(np.abs(z - ref_z[None, :]) <= rel * np.abs(ref_z)[None, :] + floor), "GELU"
    g = to_np(layer.grads[1]["mlp"][1][:h])
    ref_g = O.gelu_grad(u)
    assert np.all(np.abs(g - ref_g) <= rel * np.abs(ref_g) + floor), "GELU'"

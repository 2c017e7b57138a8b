"""Benchmark: one tensor-parallel rank's share of a GPT layer, forward +
backward, on one MI355X.

A step is one pass of the whole layer over one batch: the t ranks' calls
(attention fwd, MLP fwd, MLP bwd, attention bwd) run one after another on
one GPU, with the stand-in all-reduce (fused with the bias + residual add)
between the blocks.  The metric is model TFLOP/s per GPU for one rank's
share:

    F_rank = 72 b s h^2 (1 + s / 6h) / t      (paper-graph page, "FLOP Counting
                                               and Training Time Estimation",
                                               Eq. 3 for one layer, no
                                               recomputation, no logit layer)
    t_rank = (time of all t ranks' calls, stand-in reductions excluded) / t
    value  = F_rank / t_rank

Inputs are synthetic and seeded: weights and biases N(0, 0.02^2), X and dY
N(0, 1), drawn on the GPU by torch's generator and stored in bf16.

Two more forms of the same layer are timed beside it and reported as objects
of the same line: the pre-norm layer with sequence parallelism (LayerNorm,
bias and residual on each rank's T/t tokens; "sequence_parallel_layernorm")
and the backward with full activation recomputation ("recompute", counted
with the page's 96 b s h^2 (1 + s/6h) per layer as well as by executed
products).

The other layer shapes (1.7B, 18B, 1T) are timed the same way, fewer steps,
and reported under "shapes".

    python bench.py [--steps K] [--warmup W] [--config gpt_175b] [--no-cpu-baseline] [--no-modes]
                    [--no-shapes]

Prints one JSON line.  Only one GPU is used: --gpus above 1 is refused.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 dense bf16 FLOP/clk x 2.4 GHz (AMD MI355X spec)
PEAK_HBM_GBPS = 8000.0      # HBM3E, AMD MI355X spec
DEFAULT_CONFIG = "gpt_175b"

# A plain elementwise copy of known size (fp32 negation, COPY_BYTES read and
# COPY_BYTES written), launched once before the warm-up so that a counter
# run of this script sees the copy beside the layer's kernels and can scale
# FETCH_SIZE / WRITE_SIZE to bytes.
COPY_BYTES = 1 << 30

# Sources of the GEMM kernels and their launch plan: a traffic figure taken
# from counters is reported only while these files are unchanged.
KERNEL_SOURCES = ("megatron_tensor_layer_amd/csrc/gemm.hpp", "megatron_tensor_layer_amd/csrc/gemm_direct.hpp",
                  "megatron_tensor_layer_amd/csrc/tp_common.hpp", "megatron_tensor_layer_amd/csrc/tp_layer.hip")


def kernel_sources_digest():
    import hashlib
    hs = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            hs.update(f.read())
    return hs.hexdigest()


def measured_traffic(config, role):
    """HBM bytes per launch of `role` from the committed counter summary
    profiles/<config>_<role>_traffic.txt ('+' in the role written '_'), or
    None when there is no summary for this role or the kernel sources changed
    since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{config}_{role.replace('+', '_')}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("role") != role or kv.get("kernel_sources_sha256") != kernel_sources_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def model_flops_per_rank(h, s, b, t):
    return 72.0 * b * s * h * h * (1.0 + s / (6.0 * h)) / t


def build_layer(cfg, seed=1234):
    import torch
    from megatron_tensor_layer_amd import tplayer as tp
    from megatron_tensor_layer_amd.layer import TPLayer

    h, a, s, b, t = cfg.h, cfg.a, cfg.s, cfg.b, cfg.t
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)

    def rnd(shape, std):
        x = torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32)
        return (x * std).to(torch.bfloat16)

    weights = []
    for _ in range(t):
        w = {}
        for name, blk in (("attn", tp.TP_ATTN), ("mlp", tp.TP_MLP)):
            w[name] = tuple(rnd(shp, 0.02) for shp in tp.block_shapes(h, t, blk))
        weights.append(w)
    layer = TPLayer(h, a, s, b, t, tp.TP_BF16, weights)
    X = rnd((s * b, h), 1.0)
    dY = rnd((s * b, h), 1.0)
    return layer, X, dY


def timed_steps(layer, X, dY, steps):
    """Per step: HIP events (torch's current stream, the stream the library
    launches on) around each block's rank loop and each stand-in reduction."""
    import torch
    from megatron_tensor_layer_amd import tplayer as tp

    t = layer.t
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(9)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        e = ev[k]
        e[0].record()
        for r in range(t):
            layer.block_fwd(tp.TP_ATTN, r, X, layer.partials[r])
        e[1].record()
        layer.reduce(layer.H, layer.weights[0]["attn"][3], X)
        e[2].record()
        for r in range(t):
            layer.block_fwd(tp.TP_MLP, r, layer.H, layer.partials[r])
        e[3].record()
        layer.reduce(layer.Y, layer.weights[0]["mlp"][3], layer.H)
        e[4].record()
        for r in range(t):
            layer.block_bwd(tp.TP_MLP, r, layer.H, dY, layer.partials[r])
        e[5].record()
        layer.reduce(layer.dH, None, dY)
        e[6].record()
        for r in range(t):
            layer.block_bwd(tp.TP_ATTN, r, X, layer.dH, layer.partials[r])
        e[7].record()
        layer.reduce(layer.dX, None, layer.dH)
        e[8].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = [[ev[k][i].elapsed_time(ev[k][i + 1]) for i in range(8)] for k in range(steps)]
    return seg, wall


def segment_times(steps, segs):
    """Run `steps` passes of the (fn, counted) segments with HIP events
    (torch's current stream, the library's stream) around each; returns the
    per-step milliseconds of the counted and of the other segments."""
    import torch

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(segs) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record()
        for i, (fn, _) in enumerate(segs):
            fn()
            ev[k][i + 1].record()
    torch.cuda.synchronize()
    counted, other, per_seg = [], [], [0.0] * len(segs)
    for k in range(steps):
        c = o = 0.0
        for i, (_, cnt) in enumerate(segs):
            ms = ev[k][i].elapsed_time(ev[k][i + 1])
            per_seg[i] += ms / steps
            if cnt:
                c += ms
            else:
                o += ms
        counted.append(c)
        other.append(o)
    return counted, other, per_seg


def recompute_flops_per_rank(cfg):
    """Matmul FLOPs the recomputing backward re-runs per rank: the QKV and FC1
    products and the two attention products of the forward (the output
    products are not re-run: the backward does not read their results)."""
    h, a, s, b, t = cfg.h, cfg.a, cfg.s, cfg.b, cfg.t
    T = s * b
    return 2.0 * T * h * (3 * h // t) + 2.0 * T * h * (4 * h // t) + 2 * 2.0 * b * (a // t) * s * s * (h // a)


def measure_recompute(layer, X, dY, cfg, steps, warmup):
    """The layer with full activation recomputation: forward of both blocks
    keeps nothing, each backward re-runs its block's forward first."""
    import numpy as np
    from megatron_tensor_layer_amd import tplayer as tp
    from megatron_tensor_layer_amd.layer import TPLayer

    h, a, s, b, t = cfg.h, cfg.a, cfg.s, cfg.b, cfg.t
    rl = TPLayer(h, a, s, b, t, tp.TP_BF16, layer.weights, recompute=True)
    for _ in range(warmup):
        rl.forward(X)
        rl.backward(dY)
    segs = [(lambda: [rl.block_fwd(tp.TP_ATTN, r, X, rl.partials[r]) for r in range(t)], True),
            (lambda: rl.reduce(rl.H, rl.weights[0]["attn"][3], X), False),
            (lambda: [rl.block_fwd(tp.TP_MLP, r, rl.H, rl.partials[r]) for r in range(t)], True),
            (lambda: rl.reduce(rl.Y, rl.weights[0]["mlp"][3], rl.H), False),
            (lambda: [rl.block_bwd(tp.TP_MLP, r, rl.H, dY, rl.partials[r]) for r in range(t)], True),
            (lambda: rl.reduce(rl.dH, None, dY), False),
            (lambda: [rl.block_bwd(tp.TP_ATTN, r, X, rl.dH, rl.partials[r]) for r in range(t)], True),
            (lambda: rl.reduce(rl.dX, None, rl.dH), False)]
    counted, _, _ = segment_times(steps, segs)
    t_rank = float(np.mean(counted)) / t
    F = model_flops_per_rank(h, s, b, t)
    F96 = F * 96.0 / 72.0
    Fx = F + recompute_flops_per_rank(cfg)
    saved_bytes = sum(tp.tp_saved_bytes(h, a, s, b, t, tp.TP_BF16, blk) for blk in (tp.TP_ATTN, tp.TP_MLP))
    out = {"rank_ms": round(t_rank, 4),
           "model_tflops_96": round(F96 / (t_rank * 1e-3) / 1e12, 1),
           "pct_of_peak_96": round(100.0 * F96 / (t_rank * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "executed_tflops": round(Fx / (t_rank * 1e-3) / 1e12, 1),
           "flops_per_rank_96": F96, "flops_per_rank_executed": Fx,
           "activation_bytes_kept_per_rank_layer": 0, "activation_bytes_kept_without_recompute": saved_bytes,
           "scratch_bytes_shared": int(rl.scratch.numel()),
           "accounting": "model TFLOP/s with the paper-graph page's 96 b s h^2 (1 + s/6h) per layer (one extra "
                         "forward counted in full); executed counts the products actually re-run"}
    del rl
    return out


def ln_graph_ms(fns, reps=20):
    """GPU milliseconds of each fn (a batch of library launches) replayed from a
    captured HIP graph, or None where capture is not possible."""
    import torch

    out = []
    for fn in fns:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / reps)
            del g
        except Exception:  # pragma: no cover - capture unsupported
            torch.cuda.synchronize()
            out.append(None)
    return out


def measure_sequence_parallel(layer, X, dY, cfg, steps, warmup):
    """The pre-norm layer with sequence parallelism: LayerNorms, output
    biases and residual adds on each rank's T/t tokens (rank work), the
    stand-in sums between them (not counted)."""
    import numpy as np
    import torch
    from megatron_tensor_layer_amd import tplayer as tp
    from megatron_tensor_layer_amd.layer import SPLayer

    h, a, s, b, t = cfg.h, cfg.a, cfg.s, cfg.b, cfg.t
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    ln = ((1.0 + 0.1 * torch.randn(h, generator=g, device="cuda")).to(torch.bfloat16),
          (0.02 * torch.randn(h, generator=g, device="cuda")).to(torch.bfloat16),
          (1.0 + 0.1 * torch.randn(h, generator=g, device="cuda")).to(torch.bfloat16),
          (0.02 * torch.randn(h, generator=g, device="cuda")).to(torch.bfloat16))
    sp = SPLayer(h, a, s, b, t, tp.TP_BF16, layer.weights, ln)
    for _ in range(warmup):
        sp.forward(X)
        sp.backward(dY)
    R = range(t)
    segs = [(lambda: [sp.ln1_fwd(r, X) for r in R], True),
            (lambda: [sp.block_fwd(tp.TP_ATTN, r, sp.A, sp.partials[r]) for r in R], True),
            (sp.reduce_sum, False),
            (lambda: [sp.add_ln2_fwd(r, X) for r in R], True),
            (lambda: [sp.block_fwd(tp.TP_MLP, r, sp.B, sp.partials[r]) for r in R], True),
            (sp.reduce_sum, False),
            (lambda: [sp.add_out_fwd(r) for r in R], True),
            (lambda: [sp.block_bwd(tp.TP_MLP, r, sp.B, dY, sp.partials[r]) for r in R], True),
            (sp.reduce_sum, False),
            (lambda: [sp.ln2_bwd(r, dY) for r in R], True),
            (lambda: [sp.block_bwd(tp.TP_ATTN, r, sp.A, sp.dH, sp.partials[r]) for r in R], True),
            (sp.reduce_sum, False),
            (lambda: [sp.ln1_bwd(r, X) for r in R], True),
            (sp.reduce_ln_grads, False)]
    counted, other, per_seg = segment_times(steps, segs)
    t_rank = float(np.mean(counted)) / t
    F = model_flops_per_rank(h, s, b, t)
    # LayerNorm calls: each segment holds the t ranks' launches of one call;
    # algorithmic bytes: every [T/t, h] operand once, the [h] vectors once,
    # 8 bytes of statistics per row
    n, es = s * b // t, 2.0
    calls = {"ln1_fwd (LN1 of the block input)": (0, es * (2 * n * h + 2 * h) + 8 * n),
             "add_ln2_fwd (bias + residual + LN2)": (3, es * (4 * n * h + 3 * h) + 8 * n),
             "add_out_fwd (bias + residual)": (6, es * (3 * n * h + h)),
             "ln2_bwd (dx + residual grad, dgamma, dbeta)": (9, es * (4 * n * h + 3 * h) + 8 * n),
             "ln1_bwd (dx + residual grad, dgamma, dbeta)": (12, es * (4 * n * h + 3 * h) + 8 * n)}
    # The calls are a few microseconds each, shorter than a Python launch, so
    # the step above is partly host-bound there. Their GPU time is taken by
    # replaying each segment's t launches from a HIP graph (no host in the
    # loop); the segment timing is kept beside it.
    graph_ms = ln_graph_ms([segs[i][0] for i, _ in calls.values()], reps=20)
    kernels = {}
    for (name, (i, nbytes)), gms in zip(calls.items(), graph_ms):
        ms = gms / t if gms is not None else per_seg[i] / t
        gbps = nbytes / (ms * 1e-3) / 1e9
        kernels[name] = {"ms_per_call": round(ms, 5), "timing": "graph replay" if gms is not None else "events",
                         "ms_per_call_in_step": round(per_seg[i] / t, 5), "bound": "hbm",
                         "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": nbytes}
    out = {"rank_ms": round(t_rank, 4), "model_tflops": round(F / (t_rank * 1e-3) / 1e12, 1),
           "pct_of_peak": round(100.0 * F / (t_rank * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "rows_per_rank": s * b // t, "standin_ms_per_step": round(float(np.mean(other)), 4),
           "layernorm_calls": kernels,
           "layernorm_ms_per_rank": round(sum(per_seg[i] for i, _ in calls.values()) / t, 4),
           "note": "pre-norm layer: the same products plus LayerNorm fwd/bwd, bias and residual on T/t rows"}
    del sp
    return out


def host_info():
    """Host cores this process may use and the BLAS library numpy calls."""
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            d = libs[0]
            blas = {"internal_api": d.get("internal_api"), "version": d.get("version"),
                    "filepath": d.get("filepath"), "num_threads": d.get("num_threads")}
    except Exception:  # pragma: no cover
        pass
    return {"host_cores": cores, "os_cpu_count": os.cpu_count(), "blas": blas}


def _oracle_layer_pass(cfg, pr, ar, L, t_eff):
    """One fwd + bwd pass of the oracle over the first L tokens of each
    sequence: rank 0's share (t_eff = cfg.t, rank weights) or the unsharded
    layer (t_eff = 1, full-width weights). Returns seconds."""
    import numpy as np
    from megatron_tensor_layer_amd import inputs as I
    from oracle import tp_layer_oracle as O

    T = L * cfg.b
    X = I.activation(cfg, "X", tokens=T).astype(np.float64)
    dY = I.activation(cfg, "dY", tokens=T).astype(np.float64)
    t0 = time.perf_counter()
    if t_eff == 1:
        Y, cache = O.layer_forward(X, pr, L, cfg.b, cfg.a)
        O.layer_backward(cache, pr, dY, L, cfg.b, cfg.a)
    else:
        pa, ca = O.attention_rank_forward(X, pr, L, cfg.b, ar)
        H = O.block_output([pa], pr["bo"], X)
        pm, cm = O.mlp_rank_forward(H, pr)
        gm = O.mlp_rank_backward(cm, pr, dY)
        dH = O.block_output([gm["dH"]], residual=dY)
        O.attention_rank_backward(ca, pr, dH, L, cfg.b, ar)
    return time.perf_counter() - t0


def _timed_sample(cfg, pr, ar, t_eff, target_s):
    """Doubles L from 64 until a pass takes target_s / 3 (or L = s); repeats
    the last L to about target_s / 1.5 of CPU time. Returns (L, mean s, passes)."""
    L = 64
    el = _oracle_layer_pass(cfg, pr, ar, L, t_eff)
    while el < target_s / 3 and L * 2 <= cfg.s:
        L *= 2
        el = _oracle_layer_pass(cfg, pr, ar, L, t_eff)
    times = [el]
    while sum(times) < target_s / 1.5 and len(times) < 8:
        times.append(_oracle_layer_pass(cfg, pr, ar, L, t_eff))
    return L, sum(times) / len(times), len(times)


def cpu_baseline(cfg, target_s=15.0):
    """The fp64 oracle (as it stands) on bounded samples of the same
    workload, fwd + bwd of both blocks over the first L tokens of each
    sequence, FLOPs by the same formula:
      * rank 0's share (the reported value; like for like with the GPU's
        per-rank time);
      * the unsharded layer (all t ranks' work in one pass; its weights are
        rank 0's shards repeated t times along the split axes, which gives
        the oracle the same work as the drawn unsharded weights);
      * the fp32 check configuration on one BLAS thread."""
    import numpy as np
    from megatron_tensor_layer_amd import inputs as I

    info = host_info()
    threads = (info["blas"] or {}).get("num_threads") or info["host_cores"]
    parts = I.params_rank(cfg, 0)
    pr = {k: v.astype(np.float64) for k, v in parts.items()}
    del parts
    ar = cfg.a // cfg.t
    L, el, passes = _timed_sample(cfg, pr, ar, cfg.t, target_s)
    flops = model_flops_per_rank(cfg.h, L, cfg.b, cfg.t)
    out = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "seconds": round(el, 3), "passes": passes,
           "sample": f"rank 0 of t={cfg.t}, fwd+bwd of both blocks, first {L} of {cfg.s} tokens x b={cfg.b}, "
                     f"mean of {passes} passes (numpy float64, {threads} BLAS threads); "
                     f"FLOPs = 72 b L h^2 (1 + L/6h) / t",
           "host": info}

    # the unsharded layer: full-width weights from rank 0's shards
    t = cfg.t
    full = {}
    for k in ("Wq", "Wk", "Wv", "W1"):
        full[k] = np.tile(pr[k], (1, t))
    for k in ("bq", "bk", "bv", "b1"):
        full[k] = np.tile(pr[k], t)
    for k in ("Wo", "W2"):
        full[k] = np.tile(pr[k], (t, 1))
    full["bo"], full["b2"] = pr["bo"], pr["b2"]
    del pr
    Lu, elu, pu = _timed_sample(cfg, full, cfg.a, 1, target_s * 2 / 3)
    del full
    fu = model_flops_per_rank(cfg.h, Lu, cfg.b, 1)
    out["unsharded_layer"] = {
        "value": round(fu / elu / 1e12, 4), "unit": "TFLOP/s", "seconds": round(elu, 3), "passes": pu,
        "tokens": Lu * cfg.b,
        "sample": f"whole layer (h={cfg.h}, a={cfg.a}, unsharded), fwd+bwd, first {Lu} of {cfg.s} tokens x "
                  f"b={cfg.b}; FLOPs = 72 b L h^2 (1 + L/6h)"}

    # the fp32 check configuration, single-threaded
    chk = I.CONFIGS["check_fp32"]
    pc = {k: v.astype(np.float64) for k, v in I.params_full(chk).items()}
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    try:
        reps, tot = 0, 0.0
        while tot < 1.0 and reps < 2000:
            tot += _oracle_layer_pass(chk, pc, chk.a, chk.s, 1)
            reps += 1
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    fc = model_flops_per_rank(chk.h, chk.s, chk.b, 1)
    out["check_fp32_single_thread"] = {
        "ms_per_pass": round(1e3 * tot / reps, 4), "passes": reps, "gflops": round(fc / (tot / reps) / 1e9, 3),
        "sample": f"fp32 check configuration (h={chk.h}, a={chk.a}, s={chk.s}, b={chk.b}), whole layer unsharded, "
                  "fwd+bwd, one BLAS thread"}
    return out


def measure_shape(name, steps, warmup):
    """Per-rank throughput of another layer shape, same protocol as the
    headline figure (stand-in reductions excluded), plus its dominant GEMM
    role from one profiled step."""
    import numpy as np
    import torch
    from megatron_tensor_layer_amd import inputs as I
    from megatron_tensor_layer_amd import tplayer as tp

    cfg = I.CONFIGS[name]
    layer, X, dY = build_layer(cfg)
    for _ in range(warmup):
        layer.forward(X)
        layer.backward(dY)
    seg, _ = timed_steps(layer, X, dY, steps)
    seg = np.array(seg)
    rank_loops = seg[:, [0, 2, 4, 6]].sum(axis=1)
    t_rank = float(np.mean(rank_loops)) / cfg.t
    F = model_flops_per_rank(cfg.h, cfg.s, cfg.b, cfg.t)
    tp.tp_prof_enable(True)
    layer.forward(X)
    layer.backward(dY)
    tp.tp_prof_enable(False)
    prof = tp.tp_prof_read()
    gemm = {k: v for k, v in prof.items() if k not in NON_GEMM_ROLES}
    dom = max(gemm, key=lambda k: gemm[k]["ms"])
    de = prof[dom]
    out = {"workload": f"{cfg.name} layer shard: h={cfg.h}, a={cfg.a}, s={cfg.s}, b={cfg.b}, t={cfg.t}",
           "value": round(F / (t_rank * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
           "pct_of_peak": round(100.0 * F / (t_rank * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "rank_ms": round(t_rank, 4), "rank_ms_min": round(float(np.min(rank_loops)) / cfg.t, 4),
           "steps": steps, "flops_per_rank": F,
           "dominant": {"role": dom, "ms_per_launch": round(de["ms"] / de["launches"], 4),
                        "tflops": round(de["flops"] / (de["ms"] * 1e-3) / 1e12, 1)}}
    del layer, X, dY
    torch.cuda.empty_cache()
    return out


NON_GEMM_ROLES = ("softmax", "rowdot", "reduce", "db1", "db2", "dbo", "dbqkv", "ln_fwd", "ln_bwd")
OTHER_SHAPES = ("gpt_1.7b", "gpt_18b", "gpt_1t")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the sequence-parallel LayerNorm and recompute measurements")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the other layer shapes (1.7B, 18B, 1T) reported under 'shapes'")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the t tensor-parallel ranks "
              "run one after another on a single MI355X and no collectives run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from megatron_tensor_layer_amd import inputs as I
    from megatron_tensor_layer_amd import tplayer as tp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tp.lib()
    cfg = I.CONFIGS[args.config]
    h, a, s, b, t = cfg.h, cfg.a, cfg.s, cfg.b, cfg.t
    layer, X, dY = build_layer(cfg)
    copy_calibration()
    for _ in range(args.warmup):
        layer.forward(X)
        layer.backward(dY)
    torch.cuda.synchronize()

    seg, wall = timed_steps(layer, X, dY, args.steps)
    seg = np.array(seg)
    rank_loops = seg[:, [0, 2, 4, 6]].sum(axis=1)          # ms per step, all t ranks
    standin = seg[:, [1, 3, 5, 7]].sum(axis=1)
    step_ms = seg.sum(axis=1)
    t_rank = float(np.mean(rank_loops)) / t
    F_rank = model_flops_per_rank(h, s, b, t)
    tflops = F_rank / (t_rank * 1e-3) / 1e12

    # per-role kernel times from the library's event profiler, one extra step
    tp.tp_prof_enable(True)
    layer.forward(X)
    layer.backward(dY)
    tp.tp_prof_enable(False)
    prof = tp.tp_prof_read()
    roles = {}
    for name, e in prof.items():
        roles[name] = {"launches": e["launches"], "ms_per_launch": round(e["ms"] / e["launches"], 4),
                       "tflops": round(e["flops"] / (e["ms"] * 1e-3) / 1e12, 1) if e["ms"] > 0 else None,
                       "gbps": round(e["bytes"] / (e["ms"] * 1e-3) / 1e9, 1) if e["ms"] > 0 else None}
    gemm_roles = {k: v for k, v in prof.items() if k not in NON_GEMM_ROLES}
    dom = max(gemm_roles, key=lambda k: gemm_roles[k]["ms"])
    de = prof[dom]
    per_launch_ms = de["ms"] / de["launches"]
    achieved = de["flops"] / de["launches"] / (per_launch_ms * 1e-3) / 1e12
    traffic = measured_traffic(cfg.name, dom)
    roofline = {"bound": "mfma", "kernel": f"GEMM role {dom}", "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "traffic_unit": "bytes per launch (HBM, counters)",
                "algorithmic_bytes_per_launch": de["bytes"] / de["launches"],
                "flops_per_launch": de["flops"] / de["launches"],
                "ms_per_launch": round(per_launch_ms, 4)}

    out = {
        "metric": "model TFLOP/s per GPU (layer fwd+bwd, one TP shard) and % of bf16 MFMA peak",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) weights/biases, N(0,1) X and dY, drawn on the GPU)",
        "config": {"workload": f"{cfg.name} layer shard: h={h}, a={a}, s={s}, b={b}, t={t}, fwd+bwd, causal",
                   "h": h, "a": a, "s": s, "b": b, "t": t, "global_batch": b, "seq_len": s,
                   "parallelism": f"tp{t} ranks run sequentially on one GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "rank_ms": round(t_rank, 4),
        "rank_ms_median": round(float(np.median(rank_loops)) / t, 4),
        "rank_ms_min": round(float(np.min(rank_loops)) / t, 4),
        "peak_used": {"tflops": PEAK_BF16_TFLOPS, "cus": 256, "clock_ghz": 2.4, "flop_per_clk_per_cu": 4096,
                      "cus_on_device": int(torch.cuda.get_device_properties(0).multi_processor_count),
                      "device": torch.cuda.get_device_properties(0).name},
        "standin_reduce_ms_per_step": round(float(np.mean(standin)), 4),
        "flops_per_rank": F_rank,
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "roles": roles,
        "context": "pages: 163 TFLOP/s per A100 (52% of 312) end-to-end with recompute; not this metric",
    }
    if not args.no_modes:
        n = max(3, args.steps // 2)
        out["sequence_parallel_layernorm"] = measure_sequence_parallel(layer, X, dY, cfg, n, 1)
        out["recompute"] = measure_recompute(layer, X, dY, cfg, n, 1)
    if not args.no_shapes:
        del layer, X, dY
        torch.cuda.empty_cache()
        n = max(3, args.steps // 4)
        out["shapes"] = {name: measure_shape(name, n, 2) for name in OTHER_SHAPES if name != cfg.name}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()

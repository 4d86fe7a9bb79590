#!/usr/bin/env python3
"""Throughput of one GPipe cell training step on one MI355X.

A step is the whole hot path over one mini-batch: the forward phase keeping
boundary outputs, the backward phase re-materializing every micro-batch,
float32 gradient accumulation over the micro-batches, and the RMSProp update.
Workload: one cell of a 128-layer stack cut into 16 cells -- 8 pre-LN
Transformer layers, d_model 2048, 16 heads, d_ff 8192, seq 512, causal,
N = 64 sequences in M = 32 micro-batches, bf16 with fp32 accumulation.
Inputs are synthetic (seeded normal draws), already resident in HBM when the
timed region starts.

Prints one JSON line.  `value` is tokens per second of the full step
(update included).

--workload conv_c256_b8 times the convolutional cell instead: 8 residual
blocks (3x3 conv, micro-batch BatchNorm, ReLU, 3x3 conv, BatchNorm, skip) of
256 channels on 32 x 32 NHWC images, N = 256 in M = 16 micro-batches; its
`value` is images per second.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "train tokens/sec per cell step (fwd+remat+bwd), MFMA util; peak act bytes"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# Roles of the Transformer cell's step by how many micro-batch passes of one
# layer they make per step: the forward roles run in the forward phase and in
# the re-materialization (2 L M passes), the backward roles once (L M).  The
# step runs several streams (the forward phase's lanes, the weight gradients
# beside the input-gradient chain, the next micro-batch's re-materialization),
# so a launch's timed span is its time in the step, sharing the CUs with the
# other streams' kernels.
FWD_ROLES = ("ln1_fwd", "qkv_fwd", "scores_fwd", "softmax_fwd", "pv_fwd", "attn_fwd", "out_fwd",
             "ln2_fwd", "ffn1_fwd", "ffn2_fwd")
BWD_ROLES = ("ffn2_dgrad", "ffn2_wgrad", "ffn1_dgrad", "ffn1_wgrad", "ln2_bwd", "out_dgrad",
             "out_wgrad", "dp", "dv", "softmax_bwd", "dq", "dk", "attn_dq", "qkv_dgrad",
             "qkv_wgrad", "ln1_bwd")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# HBM traffic of the GEMM roles, measured with rocprofv3's FETCH_SIZE and
# WRITE_SIZE counters (calibrated on a streaming kernel of known size) and
# stored in a profile summary together with a digest of the GEMM sources; the
# figures are used only while the sources still hash to that digest.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "counters_cell_d2048_L8_causal.md")
GEMM_SOURCES = ("common.hpp", "kernels.hpp", "gemm_impl.hpp", "gemm_dma.hpp", "gemm.hip",
                "gemm_fwd.hip", "gemm_dgrad.hip", "gemm_wgrad.hip")


def gemm_source_digest():
    """sha256 of the GEMM sources with comments and blank lines removed (edits of
    comments alone keep the measured figures)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "micro_pipelined_re_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()


def measured_traffic(role):
    """(fetch_bytes, write_bytes) per launch of `role`, or None if not measured for these sources."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"gemm_source_digest: ([0-9a-f]+)", text)
    if not m or m.group(1) != gemm_source_digest():
        return None
    m = re.search(rf"traffic {re.escape(role)}: fetch_bytes=(\d+) write_bytes=(\d+)", text)
    return (int(m.group(1)), int(m.group(2))) if m else None


# ------------------------------------------------------------------ algorithmic work per role
def role_work(cfg, n, m):
    """Per micro-batch pass of one layer: ('mfma', flops) for the contractions,
    ('hbm', bytes) for the rest (rmsprop: the whole update)."""
    b = n // m
    S, D, H, F = cfg.seq, cfg.d_model, cfg.heads, cfg.d_ff
    dh = D // H
    T = b * S
    eb = 2 if cfg.precision == "bf16" else 4
    pairs = S * (S + 1) // 2 if cfg.causal else S * S           # (query, key) pairs kept
    attn = b * H * 2 * pairs * dh
    P = cfg.param_count()
    w = {
        "qkv_fwd": ("mfma", 2 * T * 3 * D * D), "scores_fwd": ("mfma", attn),
        "pv_fwd": ("mfma", attn), "out_fwd": ("mfma", 2 * T * D * D),
        "ffn1_fwd": ("mfma", 2 * T * F * D), "ffn2_fwd": ("mfma", 2 * T * D * F),
        "ffn2_dgrad": ("mfma", 2 * T * F * D), "ffn2_wgrad": ("mfma", 2 * D * F * T),
        "ffn1_dgrad": ("mfma", 2 * T * D * F), "ffn1_wgrad": ("mfma", 2 * F * D * T),
        "out_dgrad": ("mfma", 2 * T * D * D), "out_wgrad": ("mfma", 2 * D * D * T),
        "dp": ("mfma", attn), "dv": ("mfma", attn), "dq": ("mfma", attn), "dk": ("mfma", attn),
        # fused attention: the forward's two products, the backward's four (dP, dV, dQ, dK)
        "attn_fwd": ("mfma", 2 * attn), "attn_dq": ("mfma", 4 * attn),
        "qkv_dgrad": ("mfma", 2 * T * D * 3 * D), "qkv_wgrad": ("mfma", 2 * 3 * D * D * T),
        # LayerNorm forward: read x, write y (act) and (mean, rstd)
        "ln1_fwd": ("hbm", 2 * T * D * eb + 8 * T), "ln2_fwd": ("hbm", 2 * T * D * eb + 8 * T),
        # LayerNorm backward: read dh, residual grad (f32), x (act); write dx (f32 + act)
        "ln1_bwd": ("hbm", T * D * (12 + 2 * eb) + 8 * T),
        "ln2_bwd": ("hbm", T * D * (12 + 2 * eb) + 8 * T),
        # softmax: read the kept scores (f32), write full rows of P
        "softmax_fwd": ("hbm", b * H * (4 * pairs + eb * S * S)),
        "softmax_bwd": ("hbm", b * H * ((4 + eb) * pairs + eb * S * S)),
        # MSE: read y, t; write dy (f32 + act)
        "mse": ("hbm", T * D * (3 * eb + 4)),
        # RMSProp: read w, g, ms; write w, ms (+ bf16 copy)
        "rmsprop": ("hbm", P * (20 + (2 if eb == 2 else 0))),
    }
    return w


def step_mfma_flops(cfg, n, m):
    """Algorithmic MFMA work of one Transformer-cell step: per layer and micro-batch
    the forward and the re-materialized forward (linears + the two attention
    products each), the input- and weight-gradient linears (twice the forward's)
    and the four attention-gradient products."""
    w = role_work(cfg, n, m)
    lin = sum(w[k][1] for k in ("qkv_fwd", "out_fwd", "ffn1_fwd", "ffn2_fwd"))
    attn = w["scores_fwd"][1]
    return cfg.layers * m * (4 * lin + 8 * attn)


def conv_role_work(cfg, n, m):
    """conv cell, per micro-batch pass of one block's convolution or BatchNorm:
    ('mfma', flops) or ('hbm', bytes).  The convolutions' algorithmic work is
    2 P C 9C whatever the operand storage (a bf16 cell's split forward operands
    double the forward's MFMA work, not its algorithmic work).  Activations
    are float32 or split bf16 pairs (4 B per element) in the forward."""
    P = (n // m) * cfg.height * cfg.width          # pixels per micro-batch
    C = cfg.channels
    eb = 2 if cfg.precision == "bf16" else 4
    g = 2 * P * C * 9 * C
    return {
        "conv_fwd": ("mfma", g), "conv_dgrad": ("mfma", g), "conv_wgrad": ("mfma", g),
        "conv_fwd_implicit": ("mfma", g), "conv_dgrad_implicit": ("mfma", g),
        "conv_wgrad_implicit": ("mfma", g),
        # statistics: one pass over the float32 input
        "bn_stats": ("hbm", P * C * 4),
        # apply: read the input, the residual half the time, write the output
        "bn_apply": ("hbm", P * C * 10),
        # backward: two passes over dy and the input (+ the ReLU mask), write da
        "bn_bwd": ("hbm", P * C * (2 * (4 + 4 + 1) + eb)),
        "mse": ("hbm", P * C * (3 * eb + 4)),
        "rmsprop": ("hbm", cfg.param_count() * (20 + (2 if eb == 2 else 0))),
    }


def role_passes(cfg, m, name, conv):
    """Micro-batch passes of one layer (block) a role makes per step, or None."""
    L = cfg.blocks if conv else cfg.layers
    if name == "mse":
        return m
    if name == "rmsprop":
        return 1
    if conv:
        return {"conv_fwd": 4, "conv_fwd_implicit": 4, "conv_dgrad": 2, "conv_dgrad_implicit": 2,
                "conv_wgrad": 2, "conv_wgrad_implicit": 2, "bn_stats": 4, "bn_apply": 4,
                "bn_bwd": 2}.get(name, 0) * L * m or None
    if name in FWD_ROLES:
        return 2 * L * m
    if name in BWD_ROLES:
        return L * m
    return None


def rank_roles(names, step_work):
    """`names` in roofline order; the first is the dominant kernel.  The rank is
    the role's algorithmic work per step, among equals the role order
    (ffn1_fwd and ffn2_fwd carry the same flops).  Kernel time is no stable
    rank: the step's three streams share the chip, so a launch of 64 tiles on
    the caller's stream stretches with whatever runs beside it, and the order
    of the top roles by time changed from run to run."""
    from micro_pipelined_re_amd import gpipe
    return sorted(names, key=lambda k: (-step_work(k), gpipe.ROLES.index(k)))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ CPU baseline (oracle)
def cpu_baseline(cfg, n, m):
    """The oracle on one micro-batch of one layer (fwd + remat + bwd, float32) plus that
    layer's RMSProp, scaled to the full step: M micro-batches x L layers + L updates."""
    from micro_pipelined_re_amd import inputs
    from oracle import transformer_cell as tc
    b = n // m
    p = [inputs.layer_params(cfg.seed, 0, cfg.d_model, cfg.d_ff, bf16=True)]
    x, t = inputs.cell_data(cfg, batch=b)
    # repeat the sample for about 10 s of CPU work; average the repetitions
    reps, t_step, t_upd, t_start = 0, 0.0, 0.0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t_start < 10.0:
        t0 = time.perf_counter()
        out = tc.cell_step(p, x, t, 1, cfg.heads, cfg.causal, remat=True, dtype=np.float32,
                           denom=n * cfg.seq * cfg.d_model)
        t1 = time.perf_counter()
        ms = {k: np.zeros(v.shape, np.float32) for k, v in p[0].items()}
        for k in p[0]:
            tc.rmsprop(p[0][k], out["grads"][0][k], ms[k], np.float32(cfg.lr),
                       np.float32(cfg.decay), np.float32(cfg.eps))
        t2 = time.perf_counter()
        t_step += t1 - t0
        t_upd += t2 - t1
        reps += 1
    t1, t0, t2 = t_step / reps, 0.0, t_step / reps + t_upd / reps
    step_s = m * cfg.layers * (t1 - t0) + cfg.layers * (t2 - t1)
    threads = None
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or None
    except Exception:
        pass
    return {"value": n * cfg.seq / step_s, "unit": "tokens/s",
            "cores": threads or os.cpu_count(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"one micro-batch ({b} sequences, {b * cfg.seq} tokens) through one layer "
                       f"(forward, re-materialized forward, backward; numpy float32) plus that "
                       f"layer's RMSProp, {reps} repetitions of {t2:.2f} s, scaled by {m} "
                       f"micro-batches x {cfg.layers} layers"),
            "sample_seconds": round(t2 * reps, 2)}


def conv_cpu_baseline(cfg, n, m):
    """The oracle on one micro-batch through one block (fwd + remat + bwd, float32) plus
    that block's RMSProp, scaled to the full step: M micro-batches x blocks + updates."""
    from micro_pipelined_re_amd import inputs
    from oracle import conv_cell as cc
    from oracle import transformer_cell as tc
    b = n // m
    p = [inputs.conv_block_params(cfg.seed, 0, cfg.channels, bf16=cfg.precision == "bf16")]
    x, t = inputs.conv_cell_data(cfg, batch=b)
    reps, t_step, t_upd, t_start = 0, 0.0, 0.0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t_start < 10.0:
        t0 = time.perf_counter()
        out = cc.cell_step(p, x, t, 1, eps=cfg.bn_eps, remat=True, dtype=np.float32)
        t1 = time.perf_counter()
        for k in p[0]:
            w = p[0][k]
            tc.rmsprop(w, out["grads"][0][k], np.zeros_like(w), np.float32(cfg.lr),
                       np.float32(cfg.decay), np.float32(cfg.eps))
        t2 = time.perf_counter()
        t_step += t1 - t0
        t_upd += t2 - t1
        reps += 1
    t1, t0, t2 = t_step / reps, 0.0, t_step / reps + t_upd / reps
    step_s = m * cfg.blocks * (t1 - t0) + cfg.blocks * (t2 - t1)
    threads = None
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or None
    except Exception:
        pass
    return {"value": n / step_s, "unit": "images/s",
            "cores": threads or os.cpu_count(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"one micro-batch ({b} images of {cfg.height}x{cfg.width}x{cfg.channels}) "
                       f"through one block (forward, re-materialized forward, backward; numpy "
                       f"float32) plus that block's RMSProp, {reps} repetitions of {t2:.2f} s, "
                       f"scaled by {m} micro-batches x {cfg.blocks} blocks"),
            "sample_seconds": round(t2 * reps, 2)}


def setup_transformer(cfg, n, m, remat, dev):
    import torch
    from micro_pipelined_re_amd import gpipe, inputs
    cell = gpipe.Cell.from_config(cfg, dev)
    flat = np.empty(cell.n_params, np.float32)
    for l, offs in enumerate(cell.offsets()):
        lp = inputs.layer_params(cfg.seed, l, cfg.d_model, cfg.d_ff, bf16=True)
        for name, (o, c) in zip(gpipe.TENSORS, offs):
            flat[o:o + c] = lp[name].ravel()
    cell.load_params(flat)
    del flat
    x_h, t_h = inputs.cell_data(cfg)
    x, t = cell.to_device(x_h), cell.to_device(t_h)
    del x_h, t_h
    return cell, x, t


def setup_conv(cfg, n, m, remat, dev):
    from micro_pipelined_re_amd import gpipe, inputs
    cell = gpipe.ConvCell.from_config(cfg, dev)
    flat = np.empty(cell.n_params, np.float32)
    bf = cfg.precision == "bf16"
    for l, offs in enumerate(cell.offsets()):
        lp = inputs.conv_block_params(cfg.seed, l, cfg.channels, bf16=bf)
        for name, (o, c) in zip(gpipe.CONV_TENSORS, offs):
            flat[o:o + c] = lp[name].ravel()
    cell.load_params(flat)
    del flat
    x_h, t_h = inputs.conv_cell_data(cfg)
    x, t = cell.to_device(x_h), cell.to_device(t_h)
    del x_h, t_h
    return cell, x, t


# ------------------------------------------------------------------ memory scaling
def run_memory(args):
    """The 48-layer d_model-4096 cell: peak device bytes of one step at several M,
    against the planner's O(N + L/K * N/M) figure and a run without
    re-materialization at the largest N that fits.  Weights are drawn on the device
    (seeded torch generator; matrices N(0, 0.02^2), gamma 1, beta and biases 0)."""
    import torch
    from micro_pipelined_re_amd import configs, gpipe
    cfg = configs.MEMORY_4096
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    cell = gpipe.Cell.from_config(cfg, "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed)
    mats = {"w_qkv", "w_o", "w_1", "w_2"}
    with torch.no_grad():
        for l, offs in enumerate(cell.offsets()):
            for name, (o, c) in zip(gpipe.TENSORS, offs):
                v = cell.master[o:o + c]
                if name in mats:
                    v.normal_(0.0, 0.02, generator=gen)
                else:
                    v.fill_(1.0 if name.endswith("_g") else 0.0)
    gpipe.gpipe_cell_sync_lowp(cell.handle)
    torch.cuda.synchronize()
    state = torch.cuda.memory_allocated()
    total_mem = torch.cuda.get_device_properties(0).total_memory
    log(f"[bench] {cfg.name}: params {cell.n_params}, state {state / 1e9:.1f} GB, "
        f"device {total_mem / 1e9:.1f} GB, setup {time.perf_counter() - t0:.1f} s")
    eb = 2
    per_seq_io = cfg.seq * cfg.d_model * eb   # one sequence of x, y or dx

    def one(n, m, remat):
        x = torch.empty(n, cfg.seq, cfg.d_model, dtype=torch.bfloat16, device="cuda")
        t = torch.empty_like(x)
        x.normal_(0.0, 1.0, generator=gen)
        t.normal_(0.0, 1.0, generator=gen)
        y, dx = torch.empty_like(x), torch.empty_like(x)
        plan = gpipe.gpipe_cell_workspace_bytes(cell.handle, n, m, remat)   # raises if it does not fit
        ws = torch.empty(plan, dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gpipe.gpipe_cell_step(cell.handle, x, t, y, dx, n, m, remat, ws, plan, stream, cell.loss)
        gpipe.gpipe_apply_update(cell.handle, cfg.lr, cfg.decay, cfg.eps, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated()
        # one micro-batch's saved set: L layer slots of the plan
        o0 = gpipe.gpipe_cell_saved_offset(cell.handle, n, m, remat, 0, 1, 1)[0]
        o1 = gpipe.gpipe_cell_saved_offset(cell.handle, n, m, remat, 0, 2, 1)[0]
        set_bytes = (o1 - o0) * cfg.layers
        r = {"N": n, "M": m, "remat": remat, "ms_per_step": round(e0.elapsed_time(e1), 1),
             "tokens_per_s": round(n * cfg.seq / (e0.elapsed_time(e1) * 1e-3), 1),
             "activation_bytes_measured": peak - state,
             "workspace_plan": plan, "boundary_x_t_y_dx": 4 * n * per_seq_io,
             "saved_set_per_micro_batch": set_bytes, "peak_device_bytes": peak,
             "loss": float(cell.loss.item())}
        log(f"[bench] N={n} M={m} remat={remat}: {r['ms_per_step']} ms, activations "
            f"{r['activation_bytes_measured'] / 1e9:.2f} GB (plan {plan / 1e9:.2f} GB)")
        del x, t, y, dx, ws
        torch.cuda.empty_cache()
        return r

    def fit(xs, ys):
        """Least-squares line ys ~ a xs + b; returns slope, intercept, R^2."""
        xs, ys = np.asarray(xs, np.float64), np.asarray(ys, np.float64)
        a, b0 = np.polyfit(xs, ys, 1)
        pred = a * xs + b0
        ss = float(((ys - ys.mean()) ** 2).sum())
        r2 = 1.0 - float(((ys - pred) ** 2).sum()) / ss if ss > 0 else 1.0
        return {"slope_bytes": float(a), "intercept_bytes": float(b0), "r2": round(r2, 6)}

    # N sweep at fixed M = 8, M sweep at fixed N = 32 (re-materialization)
    by_n = [one(nn, 8, True) for nn in (8, 16, 32)]
    by_m = [one(32, mm, True) for mm in (4, 32)] + [by_n[-1]]
    by_m.sort(key=lambda r: r["M"])
    n = cfg.batch
    # M = 1: the planner's figure, refused by the library's fit check
    m1, m1_fits = gpipe.gpipe_cell_workspace_fit(cell.handle, n, 1, True)
    log(f"[bench] N={n} M=1: plan {m1 / 1e9:.1f} GB, fits={m1_fits}")
    # without re-materialization at the largest N (multiple of 8) that fits
    per_seq_keep = gpipe.gpipe_cell_workspace_fit(cell.handle, 16, 16, False)[0] / 16
    n_keep = int((0.97 * total_mem - state) // (per_seq_keep + 4 * per_seq_io)) // 8 * 8
    keep = None
    if n_keep >= 8:
        keep = [one(n_keep, n_keep // 2, False), one(n_keep, n_keep // 2, True)]
    act = lambda rs: [r["activation_bytes_measured"] for r in rs]
    out = {
        "metric": "peak activation bytes vs O(N + L/K*N/M), 48-layer d4096 cell",
        "value": by_m[-1]["activation_bytes_measured"], "unit": "bytes",
        "higher_is_better": False, "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.layers, "d_model": cfg.d_model,
                   "heads": cfg.heads, "d_ff": cfg.d_ff, "seq_len": cfg.seq,
                   "global_batch": n, "causal": cfg.causal},
        "parameter_state_bytes": state, "device_bytes": total_mem,
        "remat_runs_n_sweep_m8": by_n,
        "remat_runs_m_sweep_n32": by_m,
        # activations against N at fixed M (the boundary and the set grow with N),
        # and against L N / M at fixed N (one micro-batch's saved set)
        "fit_activation_vs_n_at_m8": fit([r["N"] for r in by_n], act(by_n)),
        "fit_activation_vs_l_n_over_m_at_n32": fit([cfg.layers * r["N"] / r["M"] for r in by_m],
                                                   act(by_m)),
        "m1_workspace_plan": m1, "m1_refused_oom": not m1_fits,
        "no_remat_vs_remat_at_largest_n": keep,
    }
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ counter summaries
def _kernel_class(name):
    """The step role of a GEMM dispatch (its last template argument) or the
    family of another kernel; None for kernels the summary leaves out."""
    import re
    from micro_pipelined_re_amd import gpipe
    m = re.search(r"gemm_(?:spec|dma|bf16)_kernel<.*, (\d+)>\(gp::GemmParams\)", name)
    if m:
        return gpipe.ROLES[int(m.group(1))]
    for key, cls in (("ln_fwd_kernel", "ln_fwd"), ("ln_bwd", "ln_bwd"), ("flash_fwd_kernel", "attn_fwd"),
                     ("flash_bwd_kernel", "attn_bwd"), ("mse_kernel", "mse"),
                     ("rmsprop_kernel", "rmsprop"), ("to_bf16_kernel", "to_bf16"),
                     ("sum_partials_kernel", "sum_partials"), ("splitk_reduce", "splitk_reduce")):
        if key in name:
            return cls
    return None


def _read_counters(d):
    """{dispatch: (class, grid, duration_ns, {counter: value})} of one rocprofv3
    --pmc run (csv output) in directory d."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
        for r in csv.DictReader(open(path)):
            cls = _kernel_class(r["Kernel_Name"])
            if cls is None:
                continue
            k = int(r["Dispatch_Id"])
            if k not in out:
                out[k] = (cls, int(r["Grid_Size"]),
                          int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {})
            out[k][3][r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def counter_summary(fetch_dir, write_dir, sq_dir=None):
    """Markdown tables of the counter passes over one step of the native
    driver: HBM bytes per dispatch (FETCH_SIZE and WRITE_SIZE, calibrated on
    the to_bf16 stream of the parameters), and for the GEMM roles the MFMA
    busy fraction and the clock implied by GRBM_GUI_ACTIVE.  Durations are
    those of the counter runs, whose dispatches run one at a time."""
    from micro_pipelined_re_amd import configs
    cfg = configs.CELL_2048
    nparam = cfg.param_count()
    fe, wr = _read_counters(fetch_dir), _read_counters(write_dir)
    cal = [v for v in fe.values() if v[0] == "to_bf16"], [v for v in wr.values() if v[0] == "to_bf16"]
    f_fetch = 4.0 * nparam / (cal[0][0][3]["FETCH_SIZE"] * 1024.0)
    f_write = 2.0 * nparam / (cal[1][0][3]["WRITE_SIZE"] * 1024.0)
    lines = [f"Calibration (to_bf16 over {nparam:,} parameters: {4 * nparam:,} B read, "
             f"{2 * nparam:,} B written): FETCH_SIZE x {f_fetch:.4f}, WRITE_SIZE x {f_write:.4f}.", ""]

    def groups(runs, key):
        g = {}
        for cls, grid, dur, c in runs.values():
            g.setdefault(key(cls, grid), []).append((dur, c))
        return g
    by = lambda cls, grid: (cls, grid)
    gf, gw = groups(fe, by), groups(wr, by)
    work = role_work(cfg, cfg.batch, cfg.micro)
    lines += ["| kernel (role) | grid | dispatches | mean us | fetch MB | write MB | GB/s |",
              "|---|---|---|---|---|---|---|"]
    for key in sorted(gf, key=lambda k: -sum(d for d, _ in gf[k])):
        f = gf[key]
        w = gw.get(key, [])
        us = sum(d for d, _ in f) / len(f) / 1e3
        fb = sum(c["FETCH_SIZE"] for _, c in f) / len(f) * 1024 * f_fetch
        wb = sum(c["WRITE_SIZE"] for _, c in w) / len(w) * 1024 * f_write if w else 0.0
        lines.append(f"| {key[0]} | {key[1]} | {len(f)} | {us:.2f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} "
                     f"| {(fb + wb) / us / 1e3:.0f} |")
    lines.append("")
    # per role over all its dispatches (the mix of one step), as bench.py reads them
    gfr, gwr = groups(fe, lambda cls, grid: cls), groups(wr, lambda cls, grid: cls)
    mach = [f"gemm_source_digest: {gemm_source_digest()}"]
    for role in sorted(gfr):
        if work.get(role, ("", 0))[0] != "mfma" or role.startswith("attn"):
            continue
        fb = sum(c["FETCH_SIZE"] for _, c in gfr[role]) / len(gfr[role]) * 1024 * f_fetch
        wb = sum(c["WRITE_SIZE"] for _, c in gwr[role]) / len(gwr[role]) * 1024 * f_write
        mach.append(f"traffic {role}: fetch_bytes={int(round(fb))} write_bytes={int(round(wb))}")
    if sq_dir:
        sq = groups(_read_counters(sq_dir), by)
        lines += ["| GEMM role | grid | dispatches | mean us | MFMA busy | flops (MOPS x 512) / algorithmic "
                  "| clock GHz (GRBM_GUI_ACTIVE per XCD / duration) |", "|---|---|---|---|---|---|---|"]
        for key in sorted(sq, key=lambda k: -sum(d for d, _ in sq[k])):
            if work.get(key[0], ("", 0))[0] != "mfma" or key[0].startswith("attn"):
                continue
            rows = sq[key]
            us = sum(d for d, _ in rows) / len(rows) / 1e3
            gui = sum(c["GRBM_GUI_ACTIVE"] for _, c in rows) / 8.0      # summed over 8 XCDs
            busy = sum(c["SQ_VALU_MFMA_BUSY_CYCLES"] for _, c in rows) / (gui * 1024)  # 1024 SIMDs
            fl = sum(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for _, c in rows) * 512 / len(rows)
            lines.append(f"| {key[0]} | {key[1]} | {len(rows)} | {us:.2f} | {busy:.3f} | "
                         f"{fl:.4g} | {gui / len(rows) / (us * 1e3):.2f} |")
        lines.append("")
    lines += ["Machine-readable lines read by bench.py (the figures hold only while the GEMM "
              "sources hash to the digest; comments excluded):", "", "```", *mach, "```"]
    return "\n".join(lines)


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--micro", type=int, default=None, help="override M")
    ap.add_argument("--no-remat", action="store_true", help="keep every micro-batch's activations")
    ap.add_argument("--workload", default="cell_d2048_L8_causal",
                    choices=("cell_d2048_L8_causal", "conv_c256_b8", "memory_4096"))
    ap.add_argument("--precision", default=None, choices=("bf16", "fp32"),
                    help="override the workload's precision")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="print the summary of rocprofv3 --pmc runs (csv) of the native driver: "
                         "FETCH_SIZE dir, WRITE_SIZE dir [, SQ/GRBM dir]")
    ap.add_argument("--profile-all", action="store_true",
                    help="time every kernel role inside the timed region")
    ap.add_argument("--time-every", type=int, default=5,
                    help="inside the timed region, time every k-th launch of the dominant "
                         "kernel (raised to the next k coprime with its launches per step, so "
                         "that the sample moves over every launch position of a step)")
    args = ap.parse_args()
    if args.counter_summary:
        print(counter_summary(*args.counter_summary[:3]))
        return 0
    if args.workload == "memory_4096" and args.gpus == 1:
        return run_memory(args)
    if args.gpus != 1:
        print(f"bench.py runs one cell on one GPU; --gpus {args.gpus} is not supported "
              f"(the library steps one pipeline cell per GPU; scheduling cells across GPUs "
              f"is outside it)", file=sys.stderr)
        sys.exit(2)

    import torch
    from micro_pipelined_re_amd import configs, gpipe, inputs

    conv = args.workload == "conv_c256_b8"
    cfg = configs.CONV_CELL if conv else configs.CELL_2048
    if args.precision:
        cfg = cfg.with_(precision=args.precision)
    n = cfg.batch
    m = args.micro or cfg.micro
    remat = not args.no_remat
    dev = "cuda"
    torch.cuda.set_device(0)
    if conv:
        log(f"[bench] {cfg.name}: blocks={cfg.blocks} C={cfg.channels} {cfg.height}x{cfg.width} "
            f"N={n} M={m} remat={remat} {cfg.precision}")
    else:
        log(f"[bench] {cfg.name}: L={cfg.layers} D={cfg.d_model} H={cfg.heads} F={cfg.d_ff} "
            f"S={cfg.seq} N={n} M={m} remat={remat}")
    t0 = time.perf_counter()
    cell, x, t = (setup_conv if conv else setup_transformer)(cfg, n, m, remat, dev)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    ws, ws_bytes = cell.workspace(n, m, remat)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t0:.1f} s; params {cell.n_params}; "
        f"workspace {ws_bytes / 1e9:.3f} GB")
    stream = torch.cuda.current_stream()

    def step():
        # the step and its update in one call: each layer's update starts as
        # soon as that layer's gradients are complete
        gpipe.gpipe_cell_step_update(cell.handle, x, t, y, dx, n, m, remat, ws, ws_bytes, stream,
                                     cell.loss, cfg.lr, cfg.decay, cfg.eps)

    # warmup; the last warmup step times every launch of every role (all streams)
    all_roles = (1 << len(gpipe.ROLES)) - 1
    for i in range(max(args.warmup, 1)):
        if i == max(args.warmup, 1) - 1:
            gpipe.gpipe_cell_profile(cell.handle, all_roles)
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i} done, loss {cell.loss.item():.6f}")
    work = (conv_role_work if conv else role_work)(cfg, n, m)
    prof = {}
    for r, name in enumerate(gpipe.ROLES):
        ms_tot, cnt = gpipe.gpipe_cell_profile_read(cell.handle, r)
        if cnt:
            prof[name] = (ms_tot, cnt)

    def step_work(name):
        """Algorithmic work of the role in one step, or None."""
        p_ = role_passes(cfg, m, name, conv)
        return work[name][1] * p_ if (p_ and name in work) else None

    def single_kernel(name):
        # a split-K GEMM role is two kernels: the split products and their ordered sum
        return gpipe.gpipe_cell_gemm_plan(cell.handle, n, m, gpipe.ROLES.index(name))[2] <= 1

    ranked = rank_roles([k for k in prof if step_work(k) and single_kernel(k)], step_work)
    dominant = ranked[0]
    dom_idx = gpipe.ROLES.index(dominant)
    log("[bench] roles by work per step; their kernel time (warmup step, all streams): " +
        ", ".join(f"{k} {prof[k][0]:.1f} ms" for k in ranked[:6]))

    # timed region: K steps; a regular sample of the dominant role's launches
    # (every k-th) is timed by events, which keeps the events' own cost (each
    # timed launch delays the next kernel of its stream) a fraction of timing
    # every launch
    every = 1 if args.profile_all else max(args.time_every, 1)
    while every > 1 and math.gcd(every, prof[dominant][1]) != 1:
        every += 1
    gpipe.gpipe_cell_profile_sampled(cell.handle, all_roles if args.profile_all else (1 << dom_idx),
                                     every)
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/step (wall {wall / args.steps * 1e3:.2f})")
    loss = cell.loss.item()
    peak_alloc = torch.cuda.max_memory_allocated()

    # per role: time and launches per step (from the timed region where timed
    # there, else from the warmup step), algorithmic rate over its kernel time
    src = {}
    for name in (gpipe.ROLES if args.profile_all else (dominant,)):
        ms_tot, cnt = gpipe.gpipe_cell_profile_read(cell.handle, gpipe.ROLES.index(name))
        if not cnt:
            continue
        if every == 1:
            src[name] = (ms_tot / args.steps, cnt // args.steps, "timed steps")
        else:
            # mean over the sampled launches times the launches of a step (the
            # warmup step timed them all)
            per_step = prof[name][1]
            src[name] = (ms_tot / cnt * per_step, per_step,
                         f"timed steps, every {every}th launch ({cnt} launches)")
    for name, (ms_tot, cnt) in prof.items():
        if name not in src:
            src[name] = (ms_tot, cnt, "warmup step")
    peak_mfma = PEAK_BF16_TFLOPS if cfg.precision == "bf16" else PEAK_FP32_TFLOPS
    kernels = {}
    for name, (ms_tot, cnt, when) in sorted(src.items(), key=lambda kv: -kv[1][0]):
        e = {"ms_per_step": round(ms_tot, 4), "launches_per_step": cnt,
             "avg_us": round(ms_tot / cnt * 1e3, 3), "from": when}
        _, _, sp_ = gpipe.gpipe_cell_gemm_plan(cell.handle, n, m, gpipe.ROLES.index(name))
        if sp_ > 1:
            e["split_k"] = sp_
        sw = step_work(name)
        if sw:
            kind = work[name][0]
            rate = sw / (ms_tot * 1e-3)
            if kind == "mfma":
                e.update(tflops=round(rate / 1e12, 1), frac_mfma_peak=round(rate / 1e12 / peak_mfma, 4))
            else:
                e.update(gbs=round(rate / 1e9, 1), frac_hbm_peak=round(rate / 1e9 / PEAK_HBM_GBS, 4))
        kernels[name] = e

    # dominant kernel roofline: its algorithmic work per step over its kernel
    # time per step (= the mean work per launch over the mean launch duration)
    kind = work[dominant][0]
    d_ms, d_cnt, _ = src[dominant]
    per = step_work(dominant) / d_cnt          # mean algorithmic work per launch
    avg_s = d_ms / d_cnt * 1e-3
    if kind == "mfma":
        roof = {"bound": "mfma", "achieved": round(per / avg_s / 1e12, 2), "peak": peak_mfma,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(per / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    tr = None if conv else measured_traffic(dominant)
    roof["traffic"] = (tr[0] + tr[1]) if tr else None
    if tr:
        roof["traffic_detail"] = {"unit": "bytes per launch", "fetch": tr[0], "write": tr[1],
                                  "source": os.path.relpath(TRAFFIC_FILE, ROOT)}
    roof["kernel"] = dominant
    tm_, tn_, sp_ = gpipe.gpipe_cell_gemm_plan(cell.handle, n, m, dom_idx)
    roof["kernel_tile"] = [tm_, tn_] if tm_ else None
    roof["avg_launch_us"] = round(avg_s * 1e6, 2)
    roof["launches_per_step"] = d_cnt
    roof["work_per_launch"] = per
    roof["kernel_ms_per_step"] = round(d_ms, 3)

    # the GEMM roles' algorithmic work over their summed kernel time, and the
    # step's whole algorithmic MFMA work over its wall time
    gemm = [k for k in src if work.get(k, ("", 0))[0] == "mfma" and step_work(k)]
    gemm_flops = sum(step_work(k) for k in gemm)
    gemm_ms = sum(src[k][0] for k in gemm)
    step_flops = gemm_flops if conv else step_mfma_flops(cfg, n, m)
    keep_bytes = gpipe.gpipe_cell_workspace_fit(cell.handle, n, m, False)[0]
    state_bytes = sum(v.numel() * v.element_size()
                      for v in (cell.master, cell.w_lowp, cell.grad, cell.ms) if v is not None)
    act_bytes = x.numel() * x.element_size()
    if conv:
        units, unit = n, "images/s"
        config = {"workload": cfg.name, "blocks": cfg.blocks, "channels": cfg.channels,
                  "height": cfg.height, "width": cfg.width, "global_batch": n,
                  "micro_batches": m, "remat": remat, "bn_momentum": cfg.bn_momentum,
                  "parallelism": "single-gpu cell"}
        metric = "train images/sec per conv cell step (fwd+remat+bwd), MFMA util; peak act bytes"
    else:
        units, unit = n * cfg.seq, "tokens/s"
        config = {"workload": cfg.name, "layers": cfg.layers, "d_model": cfg.d_model,
                  "heads": cfg.heads, "d_ff": cfg.d_ff, "seq_len": cfg.seq, "causal": cfg.causal,
                  "global_batch": n, "micro_batches": m, "remat": remat,
                  "parallelism": "single-gpu cell"}
        metric = METRIC
    out = {
        "metric": metric,
        "value": round(units / (ms_step * 1e-3), 1),
        "unit": unit,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.precision == "bf16" else "f32", "data": "synthetic",
        "config": config,
        "roofline": roof,
        "mfma_util_gemm": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / peak_mfma, 4)
        if gemm_ms else None,
        "mfma_util_gemm_note": "the GEMM roles' algorithmic flops over their summed kernel "
                               "time (kernels of different streams overlap)",
        "mfma_util_step": round(step_flops / (ms_step * 1e-3) / 1e12 / peak_mfma, 4),
        # the library allocates nothing: the step's device memory is what the
        # caller allocated from the plan; the measured peak above the parameter
        # state is the workspace plus the boundary tensors x, target, y, dx
        "peak_act_bytes": {"workspace_plan": ws_bytes, "boundary_x_t_y_dx": 4 * act_bytes,
                           "total_planned": ws_bytes + 4 * act_bytes,
                           "measured_peak_above_state": peak_alloc - state_bytes,
                           "no_remat_workspace_plan": keep_bytes},
        "loss": loss,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a CPU sample ...")
        out["cpu_baseline"] = (conv_cpu_baseline if conv else cpu_baseline)(cfg, n, m)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

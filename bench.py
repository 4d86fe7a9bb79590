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
"""
from __future__ import annotations

import argparse
import json
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic work per role
def role_work(cfg, n, m):
    """Per launch: ('mfma', flops) for the contractions, ('hbm', bytes) for the rest."""
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


# ------------------------------------------------------------------ CPU baseline (oracle)
def cpu_baseline(cfg, n, m):
    """The oracle on one micro-batch of one layer (fwd + remat + bwd, fp64) plus that
    layer's RMSProp, scaled to the full step: M micro-batches x L layers + L updates."""
    from micro_pipelined_re_amd import inputs
    from oracle import transformer_cell as tc
    b = n // m
    p = [inputs.layer_params(cfg.seed, 0, cfg.d_model, cfg.d_ff, bf16=True)]
    x, t = inputs.cell_data(cfg, batch=b)
    t0 = time.perf_counter()
    out = tc.cell_step(p, x, t, 1, cfg.heads, cfg.causal, remat=True)
    t1 = time.perf_counter()
    ms = {k: np.zeros(v.shape) for k, v in p[0].items()}
    for k in p[0]:
        tc.rmsprop(p[0][k].astype(np.float64), out["grads"][0][k], ms[k], cfg.lr, cfg.decay, cfg.eps)
    t2 = time.perf_counter()
    step_s = m * cfg.layers * (t1 - t0) + cfg.layers * (t2 - t1)
    threads = None
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) or None
    except Exception:
        pass
    return {"value": n * cfg.seq / step_s, "unit": "tokens/s",
            "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": (f"one micro-batch ({b} sequences, {b * cfg.seq} tokens) through one layer "
                       f"(forward, re-materialized forward, backward; numpy float64) plus that "
                       f"layer's RMSProp, timed {t2 - t0:.1f} s, scaled by {m} micro-batches x "
                       f"{cfg.layers} layers"),
            "sample_seconds": round(t2 - t0, 2)}


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--micro", type=int, default=None, help="override M")
    ap.add_argument("--no-remat", action="store_true", help="keep every micro-batch's activations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-all", action="store_true",
                    help="time every kernel role inside the timed region")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs one cell on one GPU; --gpus {args.gpus} is not supported "
              f"(the multi-GPU pipeline schedule is not part of this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    from micro_pipelined_re_amd import configs, gpipe, inputs

    cfg = configs.CELL_2048
    n = cfg.batch
    m = args.micro or cfg.micro
    remat = not args.no_remat
    dev = "cuda"
    torch.cuda.set_device(0)
    log(f"[bench] {cfg.name}: L={cfg.layers} D={cfg.d_model} H={cfg.heads} F={cfg.d_ff} "
        f"S={cfg.seq} N={n} M={m} remat={remat}")

    cell = gpipe.Cell.from_config(cfg, dev)
    t0 = time.perf_counter()
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
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    ws, ws_bytes = cell.workspace(n, m, remat)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t0:.1f} s; params {cell.n_params}; "
        f"workspace {ws_bytes / 1e9:.3f} GB")
    stream = torch.cuda.current_stream()

    def step():
        gpipe.gpipe_cell_step(cell.handle, x, t, y, dx, n, m, remat, ws, ws_bytes, stream, cell.loss)
        gpipe.gpipe_apply_update(cell.handle, cfg.lr, cfg.decay, cfg.eps, stream)

    # warmup; the last warmup step times every role to find the dominant kernel
    all_roles = (1 << len(gpipe.ROLES)) - 1
    for i in range(max(args.warmup, 1)):
        if i == max(args.warmup, 1) - 1:
            gpipe.gpipe_cell_profile(cell.handle, all_roles)
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i} done, loss {cell.loss.item():.6f}")
    work = role_work(cfg, n, m)
    prof = {}
    for r, name in enumerate(gpipe.ROLES):
        ms_tot, cnt = gpipe.gpipe_cell_profile_read(cell.handle, r)
        if cnt:
            prof[name] = (ms_tot, cnt)
    # the dominant kernel: the role with the most time whose launch is a single kernel
    # (a split-K GEMM role is two kernels: the split products and their ordered sum)
    def single_kernel(name):
        if name not in work or name in ("bias_grad", "norm_grad", "loss_reduce"):
            return False
        return gpipe.gpipe_cell_gemm_plan(cell.handle, n, m, gpipe.ROLES.index(name))[2] <= 1
    dominant = max((k for k in prof if single_kernel(k)), key=lambda k: prof[k][0])
    dom_idx = gpipe.ROLES.index(dominant)

    # timed region: K steps; the dominant role's launches are bracketed by events
    gpipe.gpipe_cell_profile(cell.handle, all_roles if args.profile_all else (1 << dom_idx))
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

    kernels = {}
    timed = gpipe.ROLES if args.profile_all else (dominant,)
    src = {}
    for name in timed:
        ms_tot, cnt = gpipe.gpipe_cell_profile_read(cell.handle, gpipe.ROLES.index(name))
        if cnt:
            src[name] = (ms_tot / args.steps, cnt // args.steps)
    for name, (ms_tot, cnt) in prof.items():
        if name not in src:
            src[name] = (ms_tot, cnt)
    for name, (ms_tot, cnt) in src.items():
        kind, per = work.get(name, (None, None))
        e = {"ms_per_step": round(ms_tot, 4), "launches_per_step": cnt,
             "avg_us": round(ms_tot / cnt * 1e3, 3)}
        if name in gpipe.ROLES:
            _, _, sp_ = gpipe.gpipe_cell_gemm_plan(cell.handle, n, m, gpipe.ROLES.index(name))
            if sp_ > 1:
                e["split_k"] = sp_
        if kind == "mfma":
            tf = per / (ms_tot / cnt * 1e-3) / 1e12
            e.update(tflops=round(tf, 1), frac_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        elif kind == "hbm":
            gb = per / (ms_tot / cnt * 1e-3) / 1e9
            e.update(gbs=round(gb, 1), frac_hbm_peak=round(gb / PEAK_HBM_GBS, 4))
        kernels[name] = e

    # dominant kernel roofline, from the events inside the timed region
    kind, per = work[dominant]
    d_ms, d_cnt = src[dominant]
    avg_s = d_ms / d_cnt * 1e-3
    if kind == "mfma":
        roof = {"bound": "mfma", "achieved": round(per / avg_s / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(per / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dominant
    tm_, tn_, sp_ = gpipe.gpipe_cell_gemm_plan(cell.handle, n, m, dom_idx)
    roof["kernel_tile"] = [tm_, tn_] if tm_ else None
    roof["avg_launch_us"] = round(avg_s * 1e6, 2)
    roof["work_per_launch"] = per

    gemm_flops = sum(work[k][1] * src[k][1] for k in src if work.get(k, ("", 0))[0] == "mfma")
    gemm_ms = sum(src[k][0] for k in src if work.get(k, ("", 0))[0] == "mfma")
    tokens = n * cfg.seq
    keep_bytes = gpipe.gpipe_cell_workspace_bytes(cell.handle, n, m, False)
    act_bytes = x.numel() * x.element_size()
    out = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.layers, "d_model": cfg.d_model,
                   "heads": cfg.heads, "d_ff": cfg.d_ff, "seq_len": cfg.seq, "causal": cfg.causal,
                   "global_batch": n, "micro_batches": m, "remat": remat,
                   "parallelism": "single-gpu cell"},
        "roofline": roof,
        "mfma_util_gemm": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if gemm_ms else None,
        "peak_act_bytes": {"workspace_plan": ws_bytes, "boundary_x_y_dx": 3 * act_bytes,
                           "total": ws_bytes + 3 * act_bytes,
                           "no_remat_workspace_plan": keep_bytes,
                           "torch_max_allocated": peak_alloc, "torch_base_allocated": base_alloc},
        "loss": loss,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a CPU sample ...")
        out["cpu_baseline"] = cpu_baseline(cfg, n, m)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

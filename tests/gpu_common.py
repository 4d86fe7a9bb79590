"""Shared pieces of the GPU parity tests: run the HIP cell and the oracle on the same inputs."""
import sys

import numpy as np

from micro_pipelined_re_amd import gpipe, inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def to_host(t):
    import torch
    return t.detach().float().cpu().numpy() if t.dtype != torch.float32 else t.detach().cpu().numpy()


def make_cell(cfg, params):
    cell = gpipe.Cell.from_config(cfg)
    flat = np.zeros(cell.n_params, np.float32)
    for l, offs in enumerate(cell.offsets()):
        for name, (o, c) in zip(gpipe.TENSORS, offs):
            flat[o:o + c] = np.asarray(params[l][name], np.float32).ravel()
    cell.load_params(flat)
    return cell


def run_gpu(cfg, params, x, t, N, M, remat=True, update=True, cell=None, want_dx=True):
    """One HIP step (+ update) of cfg on host inputs; returns host results."""
    import torch
    say(f"[gpu] {cfg.name} N={N} M={M} remat={remat} L={cfg.layers} D={cfg.d_model} "
        f"H={cfg.heads} F={cfg.d_ff} S={cfg.seq} causal={cfg.causal} {cfg.precision}")
    if cell is None:
        cell = make_cell(cfg, params)
    xd, td = cell.to_device(x), cell.to_device(t)
    y, dx = cell.step(xd, td, N, M, remat=remat, want_dx=want_dx)
    torch.cuda.synchronize()
    out = dict(cell=cell, y=to_host(y), loss=float(cell.loss.item()),
               dx=to_host(dx) if want_dx else None,
               grad=cell.unflatten(cell.grad.cpu().numpy().copy()))
    if update:
        cell.update(cfg.lr, cfg.decay, cfg.eps)
        torch.cuda.synchronize()
        out["w_new"] = cell.unflatten(cell.master.cpu().numpy().copy())
        out["ms_new"] = cell.unflatten(cell.ms.cpu().numpy().copy())
        if cell.bf16:
            out["w_lowp"] = cell.w_lowp.float().cpu().numpy().copy()
    return out


def concat(layers, names=gpipe.TENSORS):
    return np.concatenate([np.asarray(l[n], np.float64).ravel() for l in layers for n in names])


def compare_step(gpu, ref, tol, check_update=True, tol_update=None):
    """Per-tensor rel L2 of y, dx and every gradient; updated weights on the whole vector."""
    report = {"y": rel_l2(gpu["y"], ref["y"]),
              "loss": abs(gpu["loss"] - ref["loss"]) / abs(ref["loss"])}
    if gpu.get("dx") is not None:
        report["dx"] = rel_l2(gpu["dx"], ref["dx"])
    for l, (gg, rg) in enumerate(zip(gpu["grad"], ref["grads"])):
        for n in gpipe.TENSORS:
            report[f"g{l}.{n}"] = rel_l2(gg[n], rg[n])
    if check_update:
        report["w_new"] = rel_l2(concat(gpu["w_new"]), concat(ref["w_new"]))
        report["ms_new"] = rel_l2(concat(gpu["ms_new"]), concat(ref["ms_new"]))
    worst = sorted(report.items(), key=lambda kv: -kv[1])[:6]
    say("[cmp] worst:", ", ".join(f"{k}={v:.2e}" for k, v in worst))
    tu = tol if tol_update is None else tol_update
    bad = {k: v for k, v in report.items()
           if v > (tu if k in ("w_new", "ms_new") else tol) or not np.isfinite(v)}
    return report, bad

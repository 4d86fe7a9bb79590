"""Cells chained on one device equal one training step of the whole stack.

The review page's interface cuts a model of L layers into K cells of
contiguous layers, balanced by their cost estimates, and puts communication
only at the cell boundaries: in the forward pass cell k's output is cell k+1's
input, in the backward pass the gradient with respect to cell k+1's input is
cell k's output gradient ("GPipe algorithm in detail / minimal interface
design", "pipeline execution flow" phases 1-2).  Here the K cells run one
after another on one GPU through the C-ABI: gpipe_cell_forward for every cell
but the top one, gpipe_cell_step on the top cell (its loss), then
gpipe_cell_backward down the stack with dy = the dx of the cell above, and one
RMSProp update per cell.  The cut comes from gpipe_partition.  The oracle is
one step of the whole stack (all L layers in one cell), so y, the loss, dx
and every layer's gradient and updated weights are compared with it at the
stated bars (relative L2 <= 1e-4 fp32, <= 2e-2 bf16).
"""
import numpy as np
import pytest

from micro_pipelined_re_amd import configs, gpipe, inputs
from oracle import conv_cell as cc
from oracle import transformer_cell as tc
from oracle.transformer_cell import rmsprop
from tests.gpu_common import compare_step, concat, make_cell, rel_l2, say, to_host

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4
BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpipe.lib()
    yield


def run_chain(cfg, params, x, t, N, M, bounds, remat=True):
    """K Transformer cells (layers bounds[k] .. bounds[k+1]-1) chained through the C-ABI."""
    import torch
    K = len(bounds) - 1
    say(f"[gpu] chain {cfg.name} bounds={bounds} N={N} M={M} remat={remat} {cfg.precision}")
    cells = [make_cell(cfg.with_(layers=b1 - b0), params[b0:b1])
             for b0, b1 in zip(bounds[:-1], bounds[1:])]
    xs = [cells[0].to_device(x)]
    for c in cells[:-1]:
        xs.append(c.forward(xs[-1], N, M, remat=remat))
    y, d = cells[-1].step(xs[-1], cells[-1].to_device(t), N, M, remat=remat)
    for k in reversed(range(K - 1)):
        d = cells[k].backward(xs[k], d, N, M, remat=remat)
    torch.cuda.synchronize()
    out = dict(y=to_host(y), dx=to_host(d), loss=float(cells[-1].loss.item()),
               grad=[g for c in cells for g in c.unflatten(c.grad.cpu().numpy().copy())])
    for c in cells:
        c.update(cfg.lr, cfg.decay, cfg.eps)
    torch.cuda.synchronize()
    out["w_new"] = [w for c in cells for w in c.unflatten(c.master.cpu().numpy().copy())]
    out["ms_new"] = [m for c in cells for m in c.unflatten(c.ms.cpu().numpy().copy())]
    return out


def stack_check(cfg, total_layers, K, costs=None, remat=True, N=None, M=None):
    N = cfg.batch if N is None else N
    M = cfg.micro if M is None else M
    stack = cfg.with_(layers=total_layers)
    params = inputs.cell_params(stack)
    x, t = inputs.cell_data(stack, batch=N)
    costs = np.ones(total_layers) if costs is None else np.asarray(costs, np.float64)
    bounds, _ = gpipe.gpipe_partition(costs, K)
    gpu = run_chain(cfg, params, x, t, N, M, bounds, remat=remat)
    ref = tc.train_step(params, x, t, M, cfg.heads, cfg.causal, cfg.lr, cfg.decay, cfg.eps,
                        ln_eps=cfg.ln_eps)
    tol = FP32_TOL if cfg.precision == "fp32" else BF16_TOL
    report, bad = compare_step(gpu, ref, tol)
    assert not bad, bad
    return bounds


def test_two_cells_fp32_equal_the_five_layer_stack():
    # uniform costs over 5 layers, K = 2: the lexicographically first optimum 2 + 3
    bounds = stack_check(configs.TINY, 5, 2)
    assert bounds == [0, 2, 5]


def test_two_cells_fp32_stored_activations():
    """Without re-materialization each cell's backward reads the saved sets its
    forward call left in the cell's workspace."""
    stack_check(configs.TINY, 5, 2, remat=False)


def test_four_one_layer_cells_fp32_causal():
    bounds = stack_check(configs.TINY.with_(causal=True), 4, 4)
    assert bounds == [0, 1, 2, 3, 4]


def test_cost_balanced_cells_bf16_fused_attention():
    """bf16 cells with the fused attention (head dim 128), cut by per-layer costs
    into three cells of unequal length; each cell runs the grouped forward and
    the pipelined re-materialization on its own streams."""
    cfg = configs.SMALL.with_(name="chain_bf16", d_model=256, heads=2, d_ff=512, seq=100,
                              batch=6, micro=3, causal=True)
    # cell sums (2, 2, 4), (2, 4, 2) and (4, 2, 2) tie; the lexicographically
    # smallest bounds win
    bounds = stack_check(cfg, 6, 3, costs=[1, 1, 2, 2, 1, 1])
    assert bounds == [0, 2, 3, 6]


# ---------------------------------------------------------------- conv cells
def test_conv_cells_fp32_equal_the_stack():
    """Two conv cells (1 and 2 residual blocks, micro-batch BatchNorm) chained:
    y, loss, dx, every gradient and each cell's moving averages equal one step
    of the three-block stack."""
    import torch
    from tests.test_gpu_conv import make_conv_cell, oracle_conv_step
    cfg = configs.CONV_TINY
    stack = cfg.with_(blocks=3)
    params = inputs.conv_cell_params(stack)
    x, t = inputs.conv_cell_data(stack)
    N, M = cfg.batch, cfg.micro
    bounds, _ = gpipe.gpipe_partition(np.ones(3), 2)
    assert bounds == [0, 1, 3]
    say(f"[gpu] conv chain bounds={bounds} N={N} M={M}")
    cells = [make_conv_cell(cfg.with_(blocks=b1 - b0), params[b0:b1])
             for b0, b1 in zip(bounds[:-1], bounds[1:])]
    x0 = cells[0].to_device(x)
    x1 = cells[0].forward(x0, N, M)
    y, dx1 = cells[1].step(x1, cells[1].to_device(t), N, M)
    dx0 = cells[0].backward(x0, dx1, N, M)
    for c in cells:
        c.update(cfg.lr, cfg.decay, cfg.eps)
    torch.cuda.synchronize()
    ref = oracle_conv_step(stack, params, x, t, M)
    report = {"y": rel_l2(to_host(y), ref["y"]), "dx": rel_l2(to_host(dx0), ref["dx"]),
              "loss": abs(cells[1].loss.item() - ref["loss"]) / ref["loss"],
              "running": rel_l2(np.concatenate([c.running.cpu().numpy() for c in cells]),
                                ref["running"])}
    grads = [g for c in cells for g in c.unflatten(c.grad.cpu().numpy())]
    for l, (gg, rg) in enumerate(zip(grads, ref["grads"])):
        for n in gpipe.CONV_TENSORS:
            report[f"g{l}.{n}"] = rel_l2(gg[n], rg[n])
    w_new = [w for c in cells for w in c.unflatten(c.master.cpu().numpy())]
    report["w_new"] = rel_l2(np.concatenate([np.ravel(w[n]) for w in w_new for n in gpipe.CONV_TENSORS]),
                             np.concatenate([np.ravel(w[n]) for w in ref["w_new"]
                                             for n in gpipe.CONV_TENSORS]))
    say("[cmp] worst:", sorted(report.items(), key=lambda kv: -kv[1])[:4])
    bad = {k: v for k, v in report.items() if not v <= FP32_TOL}
    assert not bad, bad

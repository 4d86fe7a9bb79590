"""Checkpoint and resume: the caller owns the whole training state.

A cell's state between steps is the bound buffers -- fp32 master weights,
the bf16 copy, the RMSProp mean squares and, for conv cells, the BatchNorm
moving averages; the gradient is rewritten by every step.  Saving them after
a step + update (torch.save / torch.load of the tensors, through a file),
restoring them into a freshly created cell and taking the next step must
give bit for bit what two consecutive steps of one cell give: y, dx, the
loss, every gradient and the updated state.
"""
import os
import tempfile

import numpy as np
import pytest

from micro_pipelined_re_amd import configs, gpipe, inputs
from tests.gpu_common import make_cell, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpipe.lib()
    yield


def _state(cell):
    s = {"master": cell.master, "ms": cell.ms}
    if cell.w_lowp is not None:
        s["w_lowp"] = cell.w_lowp
    if hasattr(cell, "running"):
        s["running"] = cell.running
    return s


def _step(cell, cfg, x, t):
    import torch
    xd, td = cell.to_device(x), cell.to_device(t)
    y, dx = cell.step(xd, td, cfg.batch, cfg.micro)
    cell.update(cfg.lr, cfg.decay, cfg.eps)
    torch.cuda.synchronize()
    out = dict(y=to_host(y), dx=to_host(dx), loss=float(cell.loss.item()),
               grad=cell.grad.cpu().numpy().copy())
    out.update({k: v.detach().float().cpu().numpy().copy() for k, v in _state(cell).items()})
    return out


def _resume_equals_consecutive(make, cfg, x, t):
    import torch
    a = make()
    _step(a, cfg, x, t)
    two = _step(a, cfg, x, t)
    b = make()
    _step(b, cfg, x, t)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "cell_state.pt")
        torch.save({k: v.cpu() for k, v in _state(b).items()}, path)
        del b
        torch.cuda.empty_cache()
        c = make()
        saved = torch.load(path, weights_only=True)
    for k, v in _state(c).items():
        v.copy_(saved[k].to(v.device))
    resumed = _step(c, cfg, x, t)
    for k in two:
        if k == "loss":
            assert resumed[k] == two[k]
        else:
            assert np.array_equal(resumed[k], two[k]), k
    say(f"[ckpt] {cfg.name}: resumed step bitwise equal to the second of two steps")


@pytest.mark.parametrize("cfg", [configs.TINY,
                                 configs.SMALL.with_(name="small_2l_ckpt", layers=2, batch=8,
                                                     micro=4, causal=True)],
                         ids=["fp32", "bf16"])
def test_transformer_cell_resume(cfg):
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    _resume_equals_consecutive(lambda: make_cell(cfg, params), cfg, x, t)


def test_conv_cell_resume():
    from tests.test_gpu_conv import make_conv_cell
    cfg = configs.CONV_SMALL
    params = inputs.conv_cell_params(cfg)
    x, t = inputs.conv_cell_data(cfg)
    _resume_equals_consecutive(lambda: make_conv_cell(cfg, params), cfg, x, t)

"""The bf16 storage-policy model of the conv cell, on the CPU.

Pins the model to the oracle (without rounding it is the oracle's step up to
the float32 loss gradient) and records the conditioning it measures: with
bf16 storage the gradients move by a few percent while the forward output
moves by about bf16's unit roundoff.
"""
import numpy as np

from micro_pipelined_re_amd import configs, inputs
from oracle import conv_cell as cc
from tests.conv_bf16_model import model_step


def rel(a, b):
    return float(np.linalg.norm(np.ravel(a) - np.ravel(b)) / np.linalg.norm(np.ravel(b)))


def _grads_rel(g, r):
    return max(rel(g[l][k], r[l][k]) for l in range(len(r)) for k in r[l])


def test_model_without_rounding_is_the_oracle_step():
    cfg = configs.CONV_TINY
    params = inputs.conv_cell_params(cfg)
    x, t = inputs.conv_cell_data(cfg)
    ref = cc.cell_step(params, x, t, cfg.micro)
    mod = model_step(params, x, t, cfg.micro, rounding=False)
    assert rel(mod["y"], ref["y"]) == 0.0
    assert abs(mod["loss"] - ref["loss"]) <= 1e-15 * ref["loss"]
    # only the float32 cast of the loss gradient differs
    assert rel(mod["dx"], ref["dx"]) < 1e-6
    assert _grads_rel(mod["grads"], ref["grads"]) < 1e-6


def test_model_rounding_conditioning():
    cfg = configs.CONV_SMALL
    params = inputs.conv_cell_params(cfg)
    x, t = inputs.conv_cell_data(cfg)
    ref = cc.cell_step(params, x, t, cfg.micro)
    mod = model_step(params, x, t, cfg.micro)
    assert rel(mod["y"], ref["y"]) < 5e-3          # forward: about the unit roundoff
    assert 2e-2 < rel(mod["dx"], ref["dx"]) < 6e-2  # backward: amplified
    assert _grads_rel(mod["grads"], ref["grads"]) < 6e-2

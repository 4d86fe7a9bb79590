"""Why the bf16 conv cell keeps its forward exact and rounds only its backward (CPU).

On the small bf16 conv workload (2 blocks, 64 channels, 16 x 16, N 16, M 4)
the oracle's step is replayed with bf16 rounding at chosen storage points
(tests/conv_bf16_model.py): rounding any single forward activation moves dx
or a gradient by more than half the 2e-2 bar -- all of them together by more
than the bar -- while rounding every backward operand together stays an
order of magnitude below it.  The bf16 path therefore stores the forward in
float32 / split bf16 pairs and the backward's operands in bf16.
"""
import numpy as np
import pytest

from micro_pipelined_re_amd import configs, inputs
from oracle import conv_cell as cc
from tests.conv_bf16_model import BACKWARD_POINTS, FORWARD_POINTS, model_step


def rel(a, b):
    return float(np.linalg.norm(np.ravel(a) - np.ravel(b)) / np.linalg.norm(np.ravel(b)))


def worst(out, ref):
    errs = [rel(out["dx"], ref["dx"])]
    errs += [rel(g[k], r[k]) for g, r in zip(out["grads"], ref["grads"]) for k in r]
    return max(errs)


@pytest.fixture(scope="module")
def small():
    cfg = configs.CONV_SMALL
    params = inputs.conv_cell_params(cfg)
    x, t = inputs.conv_cell_data(cfg)
    return cfg, params, x, t, cc.cell_step(params, x, t, cfg.micro)


def test_model_without_rounding_is_the_oracle_step(small):
    cfg, params, x, t, ref = small
    mod = model_step(params, x, t, cfg.micro, ())
    assert rel(mod["y"], ref["y"]) < 1e-15 and rel(mod["dx"], ref["dx"]) < 1e-12
    assert worst(mod, ref) < 1e-12


@pytest.mark.parametrize("point", FORWARD_POINTS)
def test_rounding_one_forward_activation_costs_a_large_share_of_the_bar(small, point):
    cfg, params, x, t, ref = small
    assert worst(model_step(params, x, t, cfg.micro, (point,)), ref) > 1e-2


def test_rounding_the_whole_forward_breaks_the_bar(small):
    cfg, params, x, t, ref = small
    assert worst(model_step(params, x, t, cfg.micro, FORWARD_POINTS + BACKWARD_POINTS), ref) > 2e-2


def test_rounding_every_backward_operand_stays_well_below_the_bar(small):
    cfg, params, x, t, ref = small
    e = worst(model_step(params, x, t, cfg.micro, BACKWARD_POINTS), ref)
    assert e < 5e-3, e

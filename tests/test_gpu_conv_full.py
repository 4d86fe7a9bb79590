"""The conv cell at its full shape: 8 blocks of 256 channels on 32 x 32 images.

* One micro-batch (N = 16, M = 1) runs every kernel at exactly the launch
  shapes of the full workload's micro-batches (16384 pixels, K = 2304, 4608
  for the split forward operands); the oracle checks all of it: bf16 at the
  flat 2e-2; fp32 with its conditioning floor for dx, the gradients and the
  update (at this shape the oracle evaluated in float32 itself deviates from
  float64 by about 2e-3, from the cancellations in the BatchNorm backward).
* The full step (N = 256, M = 16, the timed workload) is checked on what the
  oracle can compute piecewise: the outputs of sampled micro-batches (each
  normalised with its own statistics, so a micro-batch is the unit), block
  0's first moving averages (pooled over the whole mini-batch), and
  properties that hold at any size: the loss is the MSE of the cell's own
  output, the last BN shift's gradient is the pixel sum of the loss gradient,
  and re-materialization is bitwise equal to storing.
"""
import numpy as np
import pytest

from micro_pipelined_re_amd import configs, inputs
from oracle import conv_cell as cc
from tests.gpu_common import rel_l2, say
from tests.test_gpu_conv import (BF16_TOL, _concat, check_fp32_conditioning, compare_conv,
                                 oracle_conv_step, run_conv_gpu)

pytestmark = pytest.mark.gpu

FULL = configs.CONV_CELL


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_conv_full_shape_fp32_one_micro_batch():
    cfg = FULL.with_(name="conv_c256_fp32_mb", precision="fp32", batch=16, micro=1)
    params = inputs.conv_cell_params(cfg)
    x, t = inputs.conv_cell_data(cfg)
    gpu = run_conv_gpu(cfg, params, x, t, 16, 1)
    ref = oracle_conv_step(cfg, params, x, t, 1)
    check_fp32_conditioning(cfg, params, x, t, 1, gpu, ref)


def test_conv_full_shape_bf16_one_micro_batch():
    cfg = FULL.with_(name="conv_c256_bf16_mb", batch=16, micro=1)
    params = inputs.conv_cell_params(cfg)
    x, t = inputs.conv_cell_data(cfg)
    gpu = run_conv_gpu(cfg, params, x, t, 16, 1)
    ref = oracle_conv_step(cfg, params, x, t, 1)
    _, bad = compare_conv(gpu, ref, BF16_TOL)
    assert not bad, bad


def test_conv_full_workload_sampled():
    import torch
    cfg = FULL
    N, M = cfg.batch, cfg.micro
    b = N // M
    params = inputs.conv_cell_params(cfg)
    x, t = inputs.conv_cell_data(cfg)
    gpu = run_conv_gpu(cfg, params, x, t, N, M, update=False)
    y = gpu["y"].astype(np.float64)
    # sampled micro-batches against the oracle's forward
    for m in (0, M - 1):
        sl = slice(m * b, (m + 1) * b)
        y_ref, _ = cc.cell_forward(params, np.asarray(x[sl], np.float64), cfg.bn_eps)
        e = rel_l2(y[sl], y_ref)
        say(f"[cmp] y of micro-batch {m}: {e:.2e}")
        assert e <= BF16_TOL
    # block 0, BN1 moving averages: pooled moments of conv1(x) over the mini-batch
    a = np.concatenate([cc.conv3x3(np.asarray(x[i:i + b], np.float64), params[0]["w1"])
                        .reshape(-1, cfg.channels) for i in range(0, N, b)])
    n = a.shape[0]
    mean = a.mean(axis=0)
    var = a.var(axis=0) * n / (n - 1)
    m_ref = (1 - cfg.bn_momentum) * mean
    v_ref = cfg.bn_momentum + (1 - cfg.bn_momentum) * var
    em, ev = rel_l2(gpu["running"][0, 0, 0], m_ref), rel_l2(gpu["running"][0, 0, 1], v_ref)
    say(f"[cmp] block 0 BN1 running mean {em:.2e} var {ev:.2e}")
    assert em <= BF16_TOL and ev <= BF16_TOL
    # properties at any size
    denom = float(x.size)
    r = y - np.asarray(t, np.float64)
    loss = float((r * r).sum() / denom)
    assert abs(gpu["loss"] - loss) <= 1e-5 * loss
    g_beta = (2.0 * r / denom).reshape(-1, cfg.channels).sum(axis=0)
    e = rel_l2(gpu["grad"][-1]["bn2_b"], g_beta)
    say(f"[cmp] last bn2_b gradient vs pixel sum of dy: {e:.2e}")
    assert e <= 1e-4
    # re-materialization is bitwise equal to storing every micro-batch's activations
    cell = gpu["cell"]
    cell.running[:, :, 0, :] = 0.0
    cell.running[:, :, 1, :] = 1.0
    stored = run_conv_gpu(cfg, params, x, t, N, M, remat=False, update=False, cell=cell)
    assert np.array_equal(stored["y"], gpu["y"])
    assert np.array_equal(stored["dx"], gpu["dx"])
    assert np.array_equal(stored["running"], gpu["running"])
    assert np.array_equal(_concat(stored["grad"]), _concat(gpu["grad"]))
    del gpu, stored, cell
    torch.cuda.empty_cache()

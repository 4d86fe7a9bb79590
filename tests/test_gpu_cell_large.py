"""Oracle parity of the wide cells at their real shapes.

  * The 2048-wide causal cell's layers (D 2048, H 16, F 8192, S 512) at the
    full mini-batch N = 64 in M = 32 micro-batches, the launch configuration
    the benchmark times (two layers instead of eight, for the oracle's time):
    the grouped forward phase, the pipelined re-materialization and the
    32-micro-batch float32 accumulation, with every gradient and the update
    compared with the oracle.
  * The 48-layer memory-scaling cell's layers (D 4096, H 32, F 16384,
    S 1024, not causal) at two layers, N = 2, M = 2: LayerNorm rows of 4096,
    F = 16384 products, the fused attention at S = 1024.

The oracle runs in float32 (the float64 run of these shapes takes minutes);
the bar is the bf16 one, relative L2 <= 2e-2 per tensor (updated weights and
RMSProp state on the whole vector).
"""
import numpy as np
import pytest

from micro_pipelined_re_amd import configs, gpipe, inputs
from oracle import transformer_cell as tc
from tests.gpu_common import compare_step, run_gpu, say

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpipe.lib()
    yield


def _check(cfg):
    import time
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    gpu = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro)
    t0 = time.time()
    # stored activations: the same arithmetic as re-materialization, a quarter
    # less oracle time
    ref = tc.train_step(params, x, t, cfg.micro, cfg.heads, cfg.causal, cfg.lr, cfg.decay,
                        cfg.eps, ln_eps=cfg.ln_eps, remat=False, dtype=np.float32)
    say(f"[oracle] {cfg.name}: {time.time() - t0:.1f} s")
    report, bad = compare_step(gpu, ref, BF16_TOL)
    assert not bad, bad


@pytest.mark.timeout(400)
def test_cell_2048_two_layers_full_batch_bf16():
    cfg = configs.CELL_2048.with_(name="cell2048_2l_full", layers=2)
    assert (cfg.batch, cfg.micro) == (64, 32)
    _check(cfg)


@pytest.mark.timeout(300)
def test_cell_4096_layer_shapes_bf16():
    cfg = configs.MEMORY_4096.with_(name="cell4096_2l_n2", layers=2, batch=2, micro=2)
    _check(cfg)

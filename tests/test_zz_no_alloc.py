"""The allocation-free step (gpipe_cell_step_noalloc) against gpipe_cell_step.

Two calls in a row on the same cell, the second with a smaller input, for an
fp32 cell (the two-layer 64-wide cell) and a bf16 cell with the fused
attention: y, dx, the loss and every gradient equal those of the existing
entry point bit for bit (the same kernels and plans; the step is
deterministic), and both are within the fp32 / bf16 bars of the oracle.  A
plan larger than the library's scratch is refused with nothing enqueued.
"""
import numpy as np
import pytest

from micro_pipelined_re_amd import configs, gpipe, inputs
from oracle import transformer_cell as tc
from tests.gpu_common import make_cell, rel_l2, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpipe.lib()
    yield


def _outputs(cell, y, dx):
    import torch
    torch.cuda.synchronize()
    return dict(y=to_host(y), dx=to_host(dx), loss=float(cell.loss.item()),
                grad=cell.grad.cpu().numpy().copy())


def _both(cell, x, t, N, M):
    """(existing entry point's outputs, allocation-free entry point's outputs)."""
    import torch
    xd, td = cell.to_device(x), cell.to_device(t)
    y, dx = cell.step(xd, td, N, M)
    ref = _outputs(cell, y, dx)
    y2, dx2 = torch.empty_like(xd), torch.empty_like(xd)
    cell.loss.zero_()
    cell.grad.zero_()
    gpipe.gpipe_cell_step_noalloc(cell.handle, xd, td, y2, dx2, N, M, True, None, cell.loss)
    return ref, _outputs(cell, y2, dx2)


@pytest.mark.parametrize("cfg,sizes", [
    (configs.TINY, [(8, 4), (4, 2)]),
    (configs.SMALL.with_(name="small_2l", layers=2, batch=8, micro=4), [(8, 4), (4, 2)]),
])
def test_noalloc_step_equals_the_step(cfg, sizes):
    params = inputs.cell_params(cfg)
    cell = make_cell(cfg, params)
    tol = 1e-4 if cfg.precision == "fp32" else 2e-2
    for N, M in sizes:
        assert gpipe.gpipe_cell_workspace_bytes(cell.handle, N, M, True) <= gpipe.GPIPE_SCRATCH_BYTES
        x, t = inputs.cell_data(cfg, batch=N)
        say(f"[gpu] noalloc {cfg.name} N={N} M={M}")
        a, b = _both(cell, x, t, N, M)
        assert np.array_equal(a["y"], b["y"])
        assert np.array_equal(a["dx"], b["dx"])
        assert a["loss"] == b["loss"]
        assert np.array_equal(a["grad"], b["grad"])
        ref = tc.cell_step(params, x, t, M, cfg.heads, cfg.causal)
        g = cell.unflatten(b["grad"])
        errs = {"y": rel_l2(b["y"], ref["y"]), "dx": rel_l2(b["dx"], ref["dx"]),
                "loss": abs(b["loss"] - ref["loss"]) / ref["loss"]}
        for l in range(cfg.layers):
            for n in gpipe.TENSORS:
                errs[f"g{l}.{n}"] = rel_l2(g[l][n], ref["grads"][l][n])
        worst = max(errs.items(), key=lambda kv: kv[1])
        say(f"[cmp] worst vs oracle {worst[0]}={worst[1]:.2e}")
        assert worst[1] <= tol, worst


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    import torch
    cfg = configs.SMALL   # 6 layers, N=64, M=8: ~150 MiB of workspace
    cell = gpipe.Cell.from_config(cfg)
    N, M = cfg.batch, cfg.micro
    assert gpipe.gpipe_cell_workspace_bytes(cell.handle, N, M, True) > gpipe.GPIPE_SCRATCH_BYTES
    x = torch.zeros(N, cfg.seq, cfg.d_model, dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 7.0)
    torch.cuda.synchronize()
    with pytest.raises(gpipe.GpipeError) as e:
        gpipe.gpipe_cell_step_noalloc(cell.handle, x, x, y, None, N, M, True, None, cell.loss)
    assert e.value.code == 2
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())

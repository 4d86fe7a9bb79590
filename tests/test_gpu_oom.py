"""The workspace query refuses a plan the device cannot hold (GPIPE_ERR_OOM).

The 48-layer d_model-4096 cell at N = 32: in one micro-batch its saved
activations alone are ~211 GB, and its parameter state (bf16 copy, fp32
master, gradient and RMSProp state, 14 B/param) ~135 GB, together more than
one MI355X's 288 GiB.  The page's activation bound O(N + L/K * N/M)
("preliminaries 5") is what brings it down: at M = 4 or 32 the plan fits.
The query reports the plan's bytes either way and allocates or enqueues
nothing.
"""
import pytest

from micro_pipelined_re_amd import configs, gpipe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gpipe.lib()
    yield


def test_unbound_cell_counts_its_parameter_state():
    import torch
    cfg = configs.MEMORY_4096
    h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq, False,
                                gpipe.GPIPE_BF16)
    try:
        free0, total = torch.cuda.mem_get_info()
        plan1, fits1 = gpipe.gpipe_cell_workspace_fit(h, 32, 1, True)
        plan32, fits32 = gpipe.gpipe_cell_workspace_fit(h, 32, 32, True)
        state = gpipe.gpipe_cell_param_count(h) * 14
        print(f"[oom] free {free0 / 1e9:.1f} GB of {total / 1e9:.1f}; state {state / 1e9:.1f} GB; "
              f"plan M=1 {plan1 / 1e9:.1f} GB fits={fits1}; M=32 {plan32 / 1e9:.2f} GB fits={fits32}",
              flush=True)
        assert plan1 + state > free0 and not fits1
        assert plan32 + state < free0 and fits32
        with pytest.raises(gpipe.GpipeError) as e:
            gpipe.gpipe_cell_workspace_bytes(h, 32, 1, True)
        assert e.value.code == 2
        assert torch.cuda.mem_get_info()[0] == free0
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_bound_cell_refuses_one_micro_batch_and_takes_four():
    import torch
    cfg = configs.MEMORY_4096
    cell = gpipe.Cell.from_config(cfg)       # allocates and binds the ~135 GB of state
    try:
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        alloc0 = torch.cuda.memory_allocated()
        plan1, fits1 = gpipe.gpipe_cell_workspace_fit(cell.handle, 32, 1, True)
        print(f"[oom] bound: free {free0 / 1e9:.1f} GB, plan M=1 {plan1 / 1e9:.1f} GB "
              f"fits={fits1}", flush=True)
        assert plan1 > free0 and not fits1
        plan4, fits4 = gpipe.gpipe_cell_workspace_fit(cell.handle, 32, 4, True)
        assert plan4 < free0 and fits4
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        assert torch.cuda.memory_allocated() == alloc0
        # the helper refuses too, after releasing nothing it did not hold
        with pytest.raises(gpipe.GpipeError) as e:
            cell.workspace(32, 1, True)
        assert e.value.code == 2
    finally:
        del cell
        torch.cuda.empty_cache()

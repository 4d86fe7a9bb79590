"""Parity of the HIP cell step (through the C-ABI) with the oracle.

Tolerances: relative L2 <= 1e-4 in fp32 mode and <= 2e-2 in bf16 mode with
fp32 accumulation, per tensor for y, dx and every gradient, on the whole
parameter vector for the updated weights and RMSProp state.
"""
import numpy as np
import pytest

from micro_pipelined_re_amd import configs, gpipe, inputs
from oracle import transformer_cell as tc
from tests.gpu_common import compare_step, make_cell, rel_l2, run_gpu, say, to_host

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


def oracle_step(cfg, params, x, t, M, remat=True):
    return tc.train_step(params, x, t, M, cfg.heads, cfg.causal, cfg.lr, cfg.decay, cfg.eps,
                         ln_eps=cfg.ln_eps, remat=remat)


def check(cfg, N=None, M=None, remat=True, tol=None, seed_params=None):
    N = cfg.batch if N is None else N
    M = cfg.micro if M is None else M
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg, batch=N)
    gpu = run_gpu(cfg, params, x, t, N, M, remat=remat)
    ref = oracle_step(cfg, params, x, t, M)
    tol = tol or (FP32_TOL if cfg.precision == "fp32" else BF16_TOL)
    report, bad = compare_step(gpu, ref, tol)
    assert not bad, bad
    return gpu, ref


def test_tiny_fp32_saved_activations_match_oracle():
    """No-remat run: every saved intermediate of every micro-batch vs the oracle's."""
    import torch
    cfg = configs.TINY
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    N, M = cfg.batch, cfg.micro
    cell = make_cell(cfg, params)
    gpu = run_gpu(cfg, params, x, t, N, M, remat=False, update=False, cell=cell)
    ref = tc.cell_step(params, x, t, M, cfg.heads, cfg.causal, remat=False, record=True)
    ws = cell._ws.cpu().numpy()
    b, T, D, S, H = N // M, (N // M) * cfg.seq, cfg.d_model, cfg.seq, cfg.heads
    lds = -(-S // 8) * 8
    shapes = {"x": (T, D), "h1": (T, D), "qkv": (T, 3 * D), "ctx": (T, D), "x1": (T, D),
              "h2": (T, D), "u": (T, cfg.d_ff), "g": (T, cfg.d_ff), "p": (b, H, S, lds)}
    for m in range(M):
        for l in range(cfg.layers):
            sv = ref["forward_saved"][m][l]
            for w, name in enumerate(gpipe.SAVED):
                if name in ("st1", "st2") or (l == 0 and name == "x"):
                    continue
                off, nb = gpipe.gpipe_cell_saved_offset(cell.handle, N, M, False, m, l, w)
                a = ws[off:off + nb].view(np.float32).reshape(shapes[name])
                if name == "p":
                    a = a[..., :S]
                    r = sv["prob"]
                else:
                    r = sv[name].reshape(shapes[name])
                e = rel_l2(a, r)
                assert e < FP32_TOL, (m, l, name, e)
            for w, name, key in ((2, "st1", ("mu1", "rstd1")), (8, "st2", ("mu2", "rstd2"))):
                off, nb = gpipe.gpipe_cell_saved_offset(cell.handle, N, M, False, m, l, w)
                a = ws[off:off + nb].view(np.float32).reshape(T, 2)
                assert rel_l2(a[:, 0], sv[key[0]].ravel()) < 1e-4
                assert rel_l2(a[:, 1], sv[key[1]].ravel()) < 1e-4
    assert rel_l2(gpu["y"], ref["y"]) < FP32_TOL


def test_tiny_fp32_step_and_update():
    check(configs.TINY)


def test_tiny_fp32_causal():
    check(configs.TINY.with_(causal=True))


@pytest.mark.parametrize("M", [1, 2, 8])
def test_tiny_fp32_micro_batch_counts(M):
    check(configs.TINY, M=M)


def test_ragged_shapes_fp32():
    """T = 3*40 = 120 tokens (not a tile multiple), S = 40 (ragged attention tiles)."""
    cfg = configs.TINY.with_(name="ragged_fp32", seq=40, batch=6, micro=2, d_model=96, heads=6,
                             d_ff=200)
    check(cfg)
    check(cfg.with_(causal=True))


def test_odd_sequence_length_fp32():
    """S = 13: rows of the attention matrices are not a multiple of 8."""
    cfg = configs.TINY.with_(name="s13_fp32", seq=13, batch=4, micro=2, causal=True)
    check(cfg)


def test_single_token_sequences_fp32():
    cfg = configs.TINY.with_(name="s1_fp32", seq=1, batch=8, micro=4)
    check(cfg)


def test_single_head_fp32():
    cfg = configs.TINY.with_(name="h1_fp32", heads=1, seq=24, batch=4, micro=2)
    check(cfg)


def test_remat_bitwise_equals_stored_fp32():
    cfg = configs.TINY.with_(causal=True)
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    a = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=True, update=False)
    b = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=False, update=False)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dx"], b["dx"])
    assert a["loss"] == b["loss"]
    for ga, gb in zip(a["grad"], b["grad"]):
        for n in gpipe.TENSORS:
            assert np.array_equal(ga[n], gb[n]), n


def test_step_is_deterministic_bf16():
    cfg = configs.SMALL.with_(name="small_2l", layers=2, batch=8, micro=4)
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg, batch=8)
    a = run_gpu(cfg, params, x, t, 8, 4, update=False)
    b = run_gpu(cfg, params, x, t, 8, 4, update=False, remat=False)
    c = run_gpu(cfg, params, x, t, 8, 4, update=False)
    for o in (b, c):
        assert np.array_equal(a["y"], o["y"]) and np.array_equal(a["dx"], o["dx"])
        for ga, gb in zip(a["grad"], o["grad"]):
            for n in gpipe.TENSORS:
                assert np.array_equal(ga[n], gb[n]), n


def test_small_bf16_reduced():
    """The small cell's layer shapes (D=512, H=8, F=2048, S=128) at 2 layers, N=8, M=4."""
    check(configs.SMALL.with_(name="small_2l", layers=2, batch=8, micro=4))


def test_small_bf16_causal_reduced():
    check(configs.SMALL.with_(name="small_2l_causal", layers=2, batch=4, micro=2, causal=True))


def test_ragged_shapes_bf16():
    """bf16 tiles with ragged edges: T = 80, D = 96 (head_dim 24), F = 200, S = 40."""
    cfg = configs.SMALL.with_(name="ragged_bf16", layers=2, d_model=96, heads=4, d_ff=200, seq=40,
                              batch=4, micro=2)
    check(cfg)
    check(cfg.with_(causal=True))


@pytest.fixture(scope="module")
def small_oracle():
    """One oracle step of the small cell (6 layers, N=64): the full mini-batch's
    step, which every micro-batch count reaches (M=8 here; the LayerNorm cell's
    result does not depend on M)."""
    cfg = configs.SMALL
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    return cfg, params, x, t, oracle_step(cfg, params, x, t, cfg.micro)


def test_small_bf16_full(small_oracle):
    """The small cell as specified: 6 layers, N=64, M=8."""
    cfg, params, x, t, ref = small_oracle
    gpu = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro)
    report, bad = compare_step(gpu, ref, BF16_TOL)
    assert not bad, bad


def test_small_bf16_one_micro_batch_matches_oracle(small_oracle):
    """M=1 (the full-batch step, 8192 tokens per launch) against the oracle, and
    against the M=8 run."""
    cfg, params, x, t, ref = small_oracle
    g1 = run_gpu(cfg, params, x, t, cfg.batch, 1)
    report, bad = compare_step(g1, ref, BF16_TOL)
    assert not bad, bad
    g8 = run_gpu(cfg, params, x, t, cfg.batch, 8, update=False)
    # the tile / split-K plan depends on the rows per micro-batch, so the two runs
    # sum in different orders: equal up to bf16 rounding, not bitwise
    assert rel_l2(g1["y"], g8["y"]) < 1e-2
    for a, b in zip(g1["grad"], g8["grad"]):
        for n in gpipe.TENSORS:
            assert rel_l2(a[n], b[n]) < 1e-2, n


def test_small_bf16_remat_bitwise_equals_stored():
    """The small cell as specified (N=64, M=8: its down-projection splits over k
    at 1024 rows, so the forward phase runs one micro-batch per launch on three
    lanes): re-materialization reproduces the stored run bit for bit."""
    cfg = configs.SMALL
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    a = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=True, update=False)
    b = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=False, update=False)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dx"], b["dx"])
    for ga, gb in zip(a["grad"], b["grad"]):
        for n in gpipe.TENSORS:
            assert np.array_equal(ga[n], gb[n]), n


@pytest.mark.parametrize("layers,d_ff,batch,micro", [(6, 2048, 16, 8), (4, 4096, 10, 5)])
def test_grouped_forward_with_split_products_bitwise_bf16(layers, d_ff, batch, micro):
    """Grouped forward launches whose down-projection splits over k: the small
    cell's layers at 256-token micro-batches (three per launch, 4 splits; the
    last group of two) and d_ff 4096 (two per launch, 8 splits, a last group of
    one).  Each lane's split-K partials hold the grouped launch, and the
    boundary outputs and every gradient equal the stored-activation run bit
    for bit; the step matches the oracle."""
    cfg = configs.SMALL.with_(name=f"grouped_split_l{layers}_f{d_ff}_m{micro}", layers=layers,
                              d_ff=d_ff, batch=batch, micro=micro)
    cell = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq,
                                   cfg.causal, gpipe.GPIPE_BF16)
    try:
        lanes, G, _ = gpipe.gpipe_cell_forward_plan(cell, batch, micro, True)
    finally:
        gpipe.gpipe_cell_destroy(cell)
    say(f"[plan] forward lanes={lanes} group={G}")
    assert G >= 2 and micro % G != 0
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    a = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=True, update=False)
    b = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=False, update=False)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dx"], b["dx"])
    for ga, gb in zip(a["grad"], b["grad"]):
        for n in gpipe.TENSORS:
            assert np.array_equal(ga[n], gb[n]), n
    check(cfg)


def two_steps(cfg, N=None, M=None):
    """Two consecutive GPU steps + updates (the second reads the RMSProp state and
    the bf16 copy the first update wrote, and overwrites the gradients) against two
    oracle train steps with the state carried."""
    import torch
    N = cfg.batch if N is None else N
    M = cfg.micro if M is None else M
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg, batch=N)
    tol = FP32_TOL if cfg.precision == "fp32" else BF16_TOL
    cell = make_cell(cfg, params)
    ref1 = oracle_step(cfg, params, x, t, M)
    g1 = run_gpu(cfg, params, x, t, N, M, cell=cell)
    report, bad = compare_step(g1, ref1, tol)
    assert not bad, ("step 1", bad)
    if cell.bf16:
        want = inputs.round_to_bf16(cell.master.cpu().numpy())
        assert np.array_equal(g1["w_lowp"], want), "w_lowp != bf16(master) after update 1"
    # step 2 from the oracle's own updated weights and mean-square state
    ref2 = tc.train_step(ref1["w_new"], x, t, M, cfg.heads, cfg.causal, cfg.lr, cfg.decay, cfg.eps,
                         ms=ref1["ms_new"], ln_eps=cfg.ln_eps)
    g2 = run_gpu(cfg, params, x, t, N, M, cell=cell)
    report, bad = compare_step(g2, ref2, tol)
    assert not bad, ("step 2", bad)
    if cell.bf16:
        want = inputs.round_to_bf16(cell.master.cpu().numpy())
        assert np.array_equal(g2["w_lowp"], want), "w_lowp != bf16(master) after update 2"
    torch.cuda.synchronize()


def test_two_steps_fp32():
    two_steps(configs.TINY)


def test_two_steps_bf16_reduced():
    """The small cell's layer shapes at 2 layers, N=8, M=4 (fused attention,
    grouped forward, pipelined re-materialization)."""
    two_steps(configs.SMALL.with_(name="small_2l_two_steps", layers=2, batch=8, micro=4))


def test_cell_2048_layer_shapes_bf16():
    """The 2048-wide causal cell's layers at their real micro-batch (2 sequences, 1024
    tokens): two micro-batches, so every GEMM, split and tile is the one the
    benchmark runs.  Oracle in float32 for time."""
    cfg = configs.CELL_2048.with_(name="cell2048_n4", batch=4, micro=2)
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg, batch=4)
    gpu = run_gpu(cfg, params, x, t, 4, 2)
    ref = tc.train_step(params, x, t, 2, cfg.heads, cfg.causal, cfg.lr, cfg.decay, cfg.eps,
                        dtype=np.float32)
    report, bad = compare_step(gpu, ref, BF16_TOL)
    assert not bad, bad


def test_ragged_tiles_direct_lds_path_bf16():
    """k extents multiples of 64 (the direct-to-LDS GEMM) with ragged M / N edges:
    T = 192 rows per micro-batch, D = 320, F = 832, S = 192, head_dim 64."""
    cfg = configs.SMALL.with_(name="dma_ragged_bf16", layers=2, d_model=320, heads=5, d_ff=832,
                              seq=192, batch=2, micro=2)
    check(cfg)
    check(cfg.with_(causal=True))


def test_ragged_tiles_specialised_kernel_bf16():
    """The specialised-wave GEMM (loader and MFMA waves) with ragged M / N edges on
    k-contiguous and m-contiguous operands: 128 x 128 tiles (forward products, the
    out-projection weight gradient) and 256 x 128 / 128 x 256 tiles (the other
    backward products); T = 576 rows per micro-batch, D = 1152, F = 4160, S = 288,
    head_dim 128 (the plans are checked on the host)."""
    cfg = configs.SMALL.with_(name="spec_ragged_bf16", layers=1, d_model=1152, heads=9,
                              d_ff=4160, seq=288, batch=2, micro=1)
    check(cfg)


def test_ragged_wide_tiles_specialised_kernel_bf16():
    """128 x 128 tiles of the specialised-wave GEMM with ragged M and N on a wide
    output (T = 576, D = 2528, F = 2112: ffn2_fwd and ffn1_dgrad, k-contiguous and
    m-contiguous B operands), unfused attention (head_dim 632)."""
    cfg = configs.SMALL.with_(name="spec_ragged_narrow_bf16", layers=1, d_model=2528, heads=4,
                              d_ff=2112, seq=288, batch=2, micro=1)
    check(cfg)


def test_ragged_big_tiles_specialised_kernel_bf16():
    """256 x 128 and 128 x 256 tiles of the specialised-wave GEMM with ragged M and N
    (the weight gradients and their fused bias sums: F = 4160, D = 1600, T = 640),
    head_dim 64."""
    cfg = configs.SMALL.with_(name="spec_ragged_big_bf16", layers=1, d_model=1600, heads=25,
                              d_ff=4160, seq=320, batch=2, micro=1)
    check(cfg)


@pytest.mark.parametrize("dh,seq", [(128, 100), (64, 70), (128, 64), (64, 1)])
def test_fused_attention_ragged_sequences_bf16(dh, seq):
    """The fused attention kernels (bf16, head dim 64 / 128) with sequence lengths
    that are not multiples of their 64-row blocks, causal and not."""
    heads = 2
    cfg = configs.SMALL.with_(name=f"fused_dh{dh}_s{seq}", layers=2, d_model=dh * heads,
                              heads=heads, d_ff=4 * dh, seq=seq, batch=6, micro=3)
    check(cfg)
    check(cfg.with_(causal=True))


@pytest.mark.parametrize("batch", [4, 6])
def test_remat_with_split_products_bitwise_bf16(batch):
    """With the FFN down-projection split over k (d_ff 4096) and the forward
    phase on two streams, the re-materialized intermediates, and so every
    gradient, equal the stored-activation run bit for bit."""
    cfg = configs.SMALL.with_(name=f"remat_split_b{batch}", layers=2, d_model=512, heads=4,
                              d_ff=4096, seq=128, batch=batch, micro=2, causal=True)
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    a = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=True, update=False)
    b = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=False, update=False)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dx"], b["dx"])
    for ga, gb in zip(a["grad"], b["grad"]):
        for n in gpipe.TENSORS:
            assert np.array_equal(ga[n], gb[n]), n
    check(cfg)


@pytest.mark.parametrize("layers,micro", [(4, 5), (8, 7)])
def test_grouped_forward_phase_bitwise_bf16(layers, micro):
    """The forward phase runs several micro-batches per launch (with a shorter
    last group when they do not divide evenly); its boundary outputs, and the
    re-materialized intermediates behind every gradient, equal the
    stored-activation run bit for bit."""
    cfg = configs.SMALL.with_(name=f"grouped_fwd_l{layers}_m{micro}", layers=layers, d_model=256,
                              heads=2, d_ff=512, seq=100, batch=2 * micro, micro=micro,
                              causal=True)
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    a = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=True, update=False)
    b = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=False, update=False)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dx"], b["dx"])
    for ga, gb in zip(a["grad"], b["grad"]):
        for n in gpipe.TENSORS:
            assert np.array_equal(ga[n], gb[n]), n


def test_fused_attention_remat_bitwise_bf16():
    """Remat through the fused attention equals stored activations bit for bit."""
    cfg = configs.SMALL.with_(name="fused_remat", layers=2, d_model=256, heads=2, d_ff=512,
                              seq=100, batch=4, micro=2, causal=True)
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg)
    a = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=True, update=False)
    b = run_gpu(cfg, params, x, t, cfg.batch, cfg.micro, remat=False, update=False)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dx"], b["dx"])
    for ga, gb in zip(a["grad"], b["grad"]):
        for n in gpipe.TENSORS:
            assert np.array_equal(ga[n], gb[n]), n


def test_profiled_step_bitwise_and_sampled_launch_counts():
    """Timing roles with events changes no result, and timing every k-th launch
    of a role records ceil(n / k) of its n launches."""
    import math
    cfg = configs.SMALL.with_(name="small_2l", layers=2, batch=8, micro=4)
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg, batch=8)
    plain = run_gpu(cfg, params, x, t, 8, 4, update=False)
    cell = make_cell(cfg, params)
    all_roles = (1 << len(gpipe.ROLES)) - 1
    gpipe.gpipe_cell_profile(cell.handle, all_roles)
    timed = run_gpu(cfg, params, x, t, 8, 4, update=False, cell=cell)
    assert np.array_equal(plain["y"], timed["y"]) and np.array_equal(plain["dx"], timed["dx"])
    for ga, gb in zip(plain["grad"], timed["grad"]):
        for n in gpipe.TENSORS:
            assert np.array_equal(ga[n], gb[n]), n
    full = {}
    for r, name in enumerate(gpipe.ROLES):
        ms, cnt = gpipe.gpipe_cell_profile_read(cell.handle, r)
        if cnt:
            assert ms > 0, name
            full[name] = cnt
    assert full.get("ffn1_fwd", 0) >= cfg.layers * 4, full
    for every in (3, 7):
        gpipe.gpipe_cell_profile_sampled(cell.handle, all_roles, every)
        run_gpu(cfg, params, x, t, 8, 4, update=False, cell=cell)
        for r, name in enumerate(gpipe.ROLES):
            ms, cnt = gpipe.gpipe_cell_profile_read(cell.handle, r)
            assert cnt == math.ceil(full.get(name, 0) / every), (name, every, cnt, full.get(name))
    with pytest.raises(RuntimeError):
        gpipe.gpipe_cell_profile_sampled(cell.handle, all_roles, 0)
    gpipe.gpipe_cell_profile(cell.handle, 0)


@pytest.mark.parametrize("cfg", [configs.TINY,
                                 configs.SMALL.with_(name="small_3l", layers=3, batch=8, micro=4)],
                         ids=["tiny_fp32", "small_3l_bf16"])
def test_step_update_equals_step_then_update(cfg):
    """gpipe_cell_step_update (each layer's RMSProp update enqueued once its gradients are
    complete, beside the backward of the layers below it) leaves bitwise what
    gpipe_cell_step followed by gpipe_apply_update leaves: outputs, loss, gradients,
    weights, mean squares and the bf16 copy -- over two calls in a row (the second reads
    the first's update), with re-materialization (pipelined for the bf16 cell) and
    without."""
    import torch
    params = inputs.cell_params(cfg)
    x, t = inputs.cell_data(cfg, batch=cfg.batch)
    N, M = cfg.batch, cfg.micro
    for remat in (True, False):
        a, b = make_cell(cfg, params), make_cell(cfg, params)
        xd, td = a.to_device(x), a.to_device(t)
        say(f"[gpu] step_update {cfg.name} N={N} M={M} remat={remat}")
        for k in range(2):
            ya, dxa = a.step(xd, td, N, M, remat=remat)
            a.update(cfg.lr, cfg.decay, cfg.eps)
            yb, dxb = b.step_update(xd, td, N, M, cfg.lr, cfg.decay, cfg.eps, remat=remat)
            torch.cuda.synchronize()
            assert torch.equal(ya, yb) and torch.equal(dxa, dxb), (remat, k)
            assert a.loss.item() == b.loss.item(), (remat, k)
            for name in ("grad", "master", "ms"):
                assert torch.equal(getattr(a, name), getattr(b, name)), (remat, k, name)
            if a.bf16:
                assert torch.equal(a.w_lowp, b.w_lowp), (remat, k)
    with pytest.raises(RuntimeError):
        b.step_update(xd, td, N, M, cfg.lr, 1.5, cfg.eps)

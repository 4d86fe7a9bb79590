"""Host logic of the C-ABI library, on the CPU: exports, layout, planner, partition, errors.

No device work is launched here.
"""
import os
import random
import re

import numpy as np
import pytest

from micro_pipelined_re_amd import configs, gpipe, inputs
from oracle.partition import partition_bruteforce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ws_plan(h, n, m, remat):
    """The planned workspace bytes, whether or not the current device would fit them."""
    return gpipe.gpipe_cell_workspace_fit(h, n, m, remat)[0]


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gpipe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gpipe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = gpipe.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(gpipe.EXPORTS) == names


def test_status_strings():
    assert gpipe.gpipe_status_string(0) == "ok"
    assert "memory" in gpipe.gpipe_status_string(2)


@pytest.mark.parametrize("cfg", [configs.TINY, configs.SMALL, configs.CELL_2048, configs.MEMORY_4096])
def test_param_layout_matches_documented_order(cfg):
    h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq,
                                cfg.causal, gpipe.GPIPE_BF16)
    try:
        n = gpipe.gpipe_cell_param_count(h)
        assert n == cfg.param_count()
        shapes = inputs.param_shapes(cfg.d_model, cfg.d_ff)
        expect = 0
        for l in range(cfg.layers):
            for t, name in enumerate(gpipe.TENSORS):
                off, cnt = gpipe.gpipe_cell_param_offset(h, l, t)
                assert off == expect and cnt == int(np.prod(shapes[name]))
                assert off % 8 == 0
                expect += cnt
        assert expect == n
        assert tuple(gpipe.TENSORS) == inputs.PARAM_NAMES
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_param_counts_of_the_workloads():
    # tiny: 2 * (4*64^2 + 2*64*256 + 9*64 + 256) = 99,968
    assert configs.TINY.param_count() == 99968
    assert configs.CELL_2048.param_count() == 402_866_176
    assert abs(configs.MEMORY_4096.param_count() - 9.666e9) < 1e7


def fused_attention(cfg):
    """bf16 cells with head dim 64 or 128 run the fused attention kernels."""
    return cfg.precision == "bf16" and cfg.d_model // cfg.heads in (64, 128)


def saved_set_bytes_formula(cfg, n, m, eb):
    """Per micro-batch set: L * T * ((8D + 2F) * eb + 16 + a) bytes, where the
    attention term a is H * S' * eb for stored probabilities (S' = S rounded to
    8) or 4 H for the fused kernels' row log-sum-exp."""
    b = n // m
    t = b * cfg.seq
    lds = -(-cfg.seq // 8) * 8
    attn = 4 * cfg.heads if fused_attention(cfg) else cfg.heads * lds * eb
    return cfg.layers * t * ((8 * cfg.d_model + 2 * cfg.d_ff) * eb + 16 + attn)


@pytest.mark.parametrize("cfg", [configs.TINY, configs.SMALL, configs.CELL_2048, configs.MEMORY_4096])
def test_workspace_tracks_the_activation_bound(cfg):
    """Remat keeps one micro-batch's saved set (and, where the backward phase
    is pipelined -- fused attention, two or more layers -- one spare layer
    slot for the next micro-batch's top layer), no-remat keeps M of them.

    The pages put re-materialized peak activations at O(N + L/K * N/M): the N
    term is the boundary (the caller's x / y), the second term one saved set.
    """
    eb = 4 if cfg.precision == "fp32" else 2
    prec = gpipe.GPIPE_FP32 if eb == 4 else gpipe.GPIPE_BF16
    h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq,
                                cfg.causal, prec)
    try:
        n, m = cfg.batch, cfg.micro
        remat = ws_plan(h, n, m, True)
        keep = ws_plan(h, n, m, False)
        formula = saved_set_bytes_formula(cfg, n, m, eb)
        set_bytes = (gpipe.gpipe_cell_saved_offset(h, n, m, False, 1, 0, 1)[0]
                     - gpipe.gpipe_cell_saved_offset(h, n, m, False, 0, 0, 1)[0])
        # the set is the formula up to 256-byte padding of its 11 tensors per layer
        assert formula <= set_bytes <= formula + 256 * 11 * cfg.layers
        yre = -(-(n // m) * cfg.seq * cfg.d_model * eb // 256) * 256
        spare = set_bytes // cfg.layers if fused_attention(cfg) and cfg.layers >= 2 else 0
        assert keep - remat == (m - 1) * set_bytes - yre - spare
        # transients are about one layer's worth (the spare layer slot, two
        # copies of the gradients the weight-gradient stream reads, the other
        # backward buffers) plus each stream's split-K partials, small next to
        # the set for the deep cells
        transient = remat - set_bytes
        assert transient > 0
        if cfg.layers >= 8:
            assert transient < 0.6 * set_bytes
        # halving the micro-batch halves the set
        if n % (2 * m) == 0:
            assert ws_plan(h, n, 2 * m, True) < 0.6 * remat + transient
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_memory_cell_at_one_micro_batch_exceeds_one_gpu():
    """48 layers of d_model 4096, N=32: at M=1 the saved activations (~211 GB
    with the fused attention's row statistics in place of the probabilities)
    plus the parameter state (bf16 copy, fp32 master, RMSProp and gradient:
    14 B/param, ~135 GB) exceed one GPU's 288 GB; at M=32 the workspace is
    about 1/32 of that."""
    cfg = configs.MEMORY_4096
    h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq, False,
                                gpipe.GPIPE_BF16)
    try:
        m1 = ws_plan(h, 32, 1, True)
        m32 = ws_plan(h, 32, 32, True)
        state = gpipe.gpipe_cell_param_count(h) * 14
        assert m1 + state > 288e9
        assert m1 > 200e9
        assert m1 / 40 < m32 < m1 / 25
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_create_validation():
    E = gpipe.GpipeError
    with pytest.raises(E) as e:
        gpipe.gpipe_cell_create(2, 64, 3, 256, 32, 0, 0)       # heads do not divide d_model
    assert e.value.code == 1
    with pytest.raises(E) as e:
        gpipe.gpipe_cell_create(0, 64, 4, 256, 32, 0, 0)
    assert e.value.code == 1
    with pytest.raises(E) as e:
        gpipe.gpipe_cell_create(2, 60, 4, 256, 32, 0, 0)       # d_model not a multiple of 8
    assert e.value.code == 4
    with pytest.raises(E) as e:
        gpipe.gpipe_cell_create(2, 64, 4, 256, 5000, 0, 0)     # seq too long
    assert e.value.code == 4


def test_workspace_and_step_validation_without_device():
    h = gpipe.gpipe_cell_create(2, 64, 4, 256, 32, 0, gpipe.GPIPE_FP32)
    try:
        with pytest.raises(gpipe.GpipeError):
            ws_plan(h, 8, 3, True)      # N % M != 0
        with pytest.raises(gpipe.GpipeError):
            ws_plan(h, 0, 1, True)
        # stepping an unbound cell is a state error; nothing is launched
        with pytest.raises(gpipe.GpipeError) as e:
            gpipe.gpipe_cell_step(h, 16, 16, 16, None, 8, 4, True, 16, 1 << 30, 0, 16)
        assert e.value.code == 5
        with pytest.raises(gpipe.GpipeError) as e:
            gpipe.gpipe_apply_update(h, 1e-3, 0.9, 1e-8, 0)
        assert e.value.code == 5
        # bf16 cells need the low-precision copy; fp32 cells must not get one
        with pytest.raises(gpipe.GpipeError):
            gpipe.gpipe_cell_bind(h, 256, 256, 256, 256)
        # misaligned pointers are rejected
        with pytest.raises(gpipe.GpipeError):
            gpipe.gpipe_cell_bind(h, 258, None, 256, 256)
        gpipe.gpipe_cell_bind(h, 256, None, 512, 768)            # host-side bookkeeping only
        ws = ws_plan(h, 8, 4, True)
        with pytest.raises(gpipe.GpipeError) as e:               # workspace too small
            gpipe.gpipe_cell_step(h, 16, 16, 16, None, 8, 4, True, 16, ws - 1, 0, 16)
        assert e.value.code == 1
        with pytest.raises(gpipe.GpipeError) as e:               # misaligned x
            gpipe.gpipe_cell_step(h, 18, 16, 16, None, 8, 4, True, 16, ws, 0, 16)
        assert e.value.code == 1
        with pytest.raises(gpipe.GpipeError):                    # bad decay
            gpipe.gpipe_apply_update(h, 1e-3, 1.0, 1e-8, 0)
        # the split phases: forward needs y, backward needs dy; checked before any launch
        with pytest.raises(gpipe.GpipeError) as e:
            gpipe.gpipe_cell_forward(h, 16, None, 8, 4, True, 16, ws, 0)
        assert e.value.code == 1
        with pytest.raises(gpipe.GpipeError) as e:
            gpipe.gpipe_cell_backward(h, 16, None, 16, 8, 4, True, 16, ws, 0)
        assert e.value.code == 1
        with pytest.raises(gpipe.GpipeError) as e:               # misaligned dy
            gpipe.gpipe_cell_backward(h, 16, 24, 16, 8, 4, True, 16, ws, 0)
        assert e.value.code == 1
        with pytest.raises(gpipe.GpipeError) as e:               # workspace too small
            gpipe.gpipe_cell_backward(h, 16, 32, 16, 8, 4, True, 16, ws - 1, 0)
        assert e.value.code == 1
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_saved_offsets_are_disjoint_and_inside_the_workspace():
    cfg = configs.TINY
    h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq, 0, 0)
    try:
        for remat in (True, False):
            ws = ws_plan(h, 8, 4, remat)
            spans = []
            for m in range(1 if remat else 4):
                for l in range(cfg.layers):
                    for w in range(len(gpipe.SAVED)):
                        if l == 0 and w == 0:
                            with pytest.raises(gpipe.GpipeError):
                                gpipe.gpipe_cell_saved_offset(h, 8, 4, remat, m, l, w)
                            continue
                        off, nb = gpipe.gpipe_cell_saved_offset(h, 8, 4, remat, m, l, w)
                        assert off % 256 == 0 and off + nb <= ws
                        spans.append((off, off + nb))
            spans.sort()
            for a, b in zip(spans, spans[1:]):
                assert a[1] <= b[0]
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_partition_matches_bruteforce_oracle():
    rng = random.Random(7)
    for _ in range(300):
        L = rng.randint(1, 12)
        K = rng.randint(1, L)
        costs = [float(rng.randint(0, 20)) for _ in range(L)]
        b, v = gpipe.gpipe_partition(costs, K)
        ob, ov = partition_bruteforce(costs, K)
        assert b == ob, (costs, K)
        assert v == pytest.approx(float(ov), rel=1e-12, abs=1e-12)


def test_partition_uniform_and_large():
    b, v = gpipe.gpipe_partition([1.0] * 128, 16)
    assert b == list(range(0, 129, 8)) and v == 0.0
    costs = [float(c) for c in np.random.default_rng(1).integers(1, 100, 200)]
    b, v = gpipe.gpipe_partition(costs, 16)
    assert b[0] == 0 and b[-1] == 200 and all(x < y for x, y in zip(b, b[1:]))


def test_partition_validation():
    for costs, k in [([1.0, 2.0], 3), ([1.0, -1.0], 1), ([float("nan")], 1), ([1.0], 0)]:
        with pytest.raises(gpipe.GpipeError):
            gpipe.gpipe_partition(costs, k)


# ---------------------------------------------------------------- conv cells
@pytest.mark.parametrize("cfg", [configs.CONV_TINY, configs.CONV_SMALL, configs.CONV_CELL])
def test_conv_param_layout_matches_documented_order(cfg):
    h = gpipe.gpipe_conv_cell_create(cfg.blocks, cfg.channels, cfg.height, cfg.width,
                                     cfg.bn_momentum, gpipe.GPIPE_BF16)
    try:
        n = gpipe.gpipe_cell_param_count(h)
        assert n == cfg.param_count()
        shapes = inputs.conv_param_shapes(cfg.channels)
        expect = 0
        for l in range(cfg.blocks):
            for t, name in enumerate(gpipe.CONV_TENSORS):
                off, cnt = gpipe.gpipe_cell_param_offset(h, l, t)
                assert off == expect and cnt == int(np.prod(shapes[name]))
                expect += cnt
            with pytest.raises(gpipe.GpipeError):
                gpipe.gpipe_cell_param_offset(h, l, len(gpipe.CONV_TENSORS))
        assert expect == n
        assert tuple(gpipe.CONV_TENSORS) == inputs.CONV_NAMES
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_conv_param_count_of_the_workload():
    # 8 blocks * (2 * 9 * 256^2 + 4 * 256) = 8 * 1,180,672
    assert configs.CONV_CELL.param_count() == 9_445_376


def test_conv_create_and_bind_validation():
    E = gpipe.GpipeError
    with pytest.raises(E) as e:
        gpipe.gpipe_conv_cell_create(2, 12, 8, 8, 0.9, 0)        # channels not a multiple of 8
    assert e.value.code == 4
    for bad in ((0, 16, 8, 8, 0.9), (2, 16, 0, 8, 0.9), (2, 16, 8, 8, 1.0), (2, 16, 8, 8, -0.1)):
        with pytest.raises(E) as e:
            gpipe.gpipe_conv_cell_create(*bad, 0)
        assert e.value.code == 1
    t = gpipe.gpipe_cell_create(2, 64, 4, 256, 32, 0, 0)
    try:
        with pytest.raises(E) as e:                               # not a conv cell
            gpipe.gpipe_cell_bind_running(t, 256)
        assert e.value.code == 1
    finally:
        gpipe.gpipe_cell_destroy(t)
    cfg = configs.CONV_TINY
    h = gpipe.gpipe_conv_cell_create(cfg.blocks, cfg.channels, cfg.height, cfg.width, 0.9, 0)
    try:
        gpipe.gpipe_cell_bind(h, 256, None, 512, 768)            # host-side bookkeeping only
        ws = ws_plan(h, 8, 4, True)
        with pytest.raises(E) as e:                               # moving averages not bound
            gpipe.gpipe_cell_step(h, 16, 16, 16, None, 8, 4, True, 16, ws, 0, 16)
        assert e.value.code == 5
        with pytest.raises(E):                                    # misaligned running
            gpipe.gpipe_cell_bind_running(h, 260)
        gpipe.gpipe_cell_bind_running(h, 1024)
        with pytest.raises(E) as e:                               # workspace too small
            gpipe.gpipe_cell_step(h, 16, 16, 16, None, 8, 4, True, 16, ws - 1, 0, 16)
        assert e.value.code == 1
        with pytest.raises(E) as e:                               # N % M != 0
            gpipe.gpipe_cell_step(h, 16, 16, 16, None, 8, 3, True, 16, ws, 0, 16)
        assert e.value.code == 1
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_conv_saved_offsets_and_workspace_scaling():
    cfg = configs.CONV_TINY
    h = gpipe.gpipe_conv_cell_create(cfg.blocks, cfg.channels, cfg.height, cfg.width, 0.9, 0)
    try:
        P = (8 // 4) * cfg.height * cfg.width
        for remat in (True, False):
            ws = ws_plan(h, 8, 4, remat)
            spans = []
            for m in range(1 if remat else 4):
                for l in range(cfg.blocks):
                    for w, name in enumerate(gpipe.CONV_SAVED):
                        if l == 0 and w == 0:
                            with pytest.raises(gpipe.GpipeError):
                                gpipe.gpipe_cell_saved_offset(h, 8, 4, remat, m, l, w)
                            continue
                        off, nb = gpipe.gpipe_cell_saved_offset(h, 8, 4, remat, m, l, w)
                        assert nb == (2 * cfg.channels * 4 if name.startswith("st")
                                      else P * cfg.channels * 4)
                        assert off % 256 == 0 and off + nb <= ws
                        spans.append((off, off + nb))
            spans.sort()
            for a, b in zip(spans, spans[1:]):
                assert a[1] <= b[0]
        # re-materialization keeps one micro-batch's set (plus the re-computed
        # output); without it every micro-batch's set is kept
        r = [ws_plan(h, 64, m, True) for m in (1, 2, 4)]
        s = [ws_plan(h, 64, m, False) for m in (1, 2, 4)]
        assert r[0] > r[1] > r[2]
        set_bytes = (gpipe.gpipe_cell_saved_offset(h, 64, 4, False, 1, 0, 1)[0]
                     - gpipe.gpipe_cell_saved_offset(h, 64, 4, False, 0, 0, 1)[0])
        y_bytes = 16 * cfg.height * cfg.width * cfg.channels * 4
        assert s[2] - r[2] == 3 * set_bytes - y_bytes
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_conv_workspace_drops_the_column_matrix_with_the_gathered_weight_gradient():
    """bf16, channels a multiple of 64 and pixels per micro-batch a multiple of
    64: no im2col matrix [P, 9C] in the workspace; with 105 pixels per
    micro-batch the weight gradient takes the column matrix again."""
    def ws(h, w, n, m):
        hd = gpipe.gpipe_conv_cell_create(2, 64, h, w, 0.9, gpipe.GPIPE_BF16)
        try:
            return ws_plan(hd, n, m, True)
        finally:
            gpipe.gpipe_cell_destroy(hd)
    row = 9 * 64 * 2                         # one pixel's column-matrix row, bf16
    a = ws(8, 8, 4, 4)                       # 64 pixels: gathered
    b = ws(5, 7, 6, 2)                       # 105 pixels: explicit
    assert b - a >= 105 * row


def test_conv_gemm_plan_of_the_workload():
    cfg = configs.CONV_CELL
    h = gpipe.gpipe_conv_cell_create(cfg.blocks, cfg.channels, cfg.height, cfg.width, 0.9,
                                     gpipe.GPIPE_BF16)
    try:
        R = {n: i for i, n in enumerate(gpipe.ROLES)}
        # weight gradient: [256 x 2304] reduced over 16384 pixels -> split-K
        assert gpipe.gpipe_cell_gemm_plan(h, cfg.batch, cfg.micro, R["conv_wgrad"])[2] > 1
        # the gathered weight gradient: 128 x 128 tiles, seven splits (252 workgroups)
        assert gpipe.gpipe_cell_gemm_plan(h, cfg.batch, cfg.micro,
                                          R["conv_wgrad_implicit"]) == (128, 128, 7)
        assert gpipe.gpipe_cell_gemm_plan(h, cfg.batch, cfg.micro, R["conv_fwd"])[:2] == (128, 128)
        assert gpipe.gpipe_cell_gemm_plan(h, cfg.batch, cfg.micro, R["bn_stats"]) == (0, 0, 0)
    finally:
        gpipe.gpipe_cell_destroy(h)


def _cell_plans(cfg, N, M, names):
    h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq,
                                cfg.causal, gpipe.GPIPE_BF16)
    try:
        R = {n: i for i, n in enumerate(gpipe.ROLES)}
        return {n: gpipe.gpipe_cell_gemm_plan(h, N, M, R[n]) for n in names}
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_gemm_plan_of_the_2048_cell():
    """Micro-batches of 1024 tokens: the linear products take 256 x 128 / 128 x 256
    tiles (one workgroup per CU) where the output has at least 192 of them (at
    least 64 for the backward's products), else 128 x 128 tiles, unsplit (the
    step's other streams fill the CUs they leave idle); weight gradients never
    split; 128 x 256 for the weight gradient wider than tall."""
    p = _cell_plans(configs.CELL_2048, 64, 32,
                    ["qkv_fwd", "out_fwd", "ffn1_fwd", "ffn2_fwd", "ffn2_dgrad", "ffn1_dgrad",
                     "out_dgrad", "qkv_dgrad", "ffn1_wgrad", "ffn2_wgrad", "qkv_wgrad",
                     "out_wgrad"])
    assert p["qkv_fwd"] == (128, 256, 1) and p["ffn1_fwd"] == (128, 256, 1)
    assert p["out_fwd"] == (128, 128, 1) and p["ffn2_fwd"] == (128, 128, 1)
    assert p["ffn2_dgrad"] == (256, 128, 1)
    assert p["ffn1_dgrad"] == (256, 128, 1) and p["qkv_dgrad"] == (256, 128, 1)
    assert p["out_dgrad"] == (256, 128, 1)
    for w in ("ffn1_wgrad", "qkv_wgrad", "out_wgrad"):
        assert p[w] == (256, 128, 1)
    assert p["ffn2_wgrad"] == (128, 256, 1)


def test_gemm_plan_of_the_ragged_wide_case():
    """The GPU test of ragged 128 x 128 specialised tiles with a wide output reaches
    them: T = 576 and D = 2528 (neither a multiple of the tile), F = 2112, on a
    k-contiguous (ffn2_fwd) and an m-contiguous (ffn1_dgrad) B operand."""
    cfg = configs.SMALL.with_(layers=1, d_model=2528, heads=4, d_ff=2112, seq=288)
    p = _cell_plans(cfg, 2, 1, ["ffn2_fwd", "ffn1_dgrad"])
    for n in p:
        assert p[n] == (128, 128, 1), (n, p[n])


def test_gemm_plan_of_the_ragged_specialised_case():
    """The shapes of the GPU tests of the specialised kernel's ragged edges do reach it:
    for T = 576, D = 1152, F = 4160, 128 x 128 tiles for the forward products and
    the out-projection weight gradient (45 big tiles), big tiles for the backward
    products with at least 64 of them -- 128 x 256 for the FFN2 weight gradient,
    wider than tall; 256 x 128 tiles for the taller weight gradients of T = 640,
    D = 1600, F = 4160 (128 x 256 for FFN2's)."""
    cfg = configs.SMALL.with_(layers=1, d_model=1152, heads=9, d_ff=4160, seq=288)
    p = _cell_plans(cfg, 2, 1, ["qkv_fwd", "ffn1_fwd", "ffn2_dgrad", "ffn1_wgrad", "ffn2_wgrad",
                                "qkv_wgrad", "out_wgrad"])
    want = {"qkv_fwd": (128, 128, 1), "ffn1_fwd": (128, 128, 1), "out_wgrad": (128, 128, 1),
            "ffn2_dgrad": (256, 128, 1), "ffn1_wgrad": (256, 128, 1), "qkv_wgrad": (256, 128, 1),
            "ffn2_wgrad": (128, 256, 1)}
    for n in p:
        assert p[n] == want[n], (n, p[n])
    cfg = configs.SMALL.with_(layers=1, d_model=1600, heads=25, d_ff=4160, seq=320)
    p = _cell_plans(cfg, 2, 1, ["ffn1_wgrad", "ffn2_wgrad", "qkv_wgrad", "ffn1_fwd"])
    for w in ("ffn1_wgrad", "qkv_wgrad"):
        assert p[w] == (256, 128, 1), (w, p[w])
    assert p["ffn2_wgrad"] == (128, 256, 1)
    assert p["ffn1_fwd"] == (128, 128, 1)


FWD_ROLES = ("qkv_fwd", "out_fwd", "ffn1_fwd", "ffn2_fwd")


def _fwd_out_cols(cfg, role):
    d, f = cfg.d_model, cfg.d_ff
    return {"qkv_fwd": 3 * d, "out_fwd": d, "ffn1_fwd": f, "ffn2_fwd": d}[role]


GROUP_CASES = [
    # the small cell's layers at N=16, M=8: 256-token micro-batches, grouped by
    # three, where the down-projection splits four ways at both sizes
    configs.SMALL.with_(batch=16, micro=8),
    configs.SMALL,                                       # N=64, M=8
    configs.SMALL.with_(batch=24, micro=8),
    configs.SMALL.with_(layers=2, batch=12, micro=6, d_ff=4096, causal=True),
    configs.CELL_2048,
    configs.CELL_2048.with_(batch=12, micro=6),
    configs.SMALL.with_(layers=8, d_model=256, heads=2, d_ff=512, seq=100, batch=14, micro=7),
    configs.SMALL.with_(layers=4, d_model=512, heads=4, d_ff=4096, seq=128, batch=10, micro=5),
]


@pytest.mark.parametrize("cfg", GROUP_CASES, ids=lambda c: f"{c.layers}l_d{c.d_model}_f{c.d_ff}_n{c.batch}_m{c.micro}")
def test_grouped_forward_fits_its_partials_and_keeps_the_k_order(cfg):
    """The forward phase runs G micro-batches per launch only where each forward
    product splits over k the same way at G*T (and at the last group's rows) as
    at T, and each lane's split-K region holds the largest split launch it makes."""
    h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq,
                                cfg.causal, gpipe.GPIPE_BF16)
    try:
        R = {n: i for i, n in enumerate(gpipe.ROLES)}
        N, M = cfg.batch, cfg.micro
        b = N // M
        lanes, G, lane_bytes = gpipe.gpipe_cell_forward_plan(h, N, M, True)
        assert 1 <= G <= M and lanes in (1, 2, 3)
        one = {r: gpipe.gpipe_cell_gemm_plan(h, N, M, R[r]) for r in FWD_ROLES}
        sizes = [g for g in {G, M % G} if g >= 1]
        for g in sizes:
            grp = {r: gpipe.gpipe_cell_gemm_plan(h, g * b, 1, R[r]) for r in FWD_ROLES}
            for r in FWD_ROLES:
                # same number of k-splits (the same K fixes their depth)
                assert grp[r][2] == one[r][2], (g, r, grp[r], one[r])
                rows = g * b * cfg.seq
                if grp[r][2] > 1:
                    need = grp[r][2] * rows * _fwd_out_cols(cfg, r) * 4
                    assert need <= lane_bytes, (g, r, need, lane_bytes)
        for r in FWD_ROLES:
            if one[r][2] > 1:
                assert one[r][2] * b * cfg.seq * _fwd_out_cols(cfg, r) * 4 <= lane_bytes
        # lanes x (G micro-batches' layer slot) fit in one micro-batch's saved set
        if G > 1:
            ws1 = ws_plan(h, N, M, True)
            assert ws1 > 0
        # without re-materialization the forward phase runs one micro-batch at a time
        assert gpipe.gpipe_cell_forward_plan(h, N, M, False)[:2] == (1, 1)
    finally:
        gpipe.gpipe_cell_destroy(h)


def test_grouped_forward_choices_of_the_workloads():
    """The 2048-wide cell groups four 1024-token micro-batches on two lanes; the
    small cell's micro-batches (whose down-projection splits at 1024 rows but
    not at 2048 or more) run one per launch on three lanes."""
    for cfg, want in ((configs.CELL_2048, (2, 4)), (configs.SMALL, (3, 1))):
        h = gpipe.gpipe_cell_create(cfg.layers, cfg.d_model, cfg.heads, cfg.d_ff, cfg.seq,
                                    cfg.causal, gpipe.GPIPE_BF16)
        try:
            assert gpipe.gpipe_cell_forward_plan(h, cfg.batch, cfg.micro, True)[:2] == want
        finally:
            gpipe.gpipe_cell_destroy(h)

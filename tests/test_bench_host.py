"""Host-side logic of bench.py (no GPU): the algorithmic work behind the
roofline figures, the choice of the roofline's kernel, the gate that keeps
counter-measured traffic tied to the GEMM sources it was measured on, and the
refusal of more than one GPU.

The work figures are checked against closed forms written from the model's
shapes (a GEMM of M x N x K is 2 M N K flops; causal attention keeps
S (S + 1) / 2 (query, key) pairs per head), counted here independently of
bench.py's per-role table.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from micro_pipelined_re_amd import configs  # noqa: E402

# roles one step of each workload launches, as the profiling counters report them
CELL_LAUNCHED = ("ffn1_dgrad", "ffn2_fwd", "ffn1_fwd", "ffn2_wgrad", "ffn1_wgrad", "qkv_dgrad",
                 "qkv_fwd", "out_fwd", "ffn2_dgrad", "qkv_wgrad", "attn_fwd", "attn_dq",
                 "out_dgrad", "ln2_fwd", "out_wgrad", "ln2_bwd", "ln1_fwd", "ln1_bwd", "rmsprop",
                 "mse", "norm_grad", "loss_reduce")
CONV_LAUNCHED = ("conv_fwd_implicit", "bn_bwd", "conv_dgrad_implicit", "bn_stats",
                 "bn_apply", "mse", "rmsprop", "bn_running", "loss_reduce")


def step_work_fn(cfg, conv):
    n, m = cfg.batch, cfg.micro
    work = (bench.conv_role_work if conv else bench.role_work)(cfg, n, m)

    def step_work(name):
        p = bench.role_passes(cfg, m, name, conv)
        return work[name][1] * p if (p and name in work) else None
    return step_work


def test_cell_step_work_closed_forms():
    c = configs.CELL_2048
    sw = step_work_fn(c, False)
    tok = c.batch * c.seq                      # tokens per step
    L, D, F, H, S = c.layers, c.d_model, c.d_ff, c.heads, c.seq
    # forward roles run twice per step (forward phase + re-materialization)
    assert sw("ffn1_fwd") == 2 * L * 2 * tok * D * F
    assert sw("ffn2_fwd") == 2 * L * 2 * tok * F * D
    assert sw("qkv_fwd") == 2 * L * 2 * tok * D * 3 * D
    assert sw("out_fwd") == 2 * L * 2 * tok * D * D
    # backward roles once
    assert sw("ffn1_dgrad") == L * 2 * tok * F * D
    assert sw("qkv_wgrad") == L * 2 * tok * D * 3 * D
    # causal attention: count the kept (query, key) pairs of one head by brute force
    pairs = sum(1 for q in range(S) for k in range(S) if k <= q)
    assert c.causal
    one_product = 2 * pairs * (D // H) * H * c.batch       # QK^T (or PV) over the step's sequences
    assert sw("attn_fwd") == 2 * L * 2 * one_product       # two products, two passes
    assert sw("attn_dq") == L * 4 * one_product            # dP, dV, dQ, dK once
    # the step's whole MFMA work is the sum over the roles that make it up
    total = sum(sw(r) for r in ("qkv_fwd", "out_fwd", "ffn1_fwd", "ffn2_fwd", "qkv_dgrad",
                                "out_dgrad", "ffn1_dgrad", "ffn2_dgrad", "qkv_wgrad",
                                "out_wgrad", "ffn1_wgrad", "ffn2_wgrad", "attn_fwd", "attn_dq"))
    assert bench.step_mfma_flops(c, c.batch, c.micro) == total
    assert abs(total / 1e12 - 107.8) < 0.05


def test_cell_memory_work():
    c = configs.CELL_2048
    sw = step_work_fn(c, False)
    # RMSProp: read w, g, ms (fp32), write w, ms (fp32) and the bf16 copy, once per step
    assert sw("rmsprop") == c.param_count() * (5 * 4 + 2)
    assert c.param_count() == 402866176


def test_conv_step_work_closed_forms():
    c = configs.CONV_CELL
    sw = step_work_fn(c, True)
    px = c.batch * c.height * c.width
    g = 2 * px * c.channels * 9 * c.channels         # one 3x3 convolution over the batch
    # two convolutions per block; forward and re-materialization, then dgrad and wgrad
    assert sw("conv_fwd_implicit") == c.blocks * 2 * 2 * g
    assert sw("conv_dgrad_implicit") == c.blocks * 2 * g
    assert sw("conv_wgrad_implicit") == c.blocks * 2 * g


def test_roofline_kernel_is_the_most_work():
    c = configs.CELL_2048
    sw = step_work_fn(c, False)
    ranked = bench.rank_roles([r for r in CELL_LAUNCHED if sw(r)], sw)
    # ffn1_fwd and ffn2_fwd tie on flops; role order decides, and no backward
    # role (half their work) outranks them
    assert ranked[:3] == ["ffn1_fwd", "ffn2_fwd", "qkv_fwd"]
    assert sw(ranked[0]) == sw(ranked[1]) > sw(ranked[2])
    # the order does not depend on the order the roles come in
    assert bench.rank_roles(list(reversed(ranked)), sw) == ranked
    cc = configs.CONV_CELL
    swc = step_work_fn(cc, True)
    ranked = bench.rank_roles([r for r in CONV_LAUNCHED if swc(r)], swc)
    assert ranked[0] == "conv_fwd_implicit"


def test_traffic_gate(tmp_path, monkeypatch):
    digest = bench.gemm_source_digest()
    good = tmp_path / "good.md"
    good.write_text(f"gemm_source_digest: {digest}\n"
                    "traffic ffn1_fwd: fetch_bytes=123 write_bytes=45\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.measured_traffic("ffn1_fwd") == (123, 45)
    assert bench.measured_traffic("ffn2_fwd") is None
    stale = tmp_path / "stale.md"
    stale.write_text("gemm_source_digest: " + "0" * 64 + "\n"
                     "traffic ffn1_fwd: fetch_bytes=123 write_bytes=45\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic("ffn1_fwd") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("ffn1_fwd") is None


def test_digest_ignores_comments_only(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "micro_pipelined_re_amd", "csrc")
    dst = tmp_path / "micro_pipelined_re_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in bench.GEMM_SOURCES:
        shutil.copy(os.path.join(src, f), dst / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.gemm_source_digest()
    p = dst / "gemm.hip"
    text = p.read_text()
    p.write_text("// a new comment line\n" + text.replace("\n", "  /* c */\n", 1) + "\n\n")
    assert bench.gemm_source_digest() == base
    p.write_text(text + "\nstatic const int gp_digest_probe = 1;\n")
    assert bench.gemm_source_digest() != base


def test_committed_counters_match_sources():
    # the counter summary the bench reads traffic from was taken on these GEMM sources
    assert bench.measured_traffic("ffn1_fwd") is not None


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""

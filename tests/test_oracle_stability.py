"""Pins of the oracle's stability options ("training stability challenges of
deep models" on the review page): logit clipping in front of the attention
softmax, and the feed-forward initialisation scaled down by the depth L.

Logit clipping is pinned to
  * torch float64 autograd on the same layer written with torch's own ops
    (layer_norm, linear, clamp, softmax, gelu), a library implementation of
    clip-then-softmax and of its gradient;
  * central finite differences of the loss, with the threshold placed in a
    gap of the scores so no perturbation crosses the clip's kink;
  * closed forms: a threshold below every score makes every query attend
    uniformly (ctx = mean of the visible values) and blocks every gradient
    into the queries and keys; a threshold above every score changes nothing.
The depth-scaled initialisation is pinned to exact binary scaling for powers
of two, the identity at L = 1, and the drawn matrices' spread.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from micro_pipelined_re_amd import inputs
from micro_pipelined_re_amd.configs import TINY
from oracle import transformer_cell as tc
from tests.test_oracle_transformer import random_layers


def rel(a, b):
    a, b = np.asarray(a, np.float64).ravel(), np.asarray(b, np.float64).ravel()
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def torch_layer(p, x, heads, causal, clip):
    d = x.shape[-1]
    dh = d // heads
    T = lambda a: torch.as_tensor(a)
    h1 = F.layer_norm(x, (d,), T(p["ln1_g"]), T(p["ln1_b"]), 1e-5)
    qkv = F.linear(h1, T(p["w_qkv"]), T(p["b_qkv"]))
    b, s, _ = x.shape
    q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(b, s, heads, dh).transpose(1, 2)
               for i in range(3))
    sc = torch.matmul(q, k.transpose(-1, -2)) / math.sqrt(dh)
    sc = torch.clamp(sc, -clip, clip)
    if causal:
        sc = sc.masked_fill(torch.triu(torch.ones(s, s, dtype=torch.bool), 1), float("-inf"))
    ctx = torch.matmul(torch.softmax(sc, dim=-1), v).transpose(1, 2).reshape(b, s, d)
    x1 = x + F.linear(ctx, T(p["w_o"]), T(p["b_o"]))
    h2 = F.layer_norm(x1, (d,), T(p["ln2_g"]), T(p["ln2_b"]), 1e-5)
    return x1 + F.linear(F.gelu(F.linear(h2, T(p["w_1"]), T(p["b_1"]))), T(p["w_2"]), T(p["b_2"]))


def raw_scores(params, x, heads, causal):
    """|scores| of every layer (unclipped forward), for placing the threshold."""
    out = []
    h = x
    for p in params:
        h, s = tc.layer_forward(p, h, heads, causal)
        d = h.shape[-1]
        q = s["qkv"][..., :d]
        k = s["qkv"][..., d:2 * d]
        b, n, _ = q.shape
        dh = d // heads
        q = q.reshape(b, n, heads, dh).transpose(0, 2, 1, 3)
        k = k.reshape(b, n, heads, dh).transpose(0, 2, 1, 3)
        out.append(np.abs(q @ k.transpose(0, 1, 3, 2)) / math.sqrt(dh))
    return out


def threshold_in_a_gap(scores, lo=0.3, hi=0.7):
    """A threshold clipping between lo and hi of the scores, at the middle of the
    widest gap between consecutive |scores| there; returns (threshold, half gap)."""
    v = np.sort(np.concatenate([s.ravel() for s in scores]))
    i0, i1 = int(lo * v.size), int(hi * v.size)
    gaps = v[i0 + 1:i1] - v[i0:i1 - 1]
    j = int(np.argmax(gaps))
    return 0.5 * (v[i0 + j] + v[i0 + j + 1]), 0.5 * gaps[j]


@pytest.mark.parametrize("causal", [False, True])
def test_clipped_layer_matches_torch_autograd(causal):
    rng = np.random.default_rng(11)
    n, s, d, h, f, L, micro = 4, 6, 16, 2, 32, 2, 2
    params = random_layers(rng, L, d, f, scale=2.0)
    x = rng.standard_normal((n, s, d))
    t = rng.standard_normal((n, s, d))
    clip, _ = threshold_in_a_gap(raw_scores(params, x, h, causal))
    out = tc.cell_step(params, x, t, micro, h, causal, clip=clip)
    xt = torch.tensor(x, requires_grad=True)
    tp = [{k: torch.tensor(v, requires_grad=True) for k, v in p.items()} for p in params]
    y = xt
    for p in tp:
        y = torch_layer(p, y, h, causal, clip)
    loss = ((y - torch.as_tensor(t)) ** 2).sum() / x.size
    loss.backward()
    assert rel(out["y"], y.detach().numpy()) < 1e-12
    assert abs(out["loss"] - loss.item()) < 1e-12 * loss.item()
    assert rel(out["dx"], xt.grad.numpy()) < 1e-10
    for l in range(L):
        for k in inputs.PARAM_NAMES:
            assert rel(out["grads"][l][k], tp[l][k].grad.numpy()) < 1e-10, (l, k)
    # the clip did bite: the unclipped step differs
    plain = tc.cell_step(params, x, t, micro, h, causal)
    assert rel(plain["grads"][0]["w_qkv"], out["grads"][0]["w_qkv"]) > 1e-3


def test_clipped_finite_differences():
    rng = np.random.default_rng(3)
    n, s, d, h, f, L = 2, 4, 8, 2, 16, 2
    params = random_layers(rng, L, d, f, scale=2.0)
    x = rng.standard_normal((n, s, d))
    t = rng.standard_normal((n, s, d))
    clip, half_gap = threshold_in_a_gap(raw_scores(params, x, h, False))
    eps = 1e-6
    assert half_gap > 100 * eps * 10     # no perturbation below reaches the kink
    out = tc.cell_step(params, x, t, 1, h, False, clip=clip)

    def loss():
        y, _ = tc.cell_forward(params, x, h, False, clip=clip)
        return tc.mse_loss(y, t, x.size)[0]

    num = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        v = x[idx]
        x[idx] = v + eps
        lp = loss()
        x[idx] = v - eps
        lm = loss()
        x[idx] = v
        num[idx] = (lp - lm) / (2 * eps)
    assert rel(out["dx"], num) < 1e-6
    for l in range(L):
        w = params[l]["w_qkv"].reshape(-1)
        an = out["grads"][l]["w_qkv"].reshape(-1)
        idxs = rng.choice(w.size, 48, replace=False)
        nums = []
        for i in idxs:
            v = w[i]
            w[i] = v + eps
            lp = loss()
            w[i] = v - eps
            lm = loss()
            w[i] = v
            nums.append((lp - lm) / (2 * eps))
        assert rel(an[idxs], np.array(nums)) < 1e-6, l


@pytest.mark.parametrize("causal", [False, True])
def test_threshold_below_every_score_attends_uniformly(causal):
    """Every score clipped to +-c with c ~ 0: uniform attention over the visible
    keys, and nothing flows back into the queries and keys."""
    rng = np.random.default_rng(4)
    n, s, d, h, f = 3, 5, 8, 2, 16
    params = random_layers(rng, 1, d, f, scale=2.0)
    x = rng.standard_normal((n, s, d))
    t = rng.standard_normal((n, s, d))
    y, saved = tc.cell_forward(params, x, h, causal, keep=True, clip=1e-300)
    sv = saved[0]
    v = sv["qkv"][..., 2 * d:]
    if causal:
        want = np.cumsum(v, axis=1) / np.arange(1, s + 1)[None, :, None]
    else:
        want = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    assert np.allclose(sv["ctx"], want, rtol=1e-13, atol=1e-13)
    out = tc.cell_step(params, x, t, 1, h, causal, clip=1e-300)
    g = out["grads"][0]
    assert not np.any(g["w_qkv"][:2 * d]) and not np.any(g["b_qkv"][:2 * d])
    assert np.any(g["w_qkv"][2 * d:])


def test_threshold_above_every_score_changes_nothing():
    rng = np.random.default_rng(6)
    params = random_layers(rng, 2, 8, 16, scale=2.0)
    x = rng.standard_normal((4, 4, 8))
    t = rng.standard_normal((4, 4, 8))
    a = tc.cell_step(params, x, t, 2, 2, True)
    b = tc.cell_step(params, x, t, 2, 2, True, clip=1e300)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["dx"], b["dx"])
    for ga, gb in zip(a["grads"], b["grads"]):
        for k in ga:
            assert np.array_equal(ga[k], gb[k])


# ---------------------------------------------------------------- depth-scaled FFN init
def test_depth_scaled_init_is_exact_for_powers_of_two_and_identity_at_one():
    params = inputs.cell_params(TINY)
    for L in (1, 8, 128):
        out = tc.depth_scaled_ffn_init(params, L)
        for p, q in zip(params, out):
            for k in p:
                want = np.ldexp(np.asarray(p[k], np.float64), -int(math.log2(L))) \
                    if k in ("w_1", "w_2") else np.asarray(p[k], np.float64)
                assert np.array_equal(q[k], want), (L, k)
    with pytest.raises(ValueError):
        tc.depth_scaled_ffn_init(params, 0)


def test_depth_scaled_init_spread():
    """The drawn FFN matrices (std 0.02) come out with std 0.02 / L."""
    cfg = TINY.with_(d_model=128, d_ff=512, layers=1)
    L = 48
    q = tc.depth_scaled_ffn_init(inputs.cell_params(cfg), L)[0]
    for k in ("w_1", "w_2"):
        sd = float(np.std(q[k]))
        assert abs(sd - 0.02 / L) < 0.02 * (0.02 / L), (k, sd)
    assert float(np.std(q["w_qkv"])) > 0.019

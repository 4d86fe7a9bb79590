"""Test infrastructure: the conv cell's bf16 storage policy applied to the oracle's functions.

Micro-batch BatchNorm makes the gradients of the conv cell unusually
sensitive to the rounding of stored activations: BN2 renders the loss
invariant to the scale of each block's ReLU output, so the true input
gradient of BN1 is the small remainder of a near-cancellation, and a
relative perturbation of 2^-9 in an activation moves it by a few percent.
Every bf16 implementation of the cell inherits this, whatever its kernels.

This module quantifies it.  It replays the oracle's step (oracle.conv_cell,
float64) rounding to bf16 exactly where the bf16 path stores a tensor:
block inputs and outputs, the convolution outputs a and z, the ReLU output
r, the BN input gradients (the convolution backward's GEMM operands) and the
act copy of dx; the loss gradient is float32; everything else is float64.
Tests use it to derive the tolerance of the bf16 path against the float64
oracle from the policy's own deviation on the same inputs.  It does not stand
in for the oracle.
"""
from __future__ import annotations

import numpy as np

from micro_pipelined_re_amd.inputs import round_to_bf16
from oracle import conv_cell as cc


_ROUND = [True]


def bf(a):
    if not _ROUND[0]:
        return np.asarray(a, np.float64)
    return round_to_bf16(np.asarray(a, np.float32)).astype(np.float64)


def _block_forward(p, x, eps):
    a = bf(cc.conv3x3(x, p["w1"]))
    bn1, mu1, var1 = cc.batch_norm(a, p["bn1_g"], p["bn1_b"], eps)
    r = bf(np.maximum(bn1, 0.0))
    z = bf(cc.conv3x3(r, p["w2"]))
    bn2, mu2, var2 = cc.batch_norm(z, p["bn2_g"], p["bn2_b"], eps)
    out = bf(x + bn2)
    return out, dict(x=x, a=a, mu1=mu1, var1=var1, r=r, z=z, mu2=mu2, var2=var2)


def _block_backward(p, s, dout, eps):
    g = {}
    dz, g["bn2_g"], g["bn2_b"] = cc.batch_norm_backward(dout, s["z"], s["mu2"], s["var2"],
                                                         p["bn2_g"], eps)
    dz = bf(dz)
    dr, g["w2"] = cc.conv3x3_backward(dz, s["r"], p["w2"])
    da, g["bn1_g"], g["bn1_b"] = cc.batch_norm_backward(dr * (s["r"] > 0), s["a"], s["mu1"],
                                                         s["var1"], p["bn1_g"], eps)
    da = bf(da)
    dx, g["w1"] = cc.conv3x3_backward(da, s["x"], p["w1"])
    return dout + dx, g


def model_step(params, x, t, micro, eps=cc.BN_EPS, rounding=True):
    """Same outputs as oracle.conv_cell.cell_step (y, loss, dx, grads) under the bf16 policy.

    rounding=False drops every bf16 rounding (the float32 loss gradient stays)."""
    _ROUND[0] = rounding
    try:
        return _model_step(params, x, t, micro, eps)
    finally:
        _ROUND[0] = True


def _model_step(params, x, t, micro, eps):
    params = [{k: np.asarray(v, np.float64) for k, v in p.items()} for p in params]
    x = np.asarray(x, np.float64)
    t = np.asarray(t, np.float64)
    n = x.shape[0]
    b = n // micro
    denom = x.size
    y = np.empty_like(x)
    dx = np.empty_like(x)
    loss, grads = 0.0, None
    for m in range(micro):
        sl = slice(m * b, (m + 1) * b)
        h, saved = x[sl], []
        for p in params:
            h, s = _block_forward(p, h, eps)
            saved.append(s)
        y[sl] = h
        r = h - t[sl]
        loss += float((r * r).sum() / denom)
        d = (2.0 * r / denom).astype(np.float32).astype(np.float64)
        g_m = [None] * len(params)
        for l in reversed(range(len(params))):
            d, g_m[l] = _block_backward(params[l], saved[l], d, eps)
        dx[sl] = bf(d)
        grads = g_m if grads is None else [{k: a[k] + gm[k] for k in a} for a, gm in zip(grads, g_m)]
    return dict(y=y, loss=loss, dx=dx, grads=grads)

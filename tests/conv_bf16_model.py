"""Test infrastructure: where bf16 rounding may go in the conv cell, measured on the oracle.

Micro-batch BatchNorm over residual blocks makes the conv cell's gradients
the small remainder of near-cancellations: BN2 renders the loss invariant to
the scale of each block's ReLU output, so the true input gradient of BN1 is
a small difference of large terms.  This module replays the oracle's step
(oracle.conv_cell, float64) with bf16 rounding (round to nearest even) at a
chosen set of storage points, so tests can measure what each costs:

  forward points   "out" (block outputs, the next block's input), "a", "z"
                   (the convolution outputs), "r" (the ReLU outputs);
  backward points  "dz", "da" (the BatchNorm input gradients, the
                   convolution backward's operands), "dy" (the loss
                   gradient), "dx" (the cell's input gradient).

It does not stand in for the oracle: its only use is to show which storage
policy a bf16 implementation can afford.
"""
from __future__ import annotations

import numpy as np

from micro_pipelined_re_amd.inputs import round_to_bf16
from oracle import conv_cell as cc

FORWARD_POINTS = ("out", "a", "z", "r")
BACKWARD_POINTS = ("dz", "da", "dy", "dx")


def _rounder(points):
    pts = frozenset(points)

    def bf(a, key):
        if key not in pts:
            return np.asarray(a, np.float64)
        return round_to_bf16(np.asarray(a, np.float32)).astype(np.float64)
    return bf


def _block_forward(p, x, eps, bf):
    a = bf(cc.conv3x3(x, p["w1"]), "a")
    bn1, mu1, var1 = cc.batch_norm(a, p["bn1_g"], p["bn1_b"], eps)
    r = bf(np.maximum(bn1, 0.0), "r")
    z = bf(cc.conv3x3(r, p["w2"]), "z")
    bn2, mu2, var2 = cc.batch_norm(z, p["bn2_g"], p["bn2_b"], eps)
    out = bf(x + bn2, "out")
    return out, dict(x=x, a=a, mu1=mu1, var1=var1, r=r, z=z, mu2=mu2, var2=var2)


def _block_backward(p, s, dout, eps, bf):
    g = {}
    dz, g["bn2_g"], g["bn2_b"] = cc.batch_norm_backward(dout, s["z"], s["mu2"], s["var2"],
                                                         p["bn2_g"], eps)
    dz = bf(dz, "dz")
    dr, g["w2"] = cc.conv3x3_backward(dz, s["r"], p["w2"])
    da, g["bn1_g"], g["bn1_b"] = cc.batch_norm_backward(dr * (s["r"] > 0), s["a"], s["mu1"],
                                                         s["var1"], p["bn1_g"], eps)
    da = bf(da, "da")
    dx, g["w1"] = cc.conv3x3_backward(da, s["x"], p["w1"])
    return dout + dx, g


def model_step(params, x, t, micro, points, eps=cc.BN_EPS):
    """The oracle's cell_step (y, loss, dx, grads) with bf16 rounding at `points`."""
    bf = _rounder(points)
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
            h, s = _block_forward(p, h, eps, bf)
            saved.append(s)
        y[sl] = h
        r = h - t[sl]
        loss += float((r * r).sum() / denom)
        d = bf(2.0 * r / denom, "dy")
        g_m = [None] * len(params)
        for l in reversed(range(len(params))):
            d, g_m[l] = _block_backward(params[l], saved[l], d, eps, bf)
        dx[sl] = bf(d, "dx")
        grads = g_m if grads is None else [{k: a[k] + gm[k] for k in a} for a, gm in zip(grads, g_m)]
    return dict(y=y, loss=loss, dx=dx, grads=grads)

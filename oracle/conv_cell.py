"""Oracle for a GPipe cell of convolutional residual blocks with micro-batch
BatchNorm (test infrastructure only).

BatchNorm under GPipe (GPipe technical review page, "GPipe algorithm in
detail / BatchNorm handling"): during training every micro-batch normalises
with its own statistics; moving averages over the whole mini-batch are kept
for evaluation.  The step otherwise follows "pipeline execution flow":
forward phase keeping the cell's boundary output, backward phase
re-materializing each micro-batch, gradients summed over micro-batches, one
RMSProp update.  Unlike LayerNorm, micro-batch BatchNorm makes the result
depend on M (the page's limitations section 4 and BatchNorm passage).

Block (the workload definition; the pages fix none of it):
    a = conv3x3(x, W1);  r = ReLU(BN1(a));  z = conv3x3(r, W2);  out = x + BN2(z)
3x3 convolutions with padding 1, stride 1, no bias; activations NHWC
[B, H, W, C]; weights [C_out, 3, 3, C_in].  BN normalises each channel over
(B, H, W) with the biased variance and epsilon 1e-5.

Moving averages (once per step, after the forward phase; the re-materialized
forward never touches them): the mini-batch mean and biased variance are
pooled from the M equal-size micro-batches' moments,
    mu = mean_m mu_m,   var = mean_m (var_m + mu_m^2) - mu^2,
the variance is made unbiased with n/(n-1), n = N*H*W, and
    running <- momentum * running + (1 - momentum) * stat   (momentum 0.9).

Float64 by default; im2col + numpy matmul for the convolutions.
"""
from __future__ import annotations

import numpy as np

BN_EPS = 1e-5
CONV_NAMES = ("w1", "bn1_g", "bn1_b", "w2", "bn2_g", "bn2_b")


def im2col(x):
    """[B, H, W, C] -> [B*H*W, 9*C]; column (kh*3 + kw)*C + c holds x[h+kh-1, w+kw-1, c] (0 outside)."""
    b, h, w, c = x.shape
    xp = np.pad(x, ((0, 0), (1, 1), (1, 1), (0, 0)))
    cols = [xp[:, kh:kh + h, kw:kw + w, :] for kh in range(3) for kw in range(3)]
    return np.concatenate(cols, axis=-1).reshape(b * h * w, 9 * c)


def col2im(dcol, shape):
    """Adjoint of im2col: [B*H*W, 9*C] -> [B, H, W, C] (sums the nine shifted copies)."""
    b, h, w, c = shape
    d = dcol.reshape(b, h, w, 9, c)
    out = np.zeros((b, h + 2, w + 2, c), dtype=dcol.dtype)
    for kh in range(3):
        for kw in range(3):
            out[:, kh:kh + h, kw:kw + w, :] += d[:, :, :, kh * 3 + kw, :]
    return out[:, 1:h + 1, 1:w + 1, :]


def conv3x3(x, wt):
    b, h, w, c = x.shape
    co = wt.shape[0]
    return (im2col(x) @ wt.reshape(co, 9 * c).T).reshape(b, h, w, co)


def conv3x3_backward(dy, x, wt):
    """Returns (dx, dW) of y = conv3x3(x, W)."""
    b, h, w, c = x.shape
    co = wt.shape[0]
    dy2 = dy.reshape(-1, co)
    dw = (dy2.T @ im2col(x)).reshape(wt.shape)
    dx = col2im(dy2 @ wt.reshape(co, 9 * c), x.shape)
    return dx, dw


def batch_norm(a, gamma, beta, eps=BN_EPS):
    """Training-mode BN over all axes but the last; returns (y, mu, var) with the biased var."""
    c = a.shape[-1]
    rows = a.reshape(-1, c)
    mu = rows.mean(axis=0)
    var = ((rows - mu) ** 2).mean(axis=0)
    y = (a - mu) / np.sqrt(var + eps) * gamma + beta
    return y, mu, var


def batch_norm_backward(dy, a, mu, var, gamma, eps=BN_EPS):
    """Returns (da, dgamma, dbeta) of training-mode BN (statistics of this batch)."""
    c = a.shape[-1]
    n = a.size // c
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = ((a - mu) * rstd).reshape(-1, c)
    g = dy.reshape(-1, c)
    dgamma = (g * xhat).sum(axis=0)
    dbeta = g.sum(axis=0)
    dxhat = g * gamma
    da = rstd * (dxhat - dxhat.sum(axis=0) / n - xhat * (dxhat * xhat).sum(axis=0) / n)
    return da.reshape(a.shape), dgamma, dbeta


def block_forward(p, x, eps=BN_EPS):
    a = conv3x3(x, p["w1"])
    bn1, mu1, var1 = batch_norm(a, p["bn1_g"], p["bn1_b"], eps)
    r = np.maximum(bn1, 0.0)
    z = conv3x3(r, p["w2"])
    bn2, mu2, var2 = batch_norm(z, p["bn2_g"], p["bn2_b"], eps)
    out = x + bn2
    saved = dict(x=x, a=a, mu1=mu1, var1=var1, r=r, z=z, mu2=mu2, var2=var2)
    return out, saved


def block_backward(p, s, dout, eps=BN_EPS):
    g = {}
    dz, g["bn2_g"], g["bn2_b"] = batch_norm_backward(dout, s["z"], s["mu2"], s["var2"], p["bn2_g"], eps)
    dr, g["w2"] = conv3x3_backward(dz, s["r"], p["w2"])
    dbn1 = dr * (s["r"] > 0)
    da, g["bn1_g"], g["bn1_b"] = batch_norm_backward(dbn1, s["a"], s["mu1"], s["var1"], p["bn1_g"], eps)
    dx, g["w1"] = conv3x3_backward(da, s["x"], p["w1"])
    return dout + dx, g


def cell_forward(params, x, eps=BN_EPS, keep=False):
    saved = []
    h = x
    for p in params:
        h, s = block_forward(p, h, eps)
        saved.append(s)
    return h, (saved if keep else [{k: s[k] for k in ("mu1", "var1", "mu2", "var2")} for s in saved])


def cell_step(params, x, t, micro, eps=BN_EPS, remat=True, dtype=np.float64, denom=None):
    """Phases 1 and 2 of one step: returns dict(y, loss, dx, grads, stats) where
    stats[m][block] = (mu1, var1, mu2, var2) of micro-batch m's forward phase."""
    n = x.shape[0]
    if micro < 1 or n % micro:
        raise ValueError("the mini-batch must split into equal micro-batches")
    b = n // micro
    params = [{k: np.asarray(v, dtype) for k, v in p.items()} for p in params]
    x = np.asarray(x, dtype)
    t = np.asarray(t, dtype)
    denom = x.size if denom is None else denom
    y = np.empty_like(x)
    stats, kept = [], []
    for m in range(micro):                       # phase 1: forward, boundary kept
        sl = slice(m * b, (m + 1) * b)
        y[sl], saved = cell_forward(params, x[sl], eps, keep=not remat)
        stats.append([(s["mu1"], s["var1"], s["mu2"], s["var2"]) for s in saved])
        kept.append(saved if not remat else None)
    loss, dx, grads = 0.0, np.empty_like(x), None
    for m in range(micro):                       # phase 2: re-materialize, backward
        sl = slice(m * b, (m + 1) * b)
        if remat:
            y_m, saved = cell_forward(params, x[sl], eps, keep=True)
        else:
            y_m, saved = y[sl], kept[m]
        r = y_m - t[sl]
        loss += float((r * r).sum() / denom)
        d = 2.0 * r / denom
        g_m = [None] * len(params)
        for l in reversed(range(len(params))):
            d, g_m[l] = block_backward(params[l], saved[l], d, eps)
        dx[sl] = d
        if grads is None:
            grads = g_m
        else:
            for acc, gm in zip(grads, g_m):
                for k in acc:
                    acc[k] = acc[k] + gm[k]
    return dict(y=y, loss=loss, dx=dx, grads=grads, stats=stats)


def running_update(running, stats, n_total, momentum):
    """Moving averages after the forward phase.

    running[block] = dict(mean1, var1, mean2, var2); stats as returned by
    cell_step; n_total = N*H*W.  Returns the new running dicts."""
    micro = len(stats)
    out = []
    for l, r in enumerate(running):
        new = {}
        for j, key in ((0, "1"), (2, "2")):
            mus = np.stack([stats[m][l][j] for m in range(micro)])
            vrs = np.stack([stats[m][l][j + 1] for m in range(micro)])
            mu = mus.mean(axis=0)
            var = (vrs + mus ** 2).mean(axis=0) - mu ** 2
            unbiased = var * n_total / (n_total - 1)
            new["mean" + key] = momentum * r["mean" + key] + (1 - momentum) * mu
            new["var" + key] = momentum * r["var" + key] + (1 - momentum) * unbiased
        out.append(new)
    return out

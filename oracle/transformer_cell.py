"""Oracle for one GPipe cell of pre-LN Transformer layers (test infrastructure only).

What one training step of a cell computes, following the GPipe technical
review page (zzz0906.github.io), section "GPipe algorithm in detail /
pipeline execution flow":

  phase 1 (forward): the mini-batch of N sequences is cut into M equal
      micro-batches; each runs forward through the cell and only the cell's
      boundary activation is kept, the layer intermediates are dropped;
  phase 2 (backward): for every micro-batch the cell's forward is run again
      to rebuild the dropped intermediates (re-materialization, preliminaries
      section 5), then backpropagated; the gradients are summed over the
      micro-batches and not applied yet;
  phase 3 (update): one update with the summed gradients, so the step equals
      an ordinary full-mini-batch step (preliminaries section 6, synchronous
      update).

The pages leave the layer open; the layer here is the pre-LN Transformer
layer (LayerNorm, multi-head attention, GeLU FFN) with biases on all four
linears, exact-erf GeLU, no dropout, attention scale 1/sqrt(head_dim), an
optional causal mask, LayerNorm epsilon 1e-5.  The loss is the mean squared
error over all N*S*D outputs of the mini-batch; every micro-batch uses that
global normaliser.  The optimizer is RMSProp (named in preliminaries section
2, ~12 bytes per parameter): ms <- rho*ms + (1-rho)*g^2,
w <- w - lr*g/(sqrt(ms)+eps), ms_0 = 0.

Everything is computed in `dtype` (float64 unless a caller asks otherwise);
matrix products use numpy's matmul, nothing is blocked, fused or reordered.
Weight matrices are [out_features, in_features]: y = x @ W.T + b.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

LN_EPS = 1e-5


# --------------------------------------------------------------------------
# elementary operations
# --------------------------------------------------------------------------

def layer_norm(x, gamma, beta, eps=LN_EPS):
    """LayerNorm over the last axis with the biased variance; returns (y, mu, rstd)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    y = (x - mu) * rstd * gamma + beta
    return y, mu, rstd


def layer_norm_backward(dy, x, mu, rstd, gamma):
    """Gradient of LayerNorm: returns (dx, dgamma, dbeta); sums run over all rows."""
    xhat = (x - mu) * rstd
    dxhat = dy * gamma
    d = x.shape[-1]
    mean_dxhat = dxhat.sum(axis=-1, keepdims=True) / d
    mean_dxhat_xhat = (dxhat * xhat).sum(axis=-1, keepdims=True) / d
    dx = rstd * (dxhat - mean_dxhat - xhat * mean_dxhat_xhat)
    rows = dy.reshape(-1, d)
    dgamma = (rows * xhat.reshape(-1, d)).sum(axis=0)
    dbeta = rows.sum(axis=0)
    return dx, dgamma, dbeta


def gelu(u):
    """GeLU, exact form: u * Phi(u) with Phi the standard normal CDF."""
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def gelu_derivative(u):
    """d/du [u * Phi(u)] = Phi(u) + u * phi(u)."""
    phi = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return 0.5 * (1.0 + erf(u / math.sqrt(2.0))) + u * phi


def clip_logits(s, clip):
    """Logit clipping ("training stability challenges of deep models": the
    activations in front of a softmax are clipped when they exceed a
    threshold): s limited to [-clip, clip]; clip None leaves s as it is."""
    return s if clip is None else np.clip(s, -clip, clip)


def softmax_rows(s, causal, clip=None):
    """Row softmax over the last axis with max subtraction; causal masks j > i.
    With clip, the scores are clipped first (clip_logits)."""
    s = clip_logits(s, clip)
    if causal:
        n = s.shape[-1]
        keep = np.tril(np.ones((s.shape[-2], n), dtype=bool))
        s = np.where(keep, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def softmax_backward(p, dp):
    """dS = P * (dP - rowsum(P * dP))."""
    return p * (dp - (p * dp).sum(axis=-1, keepdims=True))


def linear(x, w, b):
    return x @ w.T + b


# --------------------------------------------------------------------------
# one layer
# --------------------------------------------------------------------------

def _split_heads(a, heads):
    """[B, S, D] -> [B, H, S, dh] (head h is columns h*dh .. (h+1)*dh-1)."""
    b, s, d = a.shape
    return a.reshape(b, s, heads, d // heads).transpose(0, 2, 1, 3)


def _merge_heads(a):
    """[B, H, S, dh] -> [B, S, D]."""
    b, h, s, dh = a.shape
    return a.transpose(0, 2, 1, 3).reshape(b, s, h * dh)


def layer_forward(p, x, heads, causal, ln_eps=LN_EPS, clip=None):
    """One pre-LN layer on x [B, S, D]; returns (x_out, saved intermediates).
    clip: the attention logit-clipping threshold (None: off)."""
    d = x.shape[-1]
    dh = d // heads
    h1, mu1, rstd1 = layer_norm(x, p["ln1_g"], p["ln1_b"], ln_eps)
    qkv = linear(h1, p["w_qkv"], p["b_qkv"])
    q = _split_heads(qkv[..., 0:d], heads)
    k = _split_heads(qkv[..., d:2 * d], heads)
    v = _split_heads(qkv[..., 2 * d:3 * d], heads)
    scores = (q @ k.transpose(0, 1, 3, 2)) / math.sqrt(dh)
    prob = softmax_rows(scores, causal, clip)
    ctx = _merge_heads(prob @ v)
    x1 = x + linear(ctx, p["w_o"], p["b_o"])
    h2, mu2, rstd2 = layer_norm(x1, p["ln2_g"], p["ln2_b"], ln_eps)
    u = linear(h2, p["w_1"], p["b_1"])
    g = gelu(u)
    x_out = x1 + linear(g, p["w_2"], p["b_2"])
    saved = dict(x=x, h1=h1, mu1=mu1, rstd1=rstd1, qkv=qkv, prob=prob, ctx=ctx,
                 x1=x1, h2=h2, mu2=mu2, rstd2=rstd2, u=u, g=g)
    if clip is not None:
        # where the clip is active its output does not move with the score:
        # d clip(s) / ds is 1 for |s| <= clip and 0 beyond
        saved["keep"] = np.abs(scores) <= clip
    return x_out, saved


def layer_backward(p, saved, d_out, heads, causal):
    """Backward of layer_forward; returns (d_in, grads) with grads keyed like p."""
    x, x1 = saved["x"], saved["x1"]
    d = x.shape[-1]
    dh = d // heads
    gr = {}

    def wgrad(dy, a):
        return dy.reshape(-1, dy.shape[-1]).T @ a.reshape(-1, a.shape[-1])

    def colsum(dy):
        return dy.reshape(-1, dy.shape[-1]).sum(axis=0)

    # x_out = x1 + g @ W2.T + b2
    gr["w_2"] = wgrad(d_out, saved["g"])
    gr["b_2"] = colsum(d_out)
    dg = d_out @ p["w_2"]
    du = dg * gelu_derivative(saved["u"])
    # u = h2 @ W1.T + b1
    gr["w_1"] = wgrad(du, saved["h2"])
    gr["b_1"] = colsum(du)
    dh2 = du @ p["w_1"]
    dx1_ln, gr["ln2_g"], gr["ln2_b"] = layer_norm_backward(
        dh2, x1, saved["mu2"], saved["rstd2"], p["ln2_g"])
    dx1 = d_out + dx1_ln
    # x1 = x + ctx @ Wo.T + bo
    gr["w_o"] = wgrad(dx1, saved["ctx"])
    gr["b_o"] = colsum(dx1)
    dctx = _split_heads(dx1 @ p["w_o"], heads)
    qkv, prob = saved["qkv"], saved["prob"]
    q = _split_heads(qkv[..., 0:d], heads)
    k = _split_heads(qkv[..., d:2 * d], heads)
    v = _split_heads(qkv[..., 2 * d:3 * d], heads)
    dprob = dctx @ v.transpose(0, 1, 3, 2)
    dv = prob.transpose(0, 1, 3, 2) @ dctx
    dscores = softmax_backward(prob, dprob) / math.sqrt(dh)
    if "keep" in saved:
        dscores = dscores * saved["keep"]
    dq = dscores @ k
    dk = dscores.transpose(0, 1, 3, 2) @ q
    dqkv = np.concatenate([_merge_heads(dq), _merge_heads(dk), _merge_heads(dv)], axis=-1)
    gr["w_qkv"] = wgrad(dqkv, saved["h1"])
    gr["b_qkv"] = colsum(dqkv)
    dh1 = dqkv @ p["w_qkv"]
    dx_ln, gr["ln1_g"], gr["ln1_b"] = layer_norm_backward(
        dh1, x, saved["mu1"], saved["rstd1"], p["ln1_g"])
    return dx1 + dx_ln, gr


# --------------------------------------------------------------------------
# the cell, the loss and the step
# --------------------------------------------------------------------------

def cell_forward(params, x, heads, causal, ln_eps=LN_EPS, keep=False, clip=None):
    """Run every layer of the cell; returns (y, saved list or None)."""
    saved = [] if keep else None
    h = x
    for p in params:
        h, s = layer_forward(p, h, heads, causal, ln_eps, clip)
        if keep:
            saved.append(s)
    return h, saved


def cell_backward(params, saved, dy, heads, causal):
    grads = [None] * len(params)
    d = dy
    for l in reversed(range(len(params))):
        d, grads[l] = layer_backward(params[l], saved[l], d, heads, causal)
    return d, grads


def mse_loss(y, t, denom):
    """Sum of squared errors divided by denom (the mini-batch's N*S*D) and its gradient."""
    r = y - t
    return float((r * r).sum() / denom), 2.0 * r / denom


def cast_params(params, dtype):
    return [{k: np.asarray(v, dtype=dtype) for k, v in p.items()} for p in params]


def cell_step(params, x, t, micro, heads, causal, ln_eps=LN_EPS, remat=True,
              dtype=np.float64, record=False, denom=None, clip=None):
    """One GPipe training step of the cell without the update (phases 1 and 2).

    x, t: [N, S, D].  micro: M, must divide N.  remat=True drops the layer
    intermediates in the forward phase and rebuilds them per micro-batch in
    the backward phase; remat=False keeps every micro-batch's intermediates.
    Micro-batches are processed in order m = 0 .. M-1 in both phases.
    denom is the loss normaliser, N*S*D of x unless given (a caller taking
    some sequences of a larger mini-batch passes that mini-batch's N*S*D).
    clip is the attention logit-clipping threshold (None: off).
    Returns dict(y, loss, dx, grads) plus, if record, the forward phase's and
    the backward phase's intermediates for each micro-batch.
    """
    n = x.shape[0]
    if micro < 1 or n % micro:
        raise ValueError("the mini-batch must split into equal micro-batches")
    b = n // micro
    params = cast_params(params, dtype)
    x = np.asarray(x, dtype=dtype)
    t = np.asarray(t, dtype=dtype)
    denom = x.size if denom is None else denom
    y = np.empty_like(x)
    kept = []
    # phase 1: forward, keeping the boundary output (and, without remat, everything)
    for m in range(micro):
        sl = slice(m * b, (m + 1) * b)
        y[sl], s = cell_forward(params, x[sl], heads, causal, ln_eps,
                                keep=(not remat) or record, clip=clip)
        kept.append(s)
    # phase 2: backward, re-materializing each micro-batch's intermediates
    loss = 0.0
    dx = np.empty_like(x)
    grads = None
    rebuilt = []
    for m in range(micro):
        sl = slice(m * b, (m + 1) * b)
        if remat:
            y_m, saved = cell_forward(params, x[sl], heads, causal, ln_eps, keep=True, clip=clip)
            if record:
                rebuilt.append((y_m, saved))
        else:
            y_m, saved = y[sl], kept[m]
        l_m, dy = mse_loss(y_m, t[sl], denom)
        loss += l_m
        dx[sl], g_m = cell_backward(params, saved, dy, heads, causal)
        if grads is None:
            grads = g_m
        else:
            for acc, gm in zip(grads, g_m):
                for k in acc:
                    acc[k] = acc[k] + gm[k]
    out = dict(y=y, loss=loss, dx=dx, grads=grads)
    if record:
        out["forward_saved"] = kept
        out["rebuilt"] = rebuilt
    return out


def rmsprop(w, g, ms, lr, decay, eps):
    """One RMSProp update: returns (w_new, ms_new)."""
    ms_new = decay * ms + (1.0 - decay) * g * g
    w_new = w - lr * g / (np.sqrt(ms_new) + eps)
    return w_new, ms_new


def train_step(params, x, t, micro, heads, causal, lr, decay, eps, ms=None,
               ln_eps=LN_EPS, remat=True, dtype=np.float64, clip=None):
    """Phases 1-3: the step plus one synchronous RMSProp update of every tensor."""
    out = cell_step(params, x, t, micro, heads, causal, ln_eps, remat, dtype, clip=clip)
    p64 = cast_params(params, dtype)
    if ms is None:
        ms = [{k: np.zeros_like(v) for k, v in p.items()} for p in p64]
    new_w, new_ms = [], []
    for p, g, s in zip(p64, out["grads"], ms):
        w_l, m_l = {}, {}
        for k in p:
            w_l[k], m_l[k] = rmsprop(p[k], g[k], np.asarray(s[k], dtype), lr, decay, eps)
        new_w.append(w_l)
        new_ms.append(m_l)
    out["w_new"] = new_w
    out["ms_new"] = new_ms
    return out


def depth_scaled_ffn_init(params, total_layers, dtype=np.float64):
    """Scaled initialisation ("training stability challenges of deep models":
    the feed-forward layers' initialisation is scaled down by the number of
    layers L): every layer's FFN matrices w_1 and w_2 divided by L, the
    stack's total depth (not the cell's L/K); everything else unchanged."""
    if total_layers < 1:
        raise ValueError("total_layers must be positive")
    out = []
    for p in params:
        q = {k: np.asarray(v, dtype=dtype) for k, v in p.items()}
        for k in ("w_1", "w_2"):
            q[k] = q[k] / dtype(total_layers)
        out.append(q)
    return out

"""Plain float64 NumPy oracle of the BACKWARD of the Single-Pass mHC step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages give the forward step only; its gradient is derived here from the
forward's definitions ("DeepSeek V4.1 · Stream weights for the feed-forward",
"All 5 steps" and the Code excerpts; "DeepSeek V4.1 · MoE RMSNorm", formula and
Code) by the chain rule, one forward operation at a time, in reverse order.
Readings:

* The casts back to the stream dtype (``type_as`` in ``hc_post``, the casts in
  ``hc_pre`` and ``RMSNorm``) pass gradients through unchanged, as automatic
  differentiation treats a dtype conversion; every saved forward value used
  by the gradient (new streams, h) is the ROUNDED one the forward produced.
* The gradient of the mixes output (``mix_out``) is not an input: the mixes
  are an internal value of ``hc_mixes``.
* Upstream gradients: of the new streams (dX'), of y (dy) and of the three
  new coefficient sets (d pre', d post', d comb'). Outputs: gradients of every
  step input (X, F, pre_in, post_in, comb_in) and parameter (W, base, scale,
  gamma).
"""

from __future__ import annotations

import numpy as np

from .mhc_oracle import hc_post, hc_pre, sigmoid


def _colnorm(c, eps):
    s = c.sum(axis=1, keepdims=True) + eps        # [t, 1, k]
    return c / s, s


def _rownorm(c, eps):
    s = c.sum(axis=2, keepdims=True) + eps        # [t, j, 1]
    return c / s, s


def split_sinkhorn_backward(m, scale, base, iters, hc_eps, n, d_pre, d_post, d_comb):
    """Gradient of (pre, post, comb) = split_sinkhorn(m, ...) with respect to
    the pre-activations a_i = scale[grp(i)] * m_i + base_i of the (2+n)n
    slots ([SW] Code, the split/Sinkhorn kernel: pre = sigmoid(a) + eps,
    post = 2 sigmoid(a), comb = Sinkhorn(softmax_rows(a) + eps)).

    Forward intermediates are recomputed and kept; the reverse pass undoes
    one normalisation at a time. For Y = X / (sum + eps) along an axis,
    dX = (dY - sum_axis(dY * Y)) / (sum + eps); for P = softmax(L) along rows,
    dL = P * (dP - sum_row(dP * P)).

    Returns g [T, (2+n)n].
    """
    m = np.asarray(m, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    base = np.asarray(base, dtype=np.float64)
    t = m.shape[0]
    a = np.empty_like(m)
    a[:, :n] = scale[0] * m[:, :n] + base[:n]
    a[:, n:2 * n] = scale[1] * m[:, n:2 * n] + base[n:2 * n]
    a[:, 2 * n:] = scale[2] * m[:, 2 * n:] + base[2 * n:]
    g = np.zeros_like(m)

    sp = sigmoid(a[:, :n])
    g[:, :n] = np.asarray(d_pre, dtype=np.float64) * sp * (1.0 - sp)
    sq = sigmoid(a[:, n:2 * n])
    g[:, n:2 * n] = np.asarray(d_post, dtype=np.float64) * 2.0 * sq * (1.0 - sq)

    # forward of the comb, keeping every normalised matrix and its divisors
    logits = a[:, 2 * n:].reshape(t, n, n)
    e = np.exp(logits - logits.max(axis=2, keepdims=True))
    p = e / e.sum(axis=2, keepdims=True)
    steps = []                       # (kind, output, divisor)
    c, s = _colnorm(p + hc_eps, hc_eps)
    steps.append(("col", c, s))
    for _ in range(iters - 1):
        c, s = _rownorm(c, hc_eps)
        steps.append(("row", c, s))
        c, s = _colnorm(c, hc_eps)
        steps.append(("col", c, s))

    dc = np.asarray(d_comb, dtype=np.float64).reshape(t, n, n).copy()
    for kind, y, s in reversed(steps):
        axis = 1 if kind == "col" else 2
        dc = (dc - (dc * y).sum(axis=axis, keepdims=True)) / s
    # dc is now the gradient of softmax + eps, i.e. of p
    dl = p * (dc - (dc * p).sum(axis=2, keepdims=True))
    g[:, 2 * n:] = dl.reshape(t, n * n)
    return g


def fused_step_backward(xs, f, pre_in, post_in, comb_in, w_mix, base, scale, gamma, d_xprime,
                        d_y, d_pre, d_post, d_comb, iters: int = 20, norm_eps: float = 1e-6,
                        hc_eps: float = 1e-6, dtype: str = "bf16", xprime=None):
    """Gradients of one fused step (``mhc_oracle.fused_step``) with respect to
    all its inputs and parameters.

    Forward, per token, with S the rounding to the stream dtype:
      X'_k = S(A_k), A_k = sum_j C[j,k] X_j + u_k F          (hc_post)
      r = (mean(X'^2) + norm_eps)^-1/2, z = W flatten(X'), m = r z   (hc_mixes)
      (pre', post', comb') = split_sinkhorn(m)
      h = S(sum_k p_k X'_k)                                  (hc_pre)
      y = S(gamma * h * rho), rho = (mean(h^2) + norm_eps)^-1/2   (RMSNorm)
    Reverse, with the casts passing gradients through:
      g = d a (split/Sinkhorn backward); dm = scale_grp * g; d base = sum_t g;
      d scale_grp = sum_t sum_{i in grp} g_i m_i
      dz = r dm; dr = dm . z; dW = sum_t dz flatten(X')^T
      d flatten(X') (mixes) = W^T dz - dr r^3 flatten(X') / (n d)
      d gamma = sum_t dy * h * rho; S = sum_f dy gamma h
      dh = rho gamma dy - rho^3 S h / d; d pre_in_k = sum_f dh X'_k
      dA_k = dX'_k + (mixes part)_k + p_k dh
      dX_j = sum_k C[j,k] dA_k; dF = sum_k u_k dA_k
      d comb_in[j,k] = sum_f X_j dA_k; d post_in_k = sum_f F dA_k

    Shapes as ``fused_step``; upstream d_xprime [T,n,d], d_y [T,d], d_pre,
    d_post [T,n], d_comb [T,n,n]. ``xprime``: the new streams the forward
    stored, if given (a backward receives the forward's saved output; any
    correct rounding of it is a valid forward); otherwise recomputed. Returns
    a dict of float64 arrays (d_x and d_f unrounded) with the intermediate
    gradients da (of the new streams), dx_mix and dh.
    """
    xs = np.asarray(xs, dtype=np.float64)
    f = np.asarray(f, dtype=np.float64)
    pre_in = np.asarray(pre_in, dtype=np.float64)
    post_in = np.asarray(post_in, dtype=np.float64)
    comb_in = np.asarray(comb_in, dtype=np.float64)
    w = np.asarray(w_mix, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    d_xprime = np.asarray(d_xprime, dtype=np.float64)
    d_y = np.asarray(d_y, dtype=np.float64)
    t, n, d = xs.shape

    # forward values the gradient uses
    if xprime is None:
        xprime = hc_post(xs, f, post_in, comb_in, dtype)
    xprime = np.asarray(xprime, dtype=np.float64)
    x = xprime.reshape(t, n * d)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + norm_eps)
    z = x @ w.T
    m = z * r[:, None]
    h = hc_pre(xprime, pre_in, dtype)
    rho = 1.0 / np.sqrt(np.mean(h * h, axis=1) + norm_eps)

    # split / Sinkhorn
    g = split_sinkhorn_backward(m, scale, base, iters, hc_eps, n, d_pre, d_post, d_comb)
    s_slot = np.concatenate([np.full(n, scale[0]), np.full(n, scale[1]), np.full(n * n, scale[2])])
    dm = g * s_slot
    d_base = g.sum(axis=0)
    gm = g * m
    d_scale = np.array([gm[:, :n].sum(), gm[:, n:2 * n].sum(), gm[:, 2 * n:].sum()])

    # m = r * (W x)
    dz = dm * r[:, None]
    dr = (dm * z).sum(axis=1)
    d_w = dz.T @ x
    dx_mix = dz @ w - (dr * r ** 3 / (n * d))[:, None] * x

    # y = gamma * h * rho
    d_gamma = (d_y * h * rho[:, None]).sum(axis=0)
    dyg = d_y * gamma[None, :]
    s_sum = (dyg * h).sum(axis=1)
    dh = rho[:, None] * dyg - (rho ** 3 * s_sum / d)[:, None] * h

    # h = sum_k p_k X'_k
    d_pre_in = np.einsum("tf,tkf->tk", dh, xprime)
    da = d_xprime + dx_mix.reshape(t, n, d) + pre_in[:, :, None] * dh[:, None, :]

    # A_k = sum_j C[j,k] X_j + u_k F
    d_x = np.einsum("tjk,tkf->tjf", comb_in, da)
    d_f = np.einsum("tk,tkf->tf", post_in, da)
    d_comb_in = np.einsum("tjf,tkf->tjk", xs, da)
    d_post_in = np.einsum("tf,tkf->tk", f, da)

    return {"d_x": d_x, "d_f": d_f, "d_pre_in": d_pre_in, "d_post_in": d_post_in,
            "d_comb_in": d_comb_in, "d_w_mix": d_w, "d_base": d_base, "d_scale": d_scale,
            "d_gamma": d_gamma, "m": m, "r": r, "rho": rho, "s": s_sum, "g": g,
            "xprime": xprime, "h": h, "da": da, "dx_mix": dx_mix, "dh": dh}

"""Pins for the backward oracle (oracle/mhc_backward.py).

The pages define the forward step only, so the gradient is pinned against
the forward itself, never against its own formulas:

* central finite differences of the forward oracle evaluated without
  rounding (stream dtype "f64"), along random directions in every input and
  parameter, for n = 2, 4, 8 and several Sinkhorn round counts;
* every entry of the small coefficient and parameter tensors by finite
  differences one at a time;
* automatic differentiation (torch, float64) of an independent transcription
  of the forward written here from the pages' code excerpts, with the casts
  to bf16 as straight-through roundings (forward rounds, backward passes the
  gradient): all gradients at once, rounding included.
"""

import numpy as np
import pytest
import torch

from oracle import fused_step
from oracle.mhc_backward import fused_step_backward, split_sinkhorn_backward
from oracle import split_sinkhorn


def _case(rng, t, n, d, logit_scale=1.0):
    nm = (2 + n) * n
    return dict(
        xs=rng.standard_normal((t, n, d)),
        f=rng.standard_normal((t, d)),
        pre_in=rng.uniform(0.2, 1.0, (t, n)),
        post_in=rng.uniform(0.2, 2.0, (t, n)),
        comb_in=rng.dirichlet(np.ones(n), size=(t, n)),
        w_mix=rng.normal(0, 0.3 * logit_scale / np.sqrt(n * d), (nm, n * d)),
        base=rng.normal(0, 0.1, nm),
        scale=rng.uniform(0.5, 2.0, 3),
        gamma=1 + rng.normal(0, 0.05, d),
    )


def _upstream(rng, t, n, d):
    return dict(d_xprime=rng.standard_normal((t, n, d)), d_y=rng.standard_normal((t, d)),
                d_pre=rng.standard_normal((t, n)), d_post=rng.standard_normal((t, n)),
                d_comb=rng.standard_normal((t, n, n)))


INPUTS = ("xs", "f", "pre_in", "post_in", "comb_in", "w_mix", "base", "scale", "gamma")
GRAD_OF = {"xs": "d_x", "f": "d_f", "pre_in": "d_pre_in", "post_in": "d_post_in",
           "comb_in": "d_comb_in", "w_mix": "d_w_mix", "base": "d_base", "scale": "d_scale",
           "gamma": "d_gamma"}


def _loss(c, up, iters, dtype="f64"):
    o = fused_step(c["xs"], c["f"], c["pre_in"], c["post_in"], c["comb_in"], c["w_mix"],
                   c["base"], c["scale"], c["gamma"], iters, 1e-6, 1e-6, dtype)
    return ((up["d_xprime"] * o["xprime"]).sum() + (up["d_y"] * o["y"]).sum()
            + (up["d_pre"] * o["pre"]).sum() + (up["d_post"] * o["post"]).sum()
            + (up["d_comb"] * o["comb"]).sum())


def _grads(c, up, iters, dtype="f64"):
    return fused_step_backward(c["xs"], c["f"], c["pre_in"], c["post_in"], c["comb_in"],
                               c["w_mix"], c["base"], c["scale"], c["gamma"], up["d_xprime"],
                               up["d_y"], up["d_pre"], up["d_post"], up["d_comb"], iters, 1e-6,
                               1e-6, dtype)


@pytest.mark.parametrize("n,d,iters", [(2, 2, 1), (2, 8, 20), (4, 2, 3), (4, 8, 20), (8, 2, 5)])
def test_directional_finite_differences(n, d, iters):
    rng = np.random.default_rng(1000 + 10 * n + d + iters)
    t = 3
    c, up = _case(rng, t, n, d), _upstream(rng, t, n, d)
    g = _grads(c, up, iters)
    eps = 1e-6
    for name in INPUTS:
        for trial in range(2):
            v = rng.standard_normal(np.shape(c[name]))
            cp, cm = dict(c), dict(c)
            cp[name] = c[name] + eps * v
            cm[name] = c[name] - eps * v
            fd = (_loss(cp, up, iters) - _loss(cm, up, iters)) / (2 * eps)
            an = (g[GRAD_OF[name]] * v).sum()
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, trial, fd, an)


@pytest.mark.parametrize("name", ["comb_in", "post_in", "pre_in", "base", "scale"])
def test_entrywise_finite_differences(name):
    rng = np.random.default_rng(1100)
    n, d, t, iters = 2, 4, 2, 20
    c, up = _case(rng, t, n, d, logit_scale=3.0), _upstream(rng, t, n, d)
    g = _grads(c, up, iters)[GRAD_OF[name]]
    eps = 1e-6
    flat = np.asarray(c[name], dtype=np.float64).ravel()
    for i in range(flat.size):
        cp, cm = dict(c), dict(c)
        vp, vm = flat.copy(), flat.copy()
        vp[i] += eps
        vm[i] -= eps
        cp[name] = vp.reshape(np.shape(c[name]))
        cm[name] = vm.reshape(np.shape(c[name]))
        fd = (_loss(cp, up, iters) - _loss(cm, up, iters)) / (2 * eps)
        assert abs(fd - g.ravel()[i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, g.ravel()[i])


def test_sinkhorn_backward_finite_differences_strong_logits():
    """Sharp logits (scale 5) and many rounds: the unrolled normalisations."""
    rng = np.random.default_rng(1200)
    n, t = 4, 5
    nm = (2 + n) * n
    m = rng.normal(0, 3.0, (t, nm))
    scale, base = np.array([1.0, 1.5, 5.0]), rng.normal(0, 0.1, nm)
    dp, du, dc = rng.standard_normal((t, n)), rng.standard_normal((t, n)), rng.standard_normal((t, n, n))
    for iters in (1, 2, 20, 60):
        g = split_sinkhorn_backward(m, scale, base, iters, 1e-6, n, dp, du, dc)
        s_slot = np.concatenate([np.full(n, scale[0]), np.full(n, scale[1]), np.full(n * n, scale[2])])
        v = rng.standard_normal(m.shape)
        eps = 1e-6

        def loss(mm):
            p, u, cc = split_sinkhorn(mm, scale, base, iters, 1e-6, n)
            return (dp * p).sum() + (du * u).sum() + (dc * cc).sum()

        fd = (loss(m + eps * v) - loss(m - eps * v)) / (2 * eps)
        an = (g * s_slot * v).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (iters, fd, an)


# ---- automatic differentiation of an independent transcription --------------------------

def _torch_forward(c, iters, norm_eps, hc_eps, bf16):
    """The step written from the pages' code excerpts in torch float64; the
    casts to the stream dtype round with torch's own bf16 conversion in the
    forward and pass the gradient unchanged."""
    def cast(v):
        if not bf16:
            return v
        return v + (v.to(torch.bfloat16).to(torch.float64) - v).detach()

    xs, f, pre, post, comb = c["xs"], c["f"], c["pre_in"], c["post_in"], c["comb_in"]
    w, base, scale, gamma = c["w_mix"], c["base"], c["scale"], c["gamma"]
    t, n, d = xs.shape
    # hc_post: (comb.unsqueeze(-1) * residual.unsqueeze(-2)).sum(dim=-3) + post * x
    xp = cast((comb.unsqueeze(-1) * xs.unsqueeze(-2)).sum(dim=1) + post.unsqueeze(-1) * f.unsqueeze(1))
    flat = xp.reshape(t, n * d)
    rs = torch.rsqrt(flat.square().mean(-1, keepdim=True) + norm_eps)
    mixes = (flat @ w.T) * rs
    pre_n = torch.sigmoid(mixes[:, :n] * scale[0] + base[:n]) + hc_eps
    post_n = 2 * torch.sigmoid(mixes[:, n:2 * n] * scale[1] + base[n:2 * n])
    cm = (mixes[:, 2 * n:] * scale[2] + base[2 * n:]).view(t, n, n)
    cm = cm.softmax(-1) + hc_eps
    cm = cm / (cm.sum(-2, keepdim=True) + hc_eps)
    for _ in range(iters - 1):
        cm = cm / (cm.sum(-1, keepdim=True) + hc_eps)
        cm = cm / (cm.sum(-2, keepdim=True) + hc_eps)
    h = cast((pre.unsqueeze(-1) * xp).sum(dim=1))
    y = cast(gamma * (h * torch.rsqrt(h.square().mean(-1, keepdim=True) + norm_eps)))
    return xp, y, pre_n, post_n, cm


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("n,d", [(2, 16), (4, 32), (8, 8)])
def test_matches_autograd_of_independent_forward(n, d, bf16):
    rng = np.random.default_rng(1300 + n + d + bf16)
    t, iters = 4, 20
    c, up = _case(rng, t, n, d, logit_scale=2.0), _upstream(rng, t, n, d)
    if bf16:
        # inputs already representable in bf16, as the streams are
        for k in ("xs", "f"):
            c[k] = torch.tensor(c[k]).to(torch.bfloat16).double().numpy()
    g = _grads(c, up, iters, "bf16" if bf16 else "f64")
    tc = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True) for k, v in c.items()}
    outs = _torch_forward(tc, iters, 1e-6, 1e-6, bf16)
    ups = [up["d_xprime"], up["d_y"], up["d_pre"], up["d_post"], up["d_comb"]]
    loss = sum((o * torch.tensor(u)).sum() for o, u in zip(outs, ups))
    loss.backward()
    for name in INPUTS:
        want = tc[name].grad.numpy()
        np.testing.assert_allclose(g[GRAD_OF[name]], want, rtol=1e-9, atol=1e-11,
                                   err_msg=name)

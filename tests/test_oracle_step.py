"""Pins for the oracle's mixes, hc_post, hc_pre, RMSNorm and the whole step:
special cases with known answers, library routines (torch's rms_norm), exact
power-of-two invariances, the pages' parameter and traffic counts, and an
mpmath brute force at tiny widths written as plain loops over the pages'
definitions."""

import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import (fused_step, hc_post, hc_pre, mixes, parameter_count, rmsnorm,
                    round_bf16, round_to)
from tests.conftest import load_golden

N = 4


def _bf16_values(rng, shape, scale=1.0):
    return round_bf16(rng.standard_normal(shape) * scale)


def _inputs(rng, t, d, dtype="bf16", n=N):
    xs = rng.standard_normal((t, n, d))
    f = rng.standard_normal((t, d))
    xs, f = round_to(xs, dtype), round_to(f, dtype)
    pre = rng.uniform(0.1, 1.0, (t, n))
    post = rng.uniform(0.1, 2.0, (t, n))
    comb = rng.dirichlet(np.ones(n), size=(t, n))
    w = rng.normal(0, 0.02, ((2 + n) * n, n * d))
    base = rng.normal(0, 0.1, (2 + n) * n)
    scale = rng.uniform(0.5, 2, 3)
    gamma = 1 + rng.normal(0, 0.05, d)
    return xs, f, pre, post, comb, w, base, scale, gamma


# ---- counts the pages print ------------------------------------------------------------

def test_parameter_count_matches_page_table():
    g = load_golden("parameter_count.txt")
    got = parameter_count(4, 5120)
    for key in ("projection", "reading", "writing", "combination", "total"):
        assert got[key] == g[key], key
    assert len(np.ones(5120)) == g["rmsnorm_gain"]    # gain has one entry per feature


def test_traffic_counts():
    g = load_golden("traffic_per_token.txt")
    n, d = 4, 5120
    # three kernels + pre-norm: hc_post reads n*d + d, writes n*d; hc_mixes reads
    # n*d; hc_pre reads n*d, writes d; the norm reads d, writes d
    three = (n * d + d + n * d) + n * d + (n * d + d) + (d + d)
    fused = (n * d + d) + (n * d + d)     # read X and F, write X' and y
    assert three == g["three_kernel_elems"]
    assert fused == g["fused_elems"]
    assert three == g["ratio"] * fused


# ---- hc_post ---------------------------------------------------------------------------

def test_hc_post_identity_comb_is_exact():
    rng = np.random.default_rng(0)
    xs = _bf16_values(rng, (8, N, 64))
    f = _bf16_values(rng, (8, 64))
    out = hc_post(xs, f, np.zeros((8, N)), np.broadcast_to(np.eye(N), (8, N, N)), "bf16")
    np.testing.assert_array_equal(out, xs)


def test_hc_post_permutation_pins_orientation():
    """comb[j, pi(j)] = 1 routes residual stream j into new stream pi(j)."""
    rng = np.random.default_rng(1)
    xs = _bf16_values(rng, (3, N, 32))
    pi = [2, 0, 3, 1]
    comb = np.zeros((3, N, N))
    for j in range(N):
        comb[:, j, pi[j]] = 1.0
    out = hc_post(xs, np.zeros((3, 32)), np.zeros((3, N)), comb, "bf16")
    for j in range(N):
        np.testing.assert_array_equal(out[:, pi[j]], xs[:, j])


def test_hc_post_write_weight_places_f():
    rng = np.random.default_rng(2)
    f = rng.standard_normal((2, 48))
    for k in range(N):
        post = np.zeros((2, N))
        post[:, k] = 1.0
        out = hc_post(np.zeros((2, N, 48)), f, post, np.zeros((2, N, N)), "bf16")
        np.testing.assert_array_equal(out[:, k], round_bf16(f))
        assert not np.any(np.delete(out, k, axis=1))


def test_hc_post_uniform_comb_gives_equal_streams():
    rng = np.random.default_rng(3)
    xs = _bf16_values(rng, (4, N, 40))
    out = hc_post(xs, np.zeros((4, 40)), np.zeros((4, N)), np.full((4, N, N), 0.25), "bf16")
    for k in range(1, N):
        np.testing.assert_array_equal(out[:, k], out[:, 0])
    np.testing.assert_array_equal(out[:, 0], round_bf16(xs.sum(axis=1) / 4))


# ---- hc_pre and RMSNorm ----------------------------------------------------------------

def test_hc_pre_unit_weights_select_a_stream():
    rng = np.random.default_rng(4)
    xs = _bf16_values(rng, (5, N, 24))
    for k in range(N):
        p = np.zeros((5, N))
        p[:, k] = 1.0
        np.testing.assert_array_equal(hc_pre(xs, p, "bf16"), xs[:, k])


def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(5)
    h = _bf16_values(rng, (16, 5120))
    gamma = 1 + rng.normal(0, 0.05, 5120)
    for eps in (1e-6, 1e-20):
        want = torch.nn.functional.rms_norm(torch.from_numpy(h), (5120,),
                                            weight=torch.from_numpy(gamma), eps=eps).numpy()
        np.testing.assert_array_equal(rmsnorm(h, gamma, eps, "bf16"), round_bf16(want))


def test_rmsnorm_constant_row():
    for c in (0.75, -3.0, 1e-4):
        h = np.full((1, 256), c)
        gamma = np.linspace(0.5, 1.5, 256)
        y = rmsnorm(h, gamma, 1e-6, "f32")
        want = round_to(gamma * math.copysign(1.0, c) / math.sqrt(1 + 1e-6 / c ** 2), "f32")
        np.testing.assert_array_equal(y[0], want)


# ---- mixes -----------------------------------------------------------------------------

def test_mixes_unit_rows_select_flattened_entries():
    """W row j = e_c gives m_j = x_c / rms: pins the flatten order k*d + f."""
    rng = np.random.default_rng(6)
    d = 16
    xs = _bf16_values(rng, (3, N, d))
    cols = rng.choice(N * d, 24, replace=False)
    w = np.zeros((24, N * d))
    w[np.arange(24), cols] = 1.0
    m, *_ = mixes(xs, w, np.zeros(24), [1, 1, 1], norm_eps=0.0)
    for t in range(3):
        rms = math.sqrt(float(np.mean(xs[t] ** 2)))
        for j, c in enumerate(cols):
            k, f = divmod(int(c), d)
            assert m[t, j] == pytest.approx(xs[t, k, f] / rms, rel=1e-14)


def test_mixes_scale_invariance():
    rng = np.random.default_rng(7)
    xs = _bf16_values(rng, (8, N, 32))
    w = rng.normal(0, 0.02, (24, N * 32))
    m1, p1, u1, c1 = mixes(xs, w, np.zeros(24), [1, 1, 1], norm_eps=0.0)
    m2, p2, u2, c2 = mixes(xs * 2.0 ** 9, w, np.zeros(24), [1, 1, 1], norm_eps=0.0)
    np.testing.assert_allclose(m2, m1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(c2, c1, rtol=1e-12)


# ---- whole step: power-of-two scaling ------------------------------------------------

def test_step_power_of_two_scaling():
    rng = np.random.default_rng(8)
    xs, f, pre, post, comb, w, base, scale, gamma = _inputs(rng, 6, 64)
    a = fused_step(xs, f, pre, post, comb, w, base, scale, gamma, norm_eps=0.0)
    b = fused_step(xs * 2.0 ** 6, f * 2.0 ** 6, pre, post, comb, w, base, scale, gamma,
                   norm_eps=0.0)
    np.testing.assert_array_equal(b["xprime"], a["xprime"] * 2.0 ** 6)
    np.testing.assert_array_equal(b["h"], a["h"] * 2.0 ** 6)
    np.testing.assert_allclose(b["m"], a["m"], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(b["y"], a["y"])


# ---- brute force at tiny widths (mpmath, 60 digits, plain loops) ----------------------

def _mp_round(v, bits):
    with mpmath.workprec(bits):
        return +v


def _brute_step(xs, f, pre, post, comb, w, base, scale, gamma, iters, norm_eps, hc_eps, bits):
    """The step for ONE token written as loops over the pages' definitions."""
    mp = mpmath.mpf
    n, d = xs.shape
    # hc_post: new stream k takes comb[j][k] of residual stream j, plus post[k] * F
    xp = [[None] * d for _ in range(n)]
    for k in range(n):
        for ff in range(d):
            acc = mp(0)
            for j in range(n):
                acc += mp(comb[j][k]) * mp(xs[j][ff])
            acc += mp(post[k]) * mp(f[ff])
            xp[k][ff] = _mp_round(acc, bits)
    # hc_mixes on the flattened new streams, column k*d + f
    flat = [xp[k][ff] for k in range(n) for ff in range(d)]
    ms = mpmath.fsum(v * v for v in flat) / (n * d)
    r = 1 / mpmath.sqrt(ms + mp(norm_eps))
    m = [r * mpmath.fsum(flat[c] * mp(w[j][c]) for c in range(n * d)) for j in range((2 + n) * n)]
    sig = lambda z: 1 / (1 + mpmath.exp(-z))  # noqa: E731
    p_next = [sig(mp(scale[0]) * m[j] + mp(base[j])) + mp(hc_eps) for j in range(n)]
    u_next = [2 * sig(mp(scale[1]) * m[n + k] + mp(base[n + k])) for k in range(n)]
    lg = [[mp(scale[2]) * m[2 * n + j * n + k] + mp(base[2 * n + j * n + k]) for k in range(n)]
          for j in range(n)]
    c = [[None] * n for _ in range(n)]
    for j in range(n):
        mx = max(lg[j])
        ex = [mpmath.exp(v - mx) for v in lg[j]]
        s = mpmath.fsum(ex)
        for k in range(n):
            c[j][k] = ex[k] / s + mp(hc_eps)

    def colnorm():
        for k in range(n):
            s = mpmath.fsum(c[j][k] for j in range(n)) + mp(hc_eps)
            for j in range(n):
                c[j][k] = c[j][k] / s

    def rownorm():
        for j in range(n):
            s = mpmath.fsum(c[j]) + mp(hc_eps)
            for k in range(n):
                c[j][k] = c[j][k] / s

    colnorm()
    for _ in range(iters - 1):
        rownorm()
        colnorm()
    # hc_pre with the previous read weights, then RMSNorm
    h = [_mp_round(mpmath.fsum(mp(pre[k]) * xp[k][ff] for k in range(n)), bits) for ff in range(d)]
    rh = 1 / mpmath.sqrt(mpmath.fsum(v * v for v in h) / d + mp(norm_eps))
    y = [_mp_round(mp(gamma[ff]) * h[ff] * rh, bits) for ff in range(d)]
    return xp, m, p_next, u_next, c, h, y


@pytest.mark.parametrize("n,d", [(4, 1), (4, 2), (4, 8), (2, 1), (2, 8), (8, 1), (8, 2)])
@pytest.mark.parametrize("dtype,bits", [("bf16", 8), ("f32", 24)])
def test_step_brute_force_tiny_d(n, d, dtype, bits):
    """Every stream count the pages' shapes allow (hc_mult = 2, 4, 8): the
    mixes vector has (2+n)*n slots over n*d flattened columns."""
    rng = np.random.default_rng(100 + d + 1000 * (n != 4) * n)
    t = 3 if n == 4 else 2
    xs, f, pre, post, comb, w, base, scale, gamma = _inputs(rng, t, d, dtype, n)
    iters, norm_eps, hc_eps = 20, 1e-6, 1e-6
    o = fused_step(xs, f, pre, post, comb, w, base, scale, gamma, iters, norm_eps, hc_eps, dtype)
    with mpmath.workdps(60):
        for ti in range(t):
            xp, m, p_next, u_next, c, h, y = _brute_step(
                xs[ti], f[ti], pre[ti], post[ti], comb[ti], w, base, scale, gamma,
                iters, norm_eps, hc_eps, bits)
            np.testing.assert_array_equal(o["xprime"][ti], np.array(xp, dtype=float))
            np.testing.assert_allclose(o["m"][ti], np.array(m, dtype=float), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(o["pre"][ti], np.array(p_next, dtype=float), rtol=1e-12)
            np.testing.assert_allclose(o["post"][ti], np.array(u_next, dtype=float), rtol=1e-12)
            np.testing.assert_allclose(o["comb"][ti], np.array(c, dtype=float), rtol=1e-11)
            np.testing.assert_array_equal(o["h"][ti], np.array(h, dtype=float))
            np.testing.assert_array_equal(o["y"][ti], np.array(y, dtype=float))

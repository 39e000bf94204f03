"""Pins for the oracle's split / Sinkhorn step against values the pages fix and
against library routines (scipy's softmax and logistic), never against the
oracle's own formulas retyped."""

from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import sinkhorn_plain, split_sinkhorn
from tests.conftest import load_golden

G = load_golden("sinkhorn_2x2_worked_example.txt")


def _mat(vals):
    return np.array([float(Fraction(v)) for v in vals]).reshape(2, 2)


def _cross_ratios(c):
    """All cross-ratios c[i,j]*c[k,l] / (c[i,l]*c[k,j]) of the trailing n x n."""
    n = c.shape[-1]
    out = []
    for i in range(n):
        for k in range(n):
            for j in range(n):
                for l in range(n):
                    if i != k and j != l:
                        out.append(c[..., i, j] * c[..., k, l] / (c[..., i, l] * c[..., k, j]))
    return np.stack(out, axis=-1)


def _logits_to_m(logits, n):
    """Mixes whose comb slots hold ``logits`` (scale 1, base 0), pre/post 0."""
    t = logits.shape[0]
    m = np.zeros((t, (2 + n) * n))
    m[:, 2 * n:] = logits.reshape(t, n * n)
    return m


# ---- the course page's worked example --------------------------------------------------

def test_worked_example_plain_rounds():
    a = _mat(G["input"])
    np.testing.assert_allclose(sinkhorn_plain(a, 1), _mat(G["round1"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(sinkhorn_plain(a, 2), _mat(G["round2"]), rtol=0, atol=1e-15)


def test_worked_example_plain_limit_and_sums():
    a = _mat(G["input"])
    c = sinkhorn_plain(a, 20)
    t = G["limit_t"]
    np.testing.assert_allclose(c, [[t, 1 - t], [1 - t, t]], rtol=0, atol=1e-12)
    tol = G["sum_tol_after_20"]
    assert np.all(np.abs(c.sum(axis=0) - 1) < tol)
    assert np.all(np.abs(c.sum(axis=1) - 1) < tol)


@pytest.mark.parametrize("iters,key", [(1, "round1"), (2, "round2")])
def test_worked_example_through_split_sinkhorn_n2(iters, key):
    """Row softmax of log(A) is A's row normalisation, so with eps = 0 the
    kernel's schedule reproduces the hand-worked rounds."""
    a = _mat(G["input"])
    m = _logits_to_m(np.log(a)[None], 2)
    _, _, comb = split_sinkhorn(m, [1, 1, 1], np.zeros(8), iters=iters, hc_eps=0.0, n=2)
    np.testing.assert_allclose(comb[0], _mat(G[key]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("iters,key", [(1, "round1"), (2, "round2")])
def test_worked_example_kronecker(iters, key, n):
    """A (x) J_b (b = n/2) has Sinkhorn iterates (iterates of A) (x) J_b / b;
    this drives the n = 4 and n = 8 schedules with the course's example."""
    b = n // 2
    a = _mat(G["input"])
    big = np.kron(a, np.ones((b, b)))
    m = _logits_to_m(np.log(big)[None], n)
    _, _, comb = split_sinkhorn(m, [1, 1, 1], np.zeros((2 + n) * n), iters=iters, hc_eps=0.0,
                                n=n)
    want = np.kron(_mat(G[key]), np.ones((b, b)) / b)
    np.testing.assert_allclose(comb[0], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [4, 8])
def test_worked_example_kronecker_20_rounds(n):
    b = n // 2
    a = _mat(G["input"])
    m = _logits_to_m(np.log(np.kron(a, np.ones((b, b))))[None], n)
    _, _, comb = split_sinkhorn(m, [1, 1, 1], np.zeros((2 + n) * n), iters=20, hc_eps=0.0, n=n)
    t = G["limit_t"]
    want = np.kron(np.array([[t, 1 - t], [1 - t, t]]), np.ones((b, b)) / b)
    np.testing.assert_allclose(comb[0], want, rtol=0, atol=1e-12)
    assert np.all(np.abs(comb.sum(axis=1) - 1) < G["sum_tol_after_20"])
    assert np.all(np.abs(comb.sum(axis=2) - 1) < G["sum_tol_after_20"])


# ---- the kernel's schedule with eps != 0, worked by hand ------------------------------

GE = load_golden("sinkhorn_2x2_eps_quarter.txt")


def _eps_case_m():
    """n = 2 mixes: pre slots (log 3, -log 3), post slots (-log 3, log 3), comb
    slots log A for the course page's A."""
    a = _mat(GE["input"])
    m = _logits_to_m(np.log(a)[None], 2)
    l3 = np.log(3.0)
    m[0, 0:4] = [l3, -l3, -l3, l3]
    return m


@pytest.mark.parametrize("iters,key", [(1, "round1"), (2, "round2")])
def test_eps_quarter_schedule_hand_worked(iters, key):
    """Every placement of eps in the schedule (after the softmax, in the first
    column division, in each later row and column division) changes these
    fractions; dropping or moving any one of them fails this test."""
    eps = float(GE["eps"])
    pre, post, comb = split_sinkhorn(_eps_case_m(), [1, 1, 1], np.zeros(8), iters=iters,
                                     hc_eps=eps, n=2)
    np.testing.assert_allclose(comb[0], _mat(GE[key]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(pre[0], [float(v) for v in GE["pre"]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(post[0], [float(v) for v in GE["post"]], rtol=0, atol=1e-15)


def test_eps_quarter_fractions_follow_from_each_other():
    """The golden's intermediate lines are consistent: round 2's row step is
    round 1 divided by (row sum + eps), elementwise in exact arithmetic."""
    e = GE["eps"]
    r1 = GE["round1"]
    rows = [r1[0:2], r1[2:4]]
    want = [v / (sum(r) + e) for r in rows for v in r]
    assert want == GE["round2_rows"]


# ---- invariants and closed forms --------------------------------------------------------

def _random_m(t, seed, scale=2.86):
    return np.random.default_rng(seed).normal(0, scale, size=(t, 24))


def test_one_iteration_closed_form_with_scipy_softmax():
    """iters = 1: (softmax_k(L) + eps) divided by (its column sum + eps)."""
    rng = np.random.default_rng(1)
    m = _random_m(64, 2)
    scale = rng.uniform(0.5, 2, 3)
    base = rng.normal(0, 0.1, 24)
    eps = 1e-3
    _, _, comb = split_sinkhorn(m, scale, base, iters=1, hc_eps=eps)
    logits = (scale[2] * m[:, 8:] + base[8:]).reshape(-1, 4, 4)
    s = softmax(logits, axis=2) + eps
    want = s / (s.sum(axis=1, keepdims=True) + eps)
    np.testing.assert_allclose(comb, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_cross_ratios_are_those_of_softmax_plus_eps(eps):
    """After the softmax every step is a diagonal row or column scaling, which
    leaves all cross-ratios unchanged."""
    rng = np.random.default_rng(3)
    m = _random_m(128, 4)
    scale = rng.uniform(0.5, 2, 3)
    base = rng.normal(0, 0.1, 24)
    _, _, comb = split_sinkhorn(m, scale, base, iters=20, hc_eps=eps)
    logits = (scale[2] * m[:, 8:] + base[8:]).reshape(-1, 4, 4)
    s = softmax(logits, axis=2) + eps
    np.testing.assert_allclose(_cross_ratios(comb), _cross_ratios(s), rtol=1e-10)


def test_last_normalisation_is_over_columns():
    """The schedule ends with a column division, so column sums are within
    eps/(s + eps) of 1 while row sums need not be."""
    m = _random_m(4096, 5)
    _, _, comb = split_sinkhorn(m, [1.5, 1.5, 2.0], np.zeros(24), iters=20, hc_eps=1e-6)
    col = comb.sum(axis=1)
    assert np.all(np.abs(col - 1) <= 2e-6)
    assert np.max(np.abs(comb.sum(axis=2) - 1)) > 1e-4   # rows not converged at this scale


def test_many_rounds_converge_to_doubly_stochastic():
    rng = np.random.default_rng(6)
    a = rng.uniform(0.1, 3.0, size=(32, 4, 4))
    m = _logits_to_m(np.log(a), 4)
    _, _, comb = split_sinkhorn(m, [1, 1, 1], np.zeros(24), iters=2000, hc_eps=0.0)
    np.testing.assert_allclose(comb.sum(axis=1), 1, atol=1e-12)
    np.testing.assert_allclose(comb.sum(axis=2), 1, atol=1e-12)
    np.testing.assert_allclose(_cross_ratios(comb), _cross_ratios(a), rtol=1e-9)
    np.testing.assert_allclose(comb, sinkhorn_plain(a, 2000), atol=1e-13)


def test_comb_orientation_slot_j_k():
    """Slot 8 + 4j + k is logit (row j, column k): a dominant logit at
    (j, k) = (0, 1) puts the mass of row 0 into column 1."""
    m = np.zeros((1, 24))
    m[0, 8 + 4 * 0 + 1] = 20.0
    _, _, comb = split_sinkhorn(m, [1, 1, 1], np.zeros(24), iters=20, hc_eps=1e-6)
    c = comb[0]
    assert c[0, 1] > 0.9
    assert c[1, 0] < 0.5
    assert np.argmax(c[0]) == 1 and np.argmax(c[:, 1]) == 0


# ---- pre / post -----------------------------------------------------------------------

def test_pre_post_with_scipy_expit():
    rng = np.random.default_rng(7)
    m = _random_m(256, 8)
    scale = rng.uniform(0.5, 2, 3)
    base = rng.normal(0, 0.1, 24)
    eps = 1e-6
    pre, post, _ = split_sinkhorn(m, scale, base, iters=20, hc_eps=eps)
    np.testing.assert_allclose(pre, expit(scale[0] * m[:, :4] + base[:4]) + eps, rtol=1e-15)
    np.testing.assert_allclose(post, 2 * expit(scale[1] * m[:, 4:8] + base[4:8]), rtol=1e-15)


def test_zero_mixes():
    base = np.random.default_rng(9).normal(0, 0.1, 24)
    pre, post, _ = split_sinkhorn(np.zeros((1, 24)), [1.3, 0.7, 1.1], base, hc_eps=1e-6)
    np.testing.assert_allclose(pre[0], expit(base[:4]) + 1e-6, rtol=1e-15)
    np.testing.assert_allclose(post[0], 2 * expit(base[4:8]), rtol=1e-15)


@pytest.mark.parametrize("n,slot", [(4, s) for s in range(24)] + [(2, s) for s in range(8)]
                         + [(8, s) for s in (0, 7, 8, 15, 16, 17, 23, 42, 79)])
def test_each_slot_moves_only_its_own_output(n, slot):
    """Slots 0..n-1 feed pre[j], n..2n-1 post[k], 2n + j*n + k comb entry (j, k)."""
    nm = (2 + n) * n
    base = np.zeros(nm)
    p0, u0, c0 = split_sinkhorn(np.zeros((1, nm)), [1, 1, 1], base, iters=1, hc_eps=0.0, n=n)
    m = np.zeros((1, nm))
    m[0, slot] = 1.0
    p1, u1, c1 = split_sinkhorn(m, [1, 1, 1], base, iters=1, hc_eps=0.0, n=n)
    dp = np.nonzero(np.abs(p1 - p0)[0] > 1e-12)[0].tolist()
    du = np.nonzero(np.abs(u1 - u0)[0] > 1e-12)[0].tolist()
    # with iters = 1 and eps = 0 the column division spreads a row change over the
    # whole matrix, so look at the softmax row instead: the largest entry moves to k
    if slot < n:
        assert dp == [slot] and du == []
    elif slot < 2 * n:
        assert dp == [] and du == [slot - n]
    else:
        j, k = divmod(slot - 2 * n, n)
        assert dp == [] and du == []
        assert np.argmax(c1[0, j]) == k
        assert np.argmax(c1[0, :, k]) == j

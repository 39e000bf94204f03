"""Plain float64 NumPy oracle of the Single-Pass mHC residual step.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously correct,
no blocking, fusion or reordering beyond what the pages define.

Notation follows the pages: ``n`` streams (``hc_mult``; 4 in the model), width
``d``, mixes ``m`` of length ``(2+n)*n``, read weights ``pre`` (p), write
weights ``post`` (u) and the stream combination ``comb`` (C, indexed ``[j, k]``).
Every array argument is converted to float64 first; rounding to the stream
dtype happens exactly where the code excerpts cast back (``round_to``).

Readings taken where the pages are silent or disagree:

* ``hc_post`` contracts ``comb`` on its FIRST index: new stream ``k`` is
  ``sum_j comb[j, k] * X_j + post[k] * F``. This is what the broadcasting in the
  ``hc_post`` excerpt of "Stream weights for the feed-forward" computes; the
  course page's prose ("element (i, j) moves lane j into lane i") describes the
  transpose and is not followed.
* "20 Sinkhorn iterations" means the kernel excerpt's schedule: a row softmax
  plus eps, a column division, then 19 rounds of (row division, column
  division), each division by (sum + eps).
* The rsqrt of ``hc_mixes`` uses ``norm_eps`` (the ``Block`` attribute), the
  split/Sinkhorn uses ``hc_eps``.
* Rounding back to the stream dtype is round-to-nearest-even, applied to the
  exact (float64) value.
"""

from __future__ import annotations

import numpy as np

N_STREAMS = 4

# bf16: 8 significant bits, exponent range of float32.
_BF16_SIG_BITS = 8
_BF16_MIN_EXP = -126          # smallest normal is 2**-126
_BF16_MAX = float.fromhex("0x1.fe00000000000p+127")   # (2 - 2**-7) * 2**127


def n_mix(n: int = N_STREAMS) -> int:
    """Length of the mixes vector, ``(2 + n) * n``.

    "Stream weights for the feed-forward", Code (``Block`` constructor): the
    projection has ``(2 + hc_mult) * hc_mult`` rows over ``hc_mult * dim``
    columns.
    """
    return (2 + n) * n


def parameter_count(n: int = N_STREAMS, d: int = 5120) -> dict:
    """Learned parameters of one ``hc_mixes`` instance, from the tensor shapes.

    "Stream weights for the feed-forward", Code (``Block`` constructor: the
    ``hc_*_fn`` projection ``[mix_hc, hc*dim]``, ``hc_*_base`` ``[mix_hc]`` and
    ``hc_*_scale`` ``[3]``), grouped as in the page's "Parameters" table: the
    projection, then reading / writing / combination weights, each with its
    offsets plus one scale.
    """
    projection = n_mix(n) * (n * d)
    reading = n + 1
    writing = n + 1
    combination = n * n + 1
    return {
        "projection": projection,
        "reading": reading,
        "writing": writing,
        "combination": combination,
        "total": projection + reading + writing + combination,
    }


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    Returned as float64. Non-finite values pass through; values whose rounded
    magnitude exceeds the largest bf16 become +-inf; the subnormal range keeps
    the fixed quantum 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)                      # |x| in [2**(e-1), 2**e)
    q = np.maximum(e - _BF16_SIG_BITS, _BF16_MIN_EXP - (_BF16_SIG_BITS - 1))
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)   # np.rint rounds half to even
    over = np.abs(r) > _BF16_MAX
    r[over] = np.copysign(np.inf, xf[over])
    out[fin] = r
    return out


def round_to(x, dtype: str) -> np.ndarray:
    """Round exact values to the stream dtype (``"bf16"`` or ``"f32"``), RNE.
    ``"f64"`` returns the values unrounded (for checks that need the exact
    value before the cast)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown stream dtype {dtype!r}")


def sigmoid(z) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def split_sinkhorn(m, scale, base, iters: int = 20, hc_eps: float = 1e-6, n: int = N_STREAMS):
    """Split mixes into (pre, post, comb).

    "Stream weights for the feed-forward", Code (``hc_split_sinkhorn`` kernel)
    and the formula list "All 5 steps":

    * pre_j  = sigmoid(scale[0] * m_j + base_j) + hc_eps,            j < n
    * post_k = 2 * sigmoid(scale[1] * m_{n+k} + base_{n+k}),         k < n
    * logits L[j, k] = scale[2] * m_{2n + j*n + k} + base_{2n + j*n + k}
    * comb = row-softmax(L) + hc_eps, then divided by (column sum + hc_eps);
      then ``iters - 1`` times: divide by (row sum + hc_eps), divide by
      (column sum + hc_eps).

    ``m``: [T, (2+n)*n]; returns pre [T, n], post [T, n], comb [T, n, n].
    """
    m = np.asarray(m, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    base = np.asarray(base, dtype=np.float64)
    if iters < 1:
        raise ValueError("iters must be >= 1")
    t = m.shape[0]
    pre = sigmoid(scale[0] * m[:, :n] + base[:n]) + hc_eps
    post = 2.0 * sigmoid(scale[1] * m[:, n:2 * n] + base[n:2 * n])
    logits = (scale[2] * m[:, 2 * n:] + base[2 * n:]).reshape(t, n, n)   # [t, j, k]

    e = np.exp(logits - logits.max(axis=2, keepdims=True))
    comb = e / e.sum(axis=2, keepdims=True) + hc_eps                     # rows: sum over k
    comb = comb / (comb.sum(axis=1, keepdims=True) + hc_eps)             # columns: sum over j
    for _ in range(iters - 1):
        comb = comb / (comb.sum(axis=2, keepdims=True) + hc_eps)
        comb = comb / (comb.sum(axis=1, keepdims=True) + hc_eps)
    return pre, post, comb


def sinkhorn_plain(a, rounds: int):
    """Plain Sinkhorn-Knopp on a positive matrix: divide every row by its sum,
    then every column by its sum, ``rounds`` times; no softmax and no eps.

    "2A · Single-Pass mHC", §3 (the 20-round normalisation as the course
    describes it) and §4 (the hand-checked 2x2 example). ``a``: [..., n, n].
    """
    c = np.array(a, dtype=np.float64, copy=True)
    for _ in range(rounds):
        c = c / c.sum(axis=-1, keepdims=True)
        c = c / c.sum(axis=-2, keepdims=True)
    return c


def mixes(xs, w_mix, base, scale, iters: int = 20, norm_eps: float = 1e-6,
          hc_eps: float = 1e-6):
    """``hc_mixes``: one RMS statistic over the flattened streams, the
    ``(2+n)*n``-wide projection, then the split/Sinkhorn.

    "Stream weights for the feed-forward", Code (``hc_mixes``) and the formula
    for ``m`` in "All 5 steps": with x the token's streams flattened so that
    column ``k*d + f`` holds stream k, feature f,
    m = (x @ W^T) / sqrt(mean(x**2) + norm_eps).

    ``xs``: [T, n, d] (values already in the stream dtype); ``w_mix``:
    [(2+n)*n, n*d]. Returns (m, pre, post, comb).
    """
    xs = np.asarray(xs, dtype=np.float64)
    t, n, d = xs.shape
    x = xs.reshape(t, n * d)
    w = np.asarray(w_mix, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + norm_eps)
    m = (x @ w.T) * r[:, None]
    pre, post, comb = split_sinkhorn(m, scale, base, iters, hc_eps, n)
    return m, pre, post, comb


def hc_post(xs, f, post, comb, dtype: str):
    """``hc_post``: new stream k = sum_j comb[j, k] * X_j + post_k * F,
    rounded to the stream dtype.

    "Stream weights for the feed-forward", Code (``hc_post``): the product
    ``comb.unsqueeze(-1) * residual.unsqueeze(-2)`` pairs residual stream j
    with ``comb[j, :]`` and the sum runs over that first index; the result is
    cast back to the dtype of the sublayer output.

    ``xs``: [T, n, d], ``f``: [T, d], ``post``: [T, n], ``comb``: [T, n, n].
    """
    xs = np.asarray(xs, dtype=np.float64)
    f = np.asarray(f, dtype=np.float64)
    post = np.asarray(post, dtype=np.float64)
    comb = np.asarray(comb, dtype=np.float64)
    mixed = np.einsum("tjk,tjf->tkf", comb, xs)
    return round_to(mixed + post[:, :, None] * f[:, None, :], dtype)


def hc_pre(xs, pre, dtype: str):
    """``hc_pre``: collapse the streams with the read weights,
    h = sum_k pre_k * X_k, rounded to the stream dtype.

    "Stream weights for the feed-forward", Code (``hc_pre``).
    """
    xs = np.asarray(xs, dtype=np.float64)
    pre = np.asarray(pre, dtype=np.float64)
    return round_to(np.einsum("tk,tkf->tf", pre, xs), dtype)


def rmsnorm(h, gamma, eps: float, dtype: str):
    """RMSNorm: y = gamma * h / sqrt(mean(h**2) + eps), rounded to the dtype.

    "DeepSeek V4.1 · MoE RMSNorm", the formula and Code (``RMSNorm``).
    """
    h = np.asarray(h, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(h * h, axis=1) + eps)
    return round_to(gamma[None, :] * h * r[:, None], dtype)


def fused_step_from_xprime(xprime, pre_in, w_mix, base, scale, gamma, iters: int = 20,
                           norm_eps: float = 1e-6, hc_eps: float = 1e-6, dtype: str = "bf16"):
    """Everything of the step that follows ``hc_post``, given the new streams.

    Returns dict with m, pre, post, comb (the next coefficients, from the new
    streams with the NEXT sublayer's parameters), h and y (the next sublayer's
    normalised input, read with the PREVIOUS sublayer's ``pre``).
    "DeepSeek V4.1 · MoE RMSNorm", Code (``Block.forward``: after ``hc_post``
    the block calls ``hc_mixes`` on the new streams, ``hc_pre`` with the read
    weights computed one sublayer earlier, then the norm).
    """
    m, pre, post, comb = mixes(xprime, w_mix, base, scale, iters, norm_eps, hc_eps)
    h = hc_pre(xprime, pre_in, dtype)
    y = rmsnorm(h, gamma, norm_eps, dtype)
    return {"m": m, "pre": pre, "post": post, "comb": comb, "h": h, "y": y}


def fused_step(xs, f, pre_in, post_in, comb_in, w_mix, base, scale, gamma, iters: int = 20,
               norm_eps: float = 1e-6, hc_eps: float = 1e-6, dtype: str = "bf16"):
    """One Single-Pass mHC step at a sublayer boundary.

    Inputs from sublayer i: the streams ``xs`` that entered it, its output
    ``f`` and the coefficients (pre_in, post_in, comb_in) its ``hc_mixes``
    computed from ``xs``; parameters (w_mix, base, scale, gamma) of sublayer
    i+1. Steps, in the order of ``Block.forward`` ("DeepSeek V4.1 · MoE
    RMSNorm", Code): ``hc_post`` -> ``hc_mixes`` -> ``hc_pre`` (with pre_in)
    -> RMSNorm. Returns dict with xprime plus the keys of
    ``fused_step_from_xprime``.
    """
    xprime = hc_post(xs, f, post_in, comb_in, dtype)
    out = fused_step_from_xprime(xprime, pre_in, w_mix, base, scale, gamma, iters,
                                 norm_eps, hc_eps, dtype)
    out["xprime"] = xprime
    return out

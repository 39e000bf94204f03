"""Parity checks of HIP outputs against the float64 oracle.

Tolerances (the parity bar of this implementation):

* mixes m, pre, post and every comb entry (float32): |g - o| <= 1e-4 * max(|o|, 1).
* comb row and column sums: within 1e-5 of the oracle's same sums, and every
  column sum within 1e-5 + hc_eps of 1 (the schedule ends with a column
  division, which leaves each column short of 1 by eps/(s + eps)).
* bf16 stream outputs (new streams, y): |g - o| <= ulp_bf16(o) + 1e-3; the new
  streams are held to the stricter rule below.
* f32 stream outputs: |g - o| <= 1e-5 * max(|o|, 1).

Roundings with more than one correct result. The kernels (like the code on
the pages) evaluate the new streams and h in float32 and then round to bf16.
Every bf16 value between the roundings of (exact - b) and (exact + b), with b
the float32 evaluation error bound of that element, is a correct result; near
a rounding boundary that is two neighbours, under cancellation it can be a
few. The check demands that every element lies in its oracle-computed
interval (a single value almost everywhere). Because the later stages depend
on which correct rounding was taken, they are compared against the oracle
evaluated on the new streams as validated (each element inside its
interval), so that a correct tie choice is not reported as a mixes error.
"""

from __future__ import annotations

import numpy as np

import oracle

MIX_RTOL = 1e-4
SUM_TOL = 1e-5
BF16_ABS = 1e-3
F32_RTOL = 1e-5
# bound on the float32 evaluation error of a short fma chain, relative to the
# sum of the magnitudes of its terms (5 roundings of 2**-24, with margin)
EVAL_REL = 2.0 ** -21


def ulp_bf16(v):
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def _np(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        return a.double().numpy()
    return np.asarray(a, dtype=np.float64)


class ParityError(AssertionError):
    pass


def _fail(what, mask, got, want, extra=""):
    idx = np.argwhere(mask)
    first = tuple(idx[0]) if len(idx) else ()
    where = ""
    if mask.ndim >= 2:
        toks = np.unique(idx[:, 0])
        where = f"; tokens {toks[:12].tolist()}{' ...' if len(toks) > 12 else ''}"
        if mask.ndim == 2:
            steps = np.unique(idx[:, 1] // 32)
            where += f"; 32-feature blocks {steps[:12].tolist()}"
    raise ParityError(f"{what}: {int(mask.sum())} of {mask.size} elements out of tolerance; "
                      f"first at {first}: got {got[first]!r} want {want[first]!r} {extra}{where}")


def check_mix_like(what, got, want):
    got, want = _np(got), _np(want)
    bad = ~(np.abs(got - want) <= MIX_RTOL * np.maximum(np.abs(want), 1.0))
    if bad.any():
        _fail(what, bad, got, want)


def check_comb(got, want, hc_eps=1e-6, iters=20):
    """Entries, row and column sums against the oracle's; column sums against
    1 within the tolerance plus the shortfall eps/(s + eps) the final column
    division leaves. That shortfall is below hc_eps only once a full round has
    run (iters >= 2): after the softmax alone a column can hold little more
    than the eps floor, so the check against 1 is skipped for iters = 1."""
    got, want = _np(got), _np(want)
    check_mix_like("comb", got, want)
    for axis, name in ((1, "column"), (2, "row")):
        gs, ws = got.sum(axis=axis), want.sum(axis=axis)
        bad = ~(np.abs(gs - ws) <= SUM_TOL)
        if bad.any():
            _fail(f"comb {name} sums", bad, gs, ws)
    if iters < 2:
        return
    cs = got.sum(axis=1)
    bad = ~(np.abs(cs - 1.0) <= SUM_TOL + hc_eps)
    if bad.any():
        _fail("comb column sums vs 1", bad, cs, np.ones_like(cs))


def check_stream(what, got, want, dtype):
    got, want = _np(got), _np(want)
    if dtype == "bf16":
        bad = ~(np.abs(got - want) <= ulp_bf16(want) + BF16_ABS)
    else:
        bad = ~(np.abs(got - want) <= F32_RTOL * np.maximum(np.abs(want), 1.0))
    if bad.any():
        _fail(what, bad, got, want)


def resolve_rounding(got, exact, bound, dtype, what):
    """Check that every element of ``got`` is a rounding (to ``dtype``) of some
    value within ``exact`` +- ``bound``; return it as validated, with the count
    of elements whose interval holds more than one value."""
    lo = oracle.round_to(exact - bound, dtype)
    hi = oracle.round_to(exact + bound, dtype)
    nearest = oracle.round_to(exact, dtype)
    ok = (got >= lo) & (got <= hi) & (got == oracle.round_to(got, dtype))
    if not ok.all():
        _fail(what, ~ok, got, nearest, "(not a correct rounding of the exact value)")
    return np.where(ok, got, nearest), int((lo != hi).sum())


def check_mixes(inputs, gpu, dtype):
    """mhc_mixes outputs vs oracle.mixes on the same streams."""
    xs = _np(inputs["x"])
    m, pre, post, comb = oracle.mixes(xs, inputs["w_mix"], inputs["base"], inputs["scale"],
                                      inputs.get("iters", 20), inputs.get("norm_eps", 1e-6),
                                      inputs.get("hc_eps", 1e-6))
    if gpu.get("mix") is not None:
        check_mix_like("mix", gpu["mix"], m)
    check_mix_like("pre", gpu["pre"], pre)
    check_mix_like("post", gpu["post"], post)
    check_comb(gpu["comb"], comb, inputs.get("hc_eps", 1e-6), inputs.get("iters", 20))
    return {"m": m, "pre": pre, "post": post, "comb": comb}


def check_step(inputs, gpu, dtype, coef_abs=0.0):
    """Fused-step outputs vs the oracle.

    ``inputs``: x [T,4,d], f [T,d] (torch CPU, stream dtype), pre/post/comb
    (numpy), w_mix, base, scale, gamma, optional iters/norm_eps/hc_eps.
    ``gpu``: dict with x_out, y, pre, post, comb and optional mix.
    ``coef_abs``: per-token bound (scalar or [T]) on how far the coefficients
    the GPU consumed may be from the oracle's (chained steps, where each side
    feeds its own previous outputs forward); it widens the rounding bands of
    the new streams and of h accordingly.
    Returns the oracle's outputs (x_out as the resolved candidate) for chaining.
    """
    iters = inputs.get("iters", 20)
    norm_eps = inputs.get("norm_eps", 1e-6)
    hc_eps = inputs.get("hc_eps", 1e-6)
    xs, f = _np(inputs["x"]), _np(inputs["f"])
    pre_in, post_in, comb_in = (_np(inputs[k]) for k in ("pre", "post", "comb"))
    gx = _np(gpu["x_out"])

    coef_abs = np.broadcast_to(np.asarray(coef_abs, dtype=np.float64), (xs.shape[0],))
    exact = oracle.hc_post(xs, f, post_in, comb_in, "f64")
    if dtype == "bf16":
        mag = oracle.hc_post(np.abs(xs), np.abs(f), np.abs(post_in), np.abs(comb_in), "f64")
        spread = (np.abs(xs).sum(axis=1) + np.abs(f))[:, None, :] * coef_abs[:, None, None]
        xprime, n_ties = resolve_rounding(gx, exact, EVAL_REL * mag + spread, dtype,
                                          "new streams")
    else:
        xprime = oracle.round_to(exact, dtype)
        check_stream("new streams", gx, xprime, dtype)
        n_ties = 0

    o = oracle.fused_step_from_xprime(xprime, pre_in, inputs["w_mix"], inputs["base"],
                                      inputs["scale"], inputs["gamma"], iters, norm_eps, hc_eps,
                                      dtype)
    if gpu.get("mix") is not None:
        check_mix_like("mix", gpu["mix"], o["m"])
    check_mix_like("pre", gpu["pre"], o["pre"])
    check_mix_like("post", gpu["post"], o["post"])
    check_comb(gpu["comb"], o["comb"], hc_eps, iters)

    gy = _np(gpu["y"])
    if dtype == "bf16":
        h_exact = oracle.hc_pre(xprime, pre_in, "f64")
        h_mag = oracle.hc_pre(np.abs(xprime), np.abs(pre_in), "f64")
        h_band = EVAL_REL * h_mag + np.abs(xprime).sum(axis=1) * coef_abs[:, None]
        h_lo = oracle.round_to(h_exact - h_band, dtype)
        h_hi = oracle.round_to(h_exact + h_band, dtype)
        y_lo = oracle.rmsnorm(h_lo, inputs["gamma"], norm_eps, dtype)
        y_hi = oracle.rmsnorm(h_hi, inputs["gamma"], norm_eps, dtype)
        tol = np.maximum(ulp_bf16(y_lo), ulp_bf16(y_hi)) + BF16_ABS
        ok = (gy >= np.minimum(y_lo, y_hi) - tol) & (gy <= np.maximum(y_lo, y_hi) + tol)
        if not ok.all():
            _fail("y", ~ok, gy, o["y"])
    else:
        check_stream("y", gy, o["y"], dtype)
    o["xprime"] = xprime
    o["n_ties"] = n_ties
    return o


def coef_gap(gpu, ref):
    """Per-token max |gpu - oracle| over pre, post and comb."""
    parts = [np.abs(_np(gpu[k]) - _np(ref[k])).reshape(len(_np(ref[k])), -1)
             for k in ("pre", "post", "comb")]
    return np.concatenate(parts, axis=1).max(axis=1)


def comb_sum_stats(comb):
    c = _np(comb)
    return {"row_dev_max": float(np.abs(c.sum(axis=2) - 1).max()),
            "row_dev_median": float(np.median(np.abs(c.sum(axis=2) - 1))),
            "col_dev_max": float(np.abs(c.sum(axis=1) - 1).max())}

"""GPU parity of the step run as separate kernels (the pages' form: hc_post,
hc_mixes, hc_pre, RMSNorm) and of mhc_mixes's feature-split mode.

Each kernel is checked against the float64 oracle's function of the same
name (the rounding-interval rule of tests/parity.py for bf16 outputs). The
composition must give the fused kernel's new streams bit for bit (same
per-element arithmetic) and its y within one bf16 ulp (the sum of h^2 is
accumulated in a different order).
"""

import numpy as np
import pytest
import torch

import oracle
import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, run_step, to_dev
from tests.parity import (EVAL_REL, _np, check_comb, check_mix_like, check_mixes, check_stream,
                          resolve_rounding)

pytestmark = pytest.mark.gpu


def _dev(case):
    return {k: to_dev(case[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                         "scale", "gamma")}


def _check_rounded(what, got, exact, mag, dtype):
    if dtype == "bf16":
        return resolve_rounding(_np(got), exact, EVAL_REL * mag, dtype, what)[0]
    check_stream(what, got, exact, dtype)
    return _np(got)


@pytest.mark.parametrize("dtype,d,t", [("bf16", 5120, 37), ("bf16", 256, 100), ("f32", 64, 17)])
def test_hc_post_pre_rmsnorm_parity(dtype, d, t):
    case = make_case(wl.Workload(600 + d % 37, "unfused", t, d, dtype))
    dev = _dev(case)
    xo = mhc.hc_post(dev["x"], dev["f"], dev["post"], dev["comb"])
    torch.cuda.synchronize()
    xs, f = _np(case["x"]), _np(case["f"])
    exact = oracle.hc_post(xs, f, case["post"], case["comb"], "f64")
    mag = oracle.hc_post(np.abs(xs), np.abs(f), np.abs(case["post"]), np.abs(case["comb"]), "f64")
    xprime = _check_rounded("hc_post", xo.cpu(), exact, mag, dtype)

    h = mhc.hc_pre(xo, dev["pre"])
    torch.cuda.synchronize()
    h_exact = oracle.hc_pre(xprime, case["pre"], "f64")
    h_mag = oracle.hc_pre(np.abs(xprime), np.abs(case["pre"]), "f64")
    hv = _check_rounded("hc_pre", h.cpu(), h_exact, h_mag, dtype)

    y = mhc.rmsnorm(h, dev["gamma"], 1e-6)
    torch.cuda.synchronize()
    check_stream("rmsnorm", y.cpu(), oracle.rmsnorm(hv, case["gamma"], 1e-6, dtype), dtype)


def test_in_place_hc_post_and_rmsnorm():
    case = make_case(wl.Workload(610, "unfused_inplace", 50, 512, "bf16"))
    dev = _dev(case)
    ref = mhc.hc_post(dev["x"], dev["f"], dev["post"], dev["comb"])
    x2 = dev["x"].clone()
    mhc.hc_post(x2, dev["f"], dev["post"], dev["comb"], x_out=x2)
    hy = mhc.hc_pre(ref, dev["pre"])
    yref = mhc.rmsnorm(hy, dev["gamma"])
    mhc.rmsnorm(hy, dev["gamma"], y_out=hy)
    torch.cuda.synchronize()
    assert torch.equal(x2, ref)
    assert torch.equal(hy, yref)


@pytest.mark.parametrize("d,t", [(5120, 1000), (5120, 9000), (3072, 300), (4096, 5)])
def test_mixes_split_mode_parity(d, t):
    w = wl.Workload(620 + t % 11, "mixes_split", t, d, "bf16")
    x = wl.streams(w)
    p = wl.params(w)
    wp = mhc.pack_wmix(to_dev(p["w_mix"]), "bf16")
    ws = torch.zeros(mhc.fused_step_workspace_bytes(t, d, "bf16"), dtype=torch.uint8,
                     device="cuda")
    dx = to_dev(x)
    out = mhc.mixes(dx, wp, to_dev(p["base"]), to_dev(p["scale"]), want_mix=True, path="split",
                    workspace=ws)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    check_mixes(dict(x=x, **p), {k: v.cpu() for k, v in out.items()}, "bf16")
    tile = mhc.mixes(dx, wp, to_dev(p["base"]), to_dev(p["scale"]), want_mix=True, path="tile")
    # the two routes agree to the parity bar: on 256-feature slices the split
    # route's projection uses the hi and mid terms of W (each product within
    # 2^-16 of its magnitude), the tile route all three
    for k in ("pre", "post", "comb", "mix"):
        check_mix_like(k, out[k].cpu(), tile[k].cpu())


@pytest.mark.parametrize("t", [700, 5000])
def test_three_kernel_step_matches_fused(t):
    case = make_case(wl.Workload(630 + t % 13, "three_kernel", t, 5120, "bf16"))
    dev = _dev(case)
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    a = mhc.three_kernel_step(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp,
                              dev["base"], dev["scale"], dev["gamma"], want_mix=True)
    b, _ = run_step(case)
    torch.cuda.synchronize()
    assert torch.equal(a["x_out"].cpu(), b["x_out"])
    ya, yb = a["y"].float().cpu(), b["y"].float()
    assert ((ya - yb).abs() <= torch.maximum(ya.abs(), yb.abs()) * 2.0 ** -7 + 1e-30).all()
    for k in ("pre", "post", "mix"):
        check_mix_like(k, a[k].cpu(), _np(b[k]))
    check_comb(a["comb"].cpu(), _np(b["comb"]))

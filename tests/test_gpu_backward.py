"""GPU parity of the backward of the fused step (mhc_fused_step_backward_n).

Each case runs the forward on the GPU (mhc_fused_step_n, which stores the new
streams and the mixes), validates the new streams against the float64 oracle
(every element a correct rounding), runs the backward on the GPU, and compares
every gradient with the float64 backward oracle evaluated on the validated new
streams (the forward output a backward receives).

Tolerances follow from the float32 arithmetic: each gradient may differ from
the exact value by 1e-4 of the sum of the magnitudes of the terms that form
it (the oracle supplies those magnitudes), and the gradients in the stream
dtype additionally by one unit in the last place of that dtype.
"""

import numpy as np
import pytest
import torch

import oracle
import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, to_dev
from tests.parity import _fail, _np, check_step, ulp_bf16

pytestmark = pytest.mark.gpu

REL = 1e-4


def _log(msg):
    print(msg, flush=True)


def _check(what, got, want, mag, dtype=None):
    got, want = _np(got), np.asarray(want, dtype=np.float64)
    tol = REL * mag + 1e-6
    if dtype == "bf16":
        tol = tol + ulp_bf16(want)
    elif dtype == "f32":
        tol = tol + np.abs(want) * 2.0 ** -23
    bad = ~(np.abs(got - want) <= tol)
    if bad.any():
        _fail(what, bad, got, want)
    # how much of the float32 allowance was used (the stream-dtype ulp aside)
    extra = np.maximum(np.abs(got - want) - (tol - REL * mag - 1e-6), 0.0)
    return float((extra / (mag + 1e-30)).max())


def check_token_grads(case, got, up, xprime, iters, dtype):
    """The per-token gradients (d_x, d_f, d_comb_in, d_post_in, d_pre_in) of
    the tokens of ``case`` against the float64 backward oracle evaluated on
    the validated new streams ``xprime``; ``up``: the upstream gradients of
    those tokens (numpy). Returns the oracle's outputs and the share of each
    tolerance used."""
    xs, f = _np(case["x"]), _np(case["f"])
    t, n, d = xs.shape
    pre = np.asarray(case["pre"], np.float64)
    post = np.asarray(case["post"], np.float64)
    comb = np.asarray(case["comb"], np.float64)
    want = oracle.fused_step_backward(xs, f, pre, post, comb, case["w_mix"], case["base"],
                                      case["scale"], case["gamma"], up["d_xprime"], up["d_y"],
                                      up["d_pre"], up["d_post"], up["d_comb"], iters,
                                      case["norm_eps"], case["hc_eps"], dtype, xprime=xprime)
    # magnitudes of the terms forming each gradient
    xp, dh = want["xprime"], want["dh"]
    mag_da = (np.abs(up["d_xprime"]) + np.abs(want["dx_mix"]).reshape(t, n, d)
              + np.abs(pre)[:, :, None] * np.abs(dh)[:, None, :])
    used = {}
    used["d_x"] = _check("d_x", got["d_x"], want["d_x"],
                         np.einsum("tjk,tkf->tjf", np.abs(comb), mag_da), dtype)
    used["d_f"] = _check("d_f", got["d_f"], want["d_f"],
                         np.einsum("tk,tkf->tf", np.abs(post), mag_da), dtype)
    used["d_comb_in"] = _check("d_comb_in", got["d_comb_in"], want["d_comb_in"],
           np.einsum("tjf,tkf->tjk", np.abs(xs), mag_da))
    used["d_post_in"] = _check("d_post_in", got["d_post_in"], want["d_post_in"],
           np.einsum("tf,tkf->tk", np.abs(f), mag_da))
    used["d_pre_in"] = _check("d_pre_in", got["d_pre_in"], want["d_pre_in"],
           np.einsum("tf,tkf->tk", np.abs(dh), np.abs(xp)))
    return want, used


def run_backward_case(n, dtype, d, t, seed, iters=20):
    case = make_case(wl.Workload(seed, "backward", t, d, dtype, n=n, iters=iters))
    rng = np.random.default_rng(seed + 1)
    up = {"d_xprime": oracle.round_to(rng.standard_normal((t, n, d)), dtype),
          "d_y": oracle.round_to(rng.standard_normal((t, d)), dtype),
          "d_pre": rng.standard_normal((t, n)), "d_post": rng.standard_normal((t, n)),
          "d_comb": rng.standard_normal((t, n, n))}
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {k: to_dev(case[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base", "scale",
                                        "gamma")}
    wp = mhc.pack_wmix_n(dev["w_mix"], dtype)
    fwd = mhc.fused_step_n(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp,
                           dev["base"], dev["scale"], dev["gamma"], iters, case["norm_eps"],
                           case["hc_eps"])
    torch.cuda.synchronize()
    o = check_step(case, {k: v.cpu() for k, v in fwd.items()}, dtype)
    dup = {"d_xprime": torch.tensor(up["d_xprime"]).to(tdt).cuda(),
           "d_y": torch.tensor(up["d_y"]).to(tdt).cuda(),
           "d_pre": to_dev(up["d_pre"].astype(np.float32)),
           "d_post": to_dev(up["d_post"].astype(np.float32)),
           "d_comb": to_dev(up["d_comb"].astype(np.float32))}
    got = mhc.fused_step_backward_n(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"],
                                    fwd["x_out"], fwd["mix"], dev["w_mix"], dev["base"],
                                    dev["scale"], dev["gamma"], dup["d_xprime"], dup["d_y"],
                                    dup["d_pre"], dup["d_post"], dup["d_comb"], iters,
                                    case["norm_eps"], case["hc_eps"])
    torch.cuda.synchronize()
    got = {k: v.cpu() for k, v in got.items()}
    want, used = check_token_grads(case, got, up, o["xprime"], iters, dtype)
    xp, h = want["xprime"], want["h"]
    s_slot = np.concatenate([np.full(n, case["scale"][0]), np.full(n, case["scale"][1]),
                             np.full(n * n, case["scale"][2])]).astype(np.float64)
    dz = np.abs(want["g"] * s_slot * want["r"][:, None])
    used["d_w_mix"] = _check("d_w_mix", got["d_w_mix"], want["d_w_mix"],
                             dz.T @ np.abs(xp.reshape(t, n * d)))
    used["d_gamma"] = _check("d_gamma", got["d_gamma"], want["d_gamma"],
           (np.abs(up["d_y"]) * np.abs(h) * want["rho"][:, None]).sum(axis=0))
    gabs = np.abs(want["g"]).sum(axis=1, keepdims=True)        # per-token scale of g
    used["d_base"] = _check("d_base", got["d_base"], want["d_base"],
                            np.broadcast_to(gabs, want["g"].shape).sum(0))
    gm = np.abs(want["g"] * want["m"])
    used["d_scale"] = _check("d_scale", got["d_scale"], want["d_scale"],
           np.array([gm.sum(), gm.sum(), gm.sum()]))
    _log("  relative error used per gradient: "
         + ", ".join(f"{k} {v:.1e}" for k, v in used.items()))
    return got


CASES = [
    # n, dtype, d, tokens, iters
    (4, "bf16", 5120, 200, 20),
    (4, "bf16", 256, 129, 20),
    (4, "bf16", 1024, 1, 20),
    (2, "bf16", 512, 300, 20),
    (4, "f32", 128, 40, 20),
    (2, "f32", 64, 17, 1),
    (4, "bf16", 2080, 70, 3),
    (4, "bf16", 64, 65, 20),      # one 64-feature unit; a second workgroup with one token
]


@pytest.mark.parametrize("n,dtype,d,t,iters", CASES)
def test_backward_parity(n, dtype, d, t, iters):
    _log(f"backward n={n} {dtype} d={d} T={t} iters={iters}")
    run_backward_case(n, dtype, d, t, 900 + n + d % 13 + t % 7 + iters, iters)


def test_backward_deterministic():
    a = run_backward_case(4, "bf16", 512, 300, 950)
    b = run_backward_case(4, "bf16", 512, 300, 950)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.timeout(900)
def test_backward_ragged_wide():
    """d = 5312 (83 units of 64 features, not a multiple of 256) and 4,100
    tokens (65 workgroups of the stream kernel, the last with 4 tokens):
    every gradient checked in full."""
    run_backward_case(4, "bf16", 5312, 4100, 970)


@pytest.mark.timeout(900)
def test_backward_many_blocks():
    """8,192 tokens x d = 5120 (64 workgroups of the stream kernel, every
    token chunk of the parameter kernel): every gradient checked in full."""
    run_backward_case(4, "bf16", 5120, 8192, 960)

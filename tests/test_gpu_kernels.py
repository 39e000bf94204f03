"""GPU parity of the HIP kernels against the float64 oracle at sizes the oracle
finishes in seconds: several tiles, ragged token tails, tiny and non-register
widths, special cases, determinism, in-place use and guard bands."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, run_step, to_dev
from tests.conftest import load_golden
from tests.parity import check_comb, check_mix_like, check_mixes, check_step

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


# ---- split + Sinkhorn ------------------------------------------------------------------

@pytest.mark.parametrize("t", [1, 255, 1000])
@pytest.mark.parametrize("iters,eps", [(20, 1e-6), (1, 1e-6), (5, 0.0), (50, 1e-2)])
def test_sinkhorn4_random(t, iters, eps):
    rng = np.random.default_rng(t * 7 + iters)
    m = (rng.standard_normal((t, 24)) * 2.86).astype(np.float32)
    base = (rng.standard_normal(24) * 0.1).astype(np.float32)
    scale = rng.uniform(0.5, 2.0, 3).astype(np.float32)
    out = mhc.sinkhorn4(to_dev(m), to_dev(base), to_dev(scale), iters, eps)
    torch.cuda.synchronize()
    pre, post, comb = oracle.split_sinkhorn(m, scale, base, iters, eps)
    check_mix_like("pre", out["pre"].cpu(), pre)
    check_mix_like("post", out["post"].cpu(), post)
    if iters >= 5:
        check_comb(out["comb"].cpu(), comb, eps)
    else:
        check_mix_like("comb", out["comb"].cpu(), comb)


@pytest.mark.parametrize("iters,key", [(1, "round1"), (2, "round2"), (20, None)])
def test_sinkhorn4_worked_example(iters, key):
    """The course page's 2x2 example, embedded as A (x) J2 into the 4x4 with
    eps = 0; compared with the hand-worked fractions, not with the oracle."""
    g = load_golden("sinkhorn_2x2_worked_example.txt")
    a = np.array([float(Fraction(v)) for v in g["input"]]).reshape(2, 2)
    m = np.zeros((3, 24), np.float32)
    m[:, 8:] = np.log(np.kron(a, np.ones((2, 2)))).reshape(16)
    out = mhc.sinkhorn4(to_dev(m), to_dev(np.zeros(24, np.float32)),
                        to_dev(np.ones(3, np.float32)), iters, 0.0)
    torch.cuda.synchronize()
    if key is None:
        t = g["limit_t"]
        small = np.array([[t, 1 - t], [1 - t, t]])
    else:
        small = np.array([float(Fraction(v)) for v in g[key]]).reshape(2, 2)
    want = np.kron(small, np.ones((2, 2)) / 2)
    got = out["comb"].cpu().double().numpy()
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), atol=2e-6)
    if key is None:
        assert np.all(np.abs(got.sum(axis=1) - 1) < 1e-6)
        assert np.all(np.abs(got.sum(axis=2) - 1) < 1e-6)


# ---- packing of the projection ---------------------------------------------------------

def _unpack_bf16(buf, d):
    """Host decode of the packed bf16 layout [step][stream][tile][lane][8]."""
    s = d // 32
    u = buf.cpu().numpy().view(np.uint16).reshape(s, 4, 5, 64, 8)
    vals = (u.astype(np.uint32) << 16).view(np.float32)
    terms = np.zeros((3, 24, 4 * d), np.float64)
    pad = []
    for q in range(5):
        for lane in range(64):
            n = 16 * q + lane % 16
            grp = lane // 16
            for k in range(4):
                cols = k * d + 32 * np.arange(s)[:, None] + 8 * grp + np.arange(8)[None, :]
                v = vals[:, k, q, lane, :]
                if n < 72:
                    terms[n // 24, n % 24, cols.reshape(-1)] = v.reshape(-1)
                else:
                    pad.append(v)
    return terms, np.concatenate([p.reshape(-1) for p in pad]) if pad else np.zeros(0)


@pytest.mark.parametrize("d", [32, 160, 5120])
def test_pack_bf16_split_is_exact(d):
    rng = np.random.default_rng(d)
    w = (rng.standard_normal((24, 4 * d)) * 0.02).astype(np.float32)
    w[0, :7] = [0.0, -0.0, 1e-30, 3.0e38, -1.17549435e-38, 1.0, 1.0 + 2.0 ** -23]
    buf = mhc.pack_wmix(to_dev(w), "bf16")
    torch.cuda.synchronize()
    terms, pad = _unpack_bf16(buf, d)
    total = terms[0] + terms[1] + terms[2]                 # exact in float64
    np.testing.assert_array_equal(total, w.astype(np.float64))
    assert not np.any(pad)
    # hi is the bf16 rounding of w
    np.testing.assert_array_equal(terms[0], oracle.round_bf16(w.astype(np.float64)))


def test_pack_f32_layout():
    d = 64
    rng = np.random.default_rng(3)
    w = rng.standard_normal((24, 4 * d)).astype(np.float32)
    buf = mhc.pack_wmix(to_dev(w), "f32")
    torch.cuda.synchronize()
    v = buf.cpu().numpy().view(np.float32).reshape(d // 32, 4, 2, 64, 8)
    for s in range(d // 32):
        for k in range(4):
            for q in range(2):
                for lane in range(64):
                    n = 16 * q + lane % 16
                    cols = k * d + 32 * s + 8 * (lane // 16) + np.arange(8)
                    want = w[n, cols] if n < 24 else np.zeros(8, np.float32)
                    np.testing.assert_array_equal(v[s, k, q, lane], want)


# ---- mixes -----------------------------------------------------------------------------

MIXES_CASES = [("bf16", 5120, 37), ("bf16", 64, 100), ("bf16", 32, 16), ("bf16", 7168, 40),
               ("f32", 5120, 20), ("f32", 96, 33)]


@pytest.mark.parametrize("dtype,d,t", MIXES_CASES)
def test_mixes_parity(dtype, d, t):
    _log(f"mixes dtype={dtype} d={d} T={t}")
    w = wl.Workload(100 + d, "mixes", t, d, dtype)
    x = wl.streams(w)
    p = wl.params(w)
    dx = to_dev(x)
    wp = mhc.pack_wmix(to_dev(p["w_mix"]), dtype)
    out = mhc.mixes(dx, wp, to_dev(p["base"]), to_dev(p["scale"]), want_mix=True)
    torch.cuda.synchronize()
    check_mixes(dict(x=x, **p), {k: v.cpu() for k, v in out.items()}, dtype)


# ---- fused step ------------------------------------------------------------------------

STEP_CASES = [
    ("bf16", 5120, 37),     # register-resident h, ragged last tile
    ("bf16", 5120, 16),     # exactly one tile
    ("bf16", 256, 100),     # one step per wave
    ("bf16", 32, 5),        # a single step: only wave 0 works
    ("bf16", 1056, 50),     # steps not a multiple of the wave count
    ("bf16", 6144, 20),     # beyond the register budget: h parked in y
    ("f32", 5120, 64),      # the fp32 correctness workload shape
    ("f32", 64, 17),
]


# path "tile" always runs the tile kernels; "auto" (with a workspace) takes the
# chunked kernels for these small calls where they apply (f32, and bf16 with
# d <= 5120 and an even number of 32-feature steps), the feature-split kernel
# for d = 6144, and the tile kernels otherwise
@pytest.mark.parametrize("path", ["tile", "auto"])
@pytest.mark.parametrize("dtype,d,t", STEP_CASES)
def test_fused_step_parity(dtype, d, t, path):
    _log(f"fused dtype={dtype} d={d} T={t} path={path}")
    w = wl.Workload(200 + d % 97, "step", t, d, dtype)
    case = make_case(w)
    out, _ = run_step(case, dtype=dtype, path=path)
    o = check_step(case, out, dtype)
    _log(f"  ties in new streams: {o['n_ties']}")


def test_fused_step_outlier_tokens():
    w = wl.Workload(2, "decode_small", 300, 1024, "bf16", outlier_frac=0.01, outlier_scale=30.0)
    case = make_case(w)
    out, _ = run_step(case)
    check_step(case, out, "bf16")


def test_identity_comb_keeps_streams_bit_exact():
    w = wl.Workload(300, "ident", 48, 512, "bf16")
    case = make_case(w)
    case["comb"] = np.broadcast_to(np.eye(4, dtype=np.float32), (48, 4, 4)).copy()
    case["post"] = np.zeros((48, 4), np.float32)
    out, _ = run_step(case)
    assert torch.equal(out["x_out"], case["x"])
    check_step(case, out, "bf16")


def test_permutation_comb_routes_streams():
    """comb[j, pi(j)] = 1 sends residual stream j to new stream pi(j)."""
    w = wl.Workload(301, "perm", 20, 256, "bf16")
    case = make_case(w)
    pi = [2, 0, 3, 1]
    comb = np.zeros((20, 4, 4), np.float32)
    for j in range(4):
        comb[:, j, pi[j]] = 1.0
    case["comb"] = comb
    case["post"] = np.zeros((20, 4), np.float32)
    out, _ = run_step(case)
    for j in range(4):
        assert torch.equal(out["x_out"][:, pi[j]], case["x"][:, j])


def test_zero_tokens_rows():
    """Tokens whose streams and sublayer output are zero: m = 0, y = 0."""
    w = wl.Workload(302, "zero", 40, 512, "bf16")
    case = make_case(w)
    case["x"][5] = 0
    case["f"][5] = 0
    case["x"][39] = 0
    case["f"][39] = 0
    out, _ = run_step(case)
    check_step(case, out, "bf16")
    assert not out["y"][5].float().abs().max().item()
    assert not out["mix"][39].abs().max().item()


@pytest.mark.parametrize("path", ["tile", "auto"])
def test_in_place_equals_out_of_place(path):
    w = wl.Workload(303, "inplace", 33, 5120, "bf16")
    case = make_case(w)
    ref, dev = run_step(case, path=path)
    x_dev = dev["x"].clone()
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    out = mhc.fused_step(x_dev, dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                         dev["scale"], dev["gamma"], x_out=x_dev, want_mix=True, path=path)
    torch.cuda.synchronize()
    for k in ("x_out", "y", "pre", "post", "comb", "mix"):
        assert torch.equal(out[k].cpu(), ref[k]), k


@pytest.mark.parametrize("path", ["tile", "auto"])
def test_bitwise_deterministic(path):
    w = wl.Workload(304, "det", 70, 5120, "bf16")
    case = make_case(w)
    a, _ = run_step(case, path=path)
    b, _ = run_step(case, path=path)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_guard_bands_untouched():
    """Outputs are views into larger canary-filled buffers: nothing outside the
    views may change, everything inside must be written."""
    w = wl.Workload(305, "guard", 21, 256, "bf16")
    case = make_case(w)
    dev = {k: to_dev(case[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                        "scale", "gamma")}
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    t, d, gpad = 21, 256, 64

    def guarded(n, dtype):
        buf = torch.full((n + 2 * gpad,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[gpad:gpad + n]

    bx, vx = guarded(t * 4 * d, torch.bfloat16)
    by, vy = guarded(t * d, torch.bfloat16)
    bp, vp = guarded(t * 4, torch.float32)
    bu, vu = guarded(t * 4, torch.float32)
    bc, vc = guarded(t * 16, torch.float32)
    bm, vm = guarded(t * 24, torch.float32)
    out = mhc.fused_step(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                         dev["scale"], dev["gamma"], x_out=vx.view(t, 4, d), y_out=vy.view(t, d),
                         pre_out=vp.view(t, 4), post_out=vu.view(t, 4), comb_out=vc.view(t, 4, 4),
                         mix_out=vm.view(t, 24))
    torch.cuda.synchronize()
    for buf, view in ((bx, vx), (by, vy), (bp, vp), (bu, vu), (bc, vc), (bm, vm)):
        assert torch.isnan(buf[:gpad].float()).all() and torch.isnan(buf[-gpad:].float()).all()
        assert not torch.isnan(view.float()).any()
    check_step(case, {k: (v.cpu() if v is not None else None) for k, v in out.items()}, "bf16")


def test_zero_tokens_call_is_a_no_op():
    d = 64
    x = torch.zeros((0, 4, d), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros((0, d), dtype=torch.bfloat16, device="cuda")
    wp = mhc.pack_wmix(torch.zeros((24, 4 * d), device="cuda"), "bf16")
    z = torch.zeros((0, 4), device="cuda")
    out = mhc.fused_step(x, f, z, z, torch.zeros((0, 4, 4), device="cuda"), wp,
                         torch.zeros(24, device="cuda"), torch.ones(3, device="cuda"),
                         torch.ones(d, device="cuda"))
    torch.cuda.synchronize()
    assert out["y"].shape == (0, d)


def test_invalid_arguments_raise():
    d = 64
    x = torch.zeros((4, 4, d), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros((4, d), dtype=torch.bfloat16, device="cuda")
    wp = mhc.pack_wmix(torch.zeros((24, 4 * d), device="cuda"), "bf16")
    z = torch.zeros((4, 4), device="cuda")
    with pytest.raises(mhc.MhcError, match="sinkhorn_iters"):
        mhc.fused_step(x, f, z, z, torch.zeros((4, 4, 4), device="cuda"), wp,
                       torch.zeros(24, device="cuda"), torch.ones(3, device="cuda"),
                       torch.ones(d, device="cuda"), iters=0)

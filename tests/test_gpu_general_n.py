"""GPU parity of the general stream-count family (mhc_*_n, n in {2, 4, 8}).

Every case is checked against the float64 oracle with the rules of
tests/parity.py (new streams as correct roundings, everything after them
teacher-forced on the validated new streams). Both kernels of the family
are covered: the token-block kernel (path "block", every n and dtype), the
feature-split kernel (path "split", n = 2 and 4, bf16, slices of 64,
128 and 256 features) and the block kernel in chunks of the features (path
"chunk", every n and dtype, up to 8192 tokens). Cases cover n = 2, 4, 8, bf16
and f32 streams, widths from one 32-feature step to d = 5120, odd step counts,
token counts from one token to several 128-token blocks with a ragged last
block, in-place updates, guard bands around every output, and, at n = 4,
agreement with the tuned n = 4 kernels (same per-element arithmetic, so the
new streams must match bit for bit). The largest case runs n = 8 at the
throughput shape (65,536 tokens, d = 5120) exactly as the benchmark launches
it, with sampled tokens checked in full.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, oracle_prior, run_step, to_dev
from tests.conftest import load_golden
from tests.parity import check_comb, check_mix_like, check_mixes, check_step, comb_sum_stats

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _dev(case):
    return {k: to_dev(case[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                         "scale", "gamma")}


def run_step_n(case, dtype, **kw):
    dev = _dev(case)
    wp = mhc.pack_wmix_n(dev["w_mix"], dtype)
    out = mhc.fused_step_n(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp,
                           dev["base"], dev["scale"], dev["gamma"], case["iters"],
                           case["norm_eps"], case["hc_eps"], **kw)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}, dev


CASES = [
    # n, dtype, d, tokens
    (2, "bf16", 5120, 300),
    (2, "bf16", 256, 129),
    (2, "f32", 64, 17),
    (4, "bf16", 5120, 257),
    (4, "bf16", 2080, 100),     # 65 steps: odd count
    (4, "f32", 96, 33),
    (8, "bf16", 5120, 200),
    (8, "bf16", 32, 130),       # a single step
    (8, "bf16", 1024, 1),       # one token: one lane of one wave works
    (8, "f32", 128, 40),
]


@pytest.mark.parametrize("n,dtype,d,t", CASES)
def test_general_n_parity(n, dtype, d, t):
    """The token-block kernel (path "block")."""
    _log(f"general n={n} {dtype} d={d} T={t}")
    case = make_case(wl.Workload(700 + 10 * n + d % 7 + t % 5, "general_n", t, d, dtype, n=n))
    out, _ = run_step_n(case, dtype, path="block")
    o = check_step(case, out, dtype)
    _log(f"  ties in new streams: {o['n_ties']}; comb sums {comb_sum_stats(out['comb'])}")


SPLIT_CASES = [
    # n, d, tokens: slices of 64 * rounds features, 16 to 40 slices
    (2, 5120, 300),     # 20 slices of 256 (4 rounds)
    (2, 5120, 1),       # one token
    (2, 4096, 1000),    # 16 slices of 256
    (2, 2048, 129),     # 16 slices of 128
    (2, 1024, 70),      # 16 slices of 64
    (4, 5120, 257),     # 40 slices of 128
    (4, 3072, 600),     # 24 slices of 128
    (4, 2048, 130),     # 16 slices of 128
    (4, 1024, 33),      # 16 slices of 64
]


@pytest.mark.parametrize("n,d,t", SPLIT_CASES)
def test_general_n_split_parity(n, d, t):
    """The feature-split kernel of the n-family (path "split"), and the new
    streams identical to the block kernel's (same per-element arithmetic)."""
    _log(f"general split n={n} d={d} T={t}")
    case = make_case(wl.Workload(800 + 10 * n + d % 7 + t % 5, "general_n_split", t, d, "bf16",
                                 n=n))
    ws = torch.zeros(mhc.fused_step_n_workspace_bytes(n, t, d, "bf16"), dtype=torch.uint8,
                     device="cuda")
    out, _ = run_step_n(case, "bf16", path="split", workspace=ws)
    assert mhc.split_status(ws) == 0
    o = check_step(case, out, "bf16")
    blk, _ = run_step_n(case, "bf16", path="block")
    assert torch.equal(out["x_out"], blk["x_out"])
    np.testing.assert_allclose(out["mix"].numpy(), blk["mix"].numpy(), rtol=1e-5, atol=2e-5)
    _log(f"  ties in new streams: {o['n_ties']}; comb sums {comb_sum_stats(out['comb'])}")


@pytest.mark.parametrize("n,d,t", [(2, 5120, 3000), (4, 2048, 700)])
def test_general_n_split_cooperative_launch(n, d, t):
    """MHC_PATH_COOPERATIVE on the n-family's feature-split kernel: the
    ordinary launch's bits, every wait completed, the header zero again, and
    the oracle on every token."""
    case = make_case(wl.Workload(840 + n + t % 7, "general_n_plain", t, d, "bf16", n=n))
    ws = mhc.new_workspace(mhc.fused_step_n_workspace_bytes(n, t, d, "bf16"))
    ref, _ = run_step_n(case, "bf16", path="split", workspace=ws)
    out, _ = run_step_n(case, "bf16", path="split", workspace=ws, cooperative=True)
    assert mhc.split_status(ws) == 0
    assert ws[:16384].count_nonzero().item() == 0
    for k in ref:
        assert torch.equal(out[k], ref[k]), k
    check_step(case, out, "bf16")


CHUNK_CASES = [
    # n, dtype, d, tokens
    (2, "bf16", 5120, 300),     # 80 units of 64 features: one per chunk
    (2, "f32", 64, 17),         # 2 units of 32
    (2, "bf16", 2048, 2048),
    (4, "bf16", 5120, 257),
    (4, "bf16", 2080, 100),     # 65 steps: odd count, units of 32 features
    (4, "bf16", 6400, 5),       # 100 units of 64: 2 per chunk, 50 chunks
    (4, "f32", 96, 33),
    (8, "bf16", 5120, 200),     # 160 units of 32: 2 per chunk
    (8, "bf16", 32, 130),       # a single step
    (8, "bf16", 1024, 1),       # one token
    (8, "bf16", 224, 10),       # 7 units
    (8, "f32", 128, 40),
    (8, "bf16", 1024, 8192),    # the largest chunked call
]


@pytest.mark.parametrize("n,dtype,d,t", CHUNK_CASES)
def test_general_n_chunk_parity(n, dtype, d, t):
    """The chunked block kernel (path "chunk"): parity with the oracle, and
    the new streams identical to the block kernel's (same per-element
    arithmetic)."""
    _log(f"general chunk n={n} {dtype} d={d} T={t}")
    case = make_case(wl.Workload(900 + 10 * n + d % 7 + t % 5, "general_n_chunk", t, d, dtype,
                                 n=n))
    assert mhc.fused_step_route_n(n, "chunk", t, d, dtype) == "chunk"
    ws = torch.zeros(mhc.fused_step_n_workspace_bytes(n, t, d, dtype), dtype=torch.uint8,
                     device="cuda")
    out, _ = run_step_n(case, dtype, path="chunk", workspace=ws)
    o = check_step(case, out, dtype)
    blk, _ = run_step_n(case, dtype, path="block")
    assert torch.equal(out["x_out"], blk["x_out"])
    np.testing.assert_allclose(out["mix"].numpy(), blk["mix"].numpy(), rtol=1e-5, atol=2e-5)
    _log(f"  ties in new streams: {o['n_ties']}; comb sums {comb_sum_stats(out['comb'])}")


@pytest.mark.parametrize("n,dtype,d,t", [(8, "bf16", 2048, 300), (2, "f32", 64, 129),
                                         (4, "bf16", 5120, 1000)])
def test_mixes_n_chunk_parity(n, dtype, d, t):
    w = wl.Workload(940 + n, "mixes_n_chunk", t, d, dtype, n=n)
    x = wl.streams(w)
    p = wl.params(w)
    out = mhc.mixes_n(to_dev(x), mhc.pack_wmix_n(to_dev(p["w_mix"]), dtype), to_dev(p["base"]),
                      to_dev(p["scale"]), path="chunk")
    torch.cuda.synchronize()
    check_mixes(dict(x=x, **p), {k: v.cpu() for k, v in out.items()}, dtype)


def test_general_n_chunk_workspace_reused_for_a_smaller_call():
    """One workspace, two calls in a row, the second with fewer tokens (the
    partial rows are laid out by the call's own token count)."""
    n, d = 8, 1024
    ws = torch.zeros(mhc.fused_step_n_workspace_bytes(n, 500, d, "bf16"), dtype=torch.uint8,
                     device="cuda")
    for t in (500, 77):
        case = make_case(wl.Workload(960 + t, "general_n_chunk_reuse", t, d, "bf16", n=n))
        out, _ = run_step_n(case, "bf16", path="chunk", workspace=ws)
        check_step(case, out, "bf16")


def test_general_n_split_guard_bands_and_in_place():
    """n = 2, d = 1024 (16 slices of 64) through the split kernel: nothing is
    written outside the outputs, and x_out = x gives the same results."""
    n, t, d, gpad = 2, 150, 1024, 64
    case = make_case(wl.Workload(820, "general_n_split_guard", t, d, "bf16", n=n))
    dev = _dev(case)
    wp = mhc.pack_wmix_n(dev["w_mix"], "bf16")

    def guarded(count, dtype):
        buf = torch.full((count + 2 * gpad,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[gpad:gpad + count]

    nm = (2 + n) * n
    bx, vx = guarded(t * n * d, torch.bfloat16)
    by, vy = guarded(t * d, torch.bfloat16)
    bp, vp = guarded(t * n, torch.float32)
    bu, vu = guarded(t * n, torch.float32)
    bc, vc = guarded(t * n * n, torch.float32)
    bm, vm = guarded(t * nm, torch.float32)
    out = mhc.fused_step_n(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp,
                           dev["base"], dev["scale"], dev["gamma"], x_out=vx.view(t, n, d),
                           y_out=vy.view(t, d), pre_out=vp.view(t, n), post_out=vu.view(t, n),
                           comb_out=vc.view(t, n, n), mix_out=vm.view(t, nm), path="split")
    torch.cuda.synchronize()
    for buf, view in ((bx, vx), (by, vy), (bp, vp), (bu, vu), (bc, vc), (bm, vm)):
        assert torch.isnan(buf[:gpad].float()).all() and torch.isnan(buf[-gpad:].float()).all()
        assert not torch.isnan(view.float()).any()
    ref = {k: v.cpu() for k, v in out.items()}
    check_step(case, ref, "bf16")
    x = dev["x"].clone()
    again = mhc.fused_step_n(x, dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                             dev["scale"], dev["gamma"], x_out=x, path="split")
    torch.cuda.synchronize()
    for k in ("x_out", "y", "pre", "post", "comb", "mix"):
        assert torch.equal(again[k].cpu(), ref[k]), k


@pytest.mark.parametrize("n,d,t", [(2, 5120, 700), (4, 2048, 260)])
def test_mixes_n_split_parity(n, d, t):
    w = wl.Workload(830 + n, "mixes_n_split", t, d, "bf16", n=n)
    x = wl.streams(w)
    p = wl.params(w)
    out = mhc.mixes_n(to_dev(x), mhc.pack_wmix_n(to_dev(p["w_mix"]), "bf16"), to_dev(p["base"]),
                      to_dev(p["scale"]), path="split")
    torch.cuda.synchronize()
    check_mixes(dict(x=x, **p), {k: v.cpu() for k, v in out.items()}, "bf16")


def test_one_workspace_serves_every_route_in_turn():
    """One zero-filled workspace shared, in turn, by the backward, the chunked
    route and feature-split calls with 16, 6 and 12 groups (fused and
    mixes-only): each route leaves the header (status, abort and done words,
    the group counters) zero for the next, and keeps its own data out of it,
    so every forward result matches the oracle."""
    calls = [  # n, d, tokens, path, mixes only
        (2, 1024, 150, "split", False),    # 16 slices of 64: 16 groups
        (4, 5120, 300, "split", False),    # 40 slices of 128: 6 groups
        (2, 5120, 700, "split", True),     # 20 slices of 256: 12 groups
        (4, 5120, 200, "chunk", False),
        (2, 1024, 150, "split", True),
    ]
    need = max(mhc.fused_step_n_workspace_bytes(n, t, d, "bf16") for n, d, t, _, _ in calls)
    need = max(need, mhc.fused_step_backward_workspace_bytes_n(4, 64, 1024))
    ws = mhc.new_workspace(need)
    # a backward call first: its regions lie after the header
    bc = make_case(wl.Workload(841, "ws_backward", 64, 1024, "bf16", n=4))
    bo, bdev = run_step_n(bc, "bf16", path="block")
    g = torch.Generator(device="cuda").manual_seed(5)
    mhc.fused_step_backward_n(
        bdev["x"], bdev["f"], bdev["pre"], bdev["post"], bdev["comb"], bo["x_out"].cuda(),
        bo["mix"].cuda(), bdev["w_mix"], bdev["base"], bdev["scale"], bdev["gamma"],
        torch.randn(bdev["x"].shape, device="cuda", generator=g).bfloat16(),
        torch.randn(bdev["f"].shape, device="cuda", generator=g).bfloat16(),
        torch.randn((64, 4), device="cuda", generator=g),
        torch.randn((64, 4), device="cuda", generator=g),
        torch.randn((64, 4, 4), device="cuda", generator=g), workspace=ws)
    torch.cuda.synchronize()
    for i, (n, d, t, path, mixes_only) in enumerate(calls):
        case = make_case(wl.Workload(842 + i, "ws_shared", t, d, "bf16", n=n))
        if mixes_only:
            dev = _dev(case)
            out = mhc.mixes_n(dev["x"], mhc.pack_wmix_n(dev["w_mix"], "bf16"), dev["base"],
                              dev["scale"], path=path, workspace=ws)
            torch.cuda.synchronize()
            check_mixes(case, {k: v.cpu() for k, v in out.items()}, "bf16")
        else:
            out, _ = run_step_n(case, "bf16", path=path, workspace=ws)
            check_step(case, out, "bf16")
        assert mhc.split_status(ws) == 0
        words = ws[:16384].view(torch.int32)
        assert int(words[1:3].abs().sum().item()) == 0
        assert int(words[64:].abs().sum().item()) == 0   # counters (bytes 256 on) are zero
        _log(f"shared workspace: n={n} d={d} T={t} {path}{' mixes' if mixes_only else ''} ok")


@pytest.mark.timeout(900)
def test_general_n2_throughput_shape_sampled():
    """n = 2 at 65,536 tokens x d = 5120 through the feature-split kernel, as
    the benchmark launches it; first and last blocks plus a seeded random
    sample of tokens checked in full."""
    w = wl.Workload(3, "large_prefill_n2", 65536, 5120, "bf16", batch=4, n=2)
    t_start = time.time()
    x = wl.streams(w)
    f = wl.sublayer_out(w)
    prev, cur = wl.params(w, prev=True), wl.params(w)
    pre, post, comb = oracle_prior(x, prev)
    _log(f"n2 large: inputs and oracle prior in {time.time() - t_start:.1f}s")
    case = dict(x=x, f=f, pre=pre, post=post, comb=comb, iters=w.iters, norm_eps=w.norm_eps,
                hc_eps=w.hc_eps, **cur)
    out, _ = run_step_n(case, "bf16", path="split")
    t = w.tokens
    rng = np.random.default_rng(12345)
    idx = np.unique(np.concatenate([np.arange(128), np.arange(t - 128, t),
                                    rng.choice(t, 256, replace=False)]))
    sub = dict(case)
    for k in ("x", "f", "pre", "post", "comb"):
        sub[k] = case[k][idx]
    check_step(sub, {k: v[idx] for k, v in out.items()}, "bf16")
    _log(f"n2 large: {len(idx)} sampled tokens match; comb sums {comb_sum_stats(out['comb'])}")


@pytest.mark.parametrize("npath", ["block", "split", "chunk"])
def test_general_n4_matches_tuned_kernels(npath):
    case = make_case(wl.Workload(760, "general_n4", 700, 5120, "bf16"))
    a, _ = run_step_n(case, "bf16", path=npath)
    for path in ("split", "tile"):
        b, _ = run_step(case, path=path)
        assert torch.equal(a["x_out"], b["x_out"]), path
        ya, yb = a["y"].float(), b["y"].float()
        assert ((ya - yb).abs() <= torch.maximum(ya.abs(), yb.abs()) * 2.0 ** -7 + 1e-30).all()
        # the mixes are summed in another order (|m| up to ~10 here)
        for k in ("pre", "post", "comb", "mix"):
            np.testing.assert_allclose(a[k].numpy(), b[k].numpy(), rtol=1e-5, atol=2e-5)


@pytest.mark.parametrize("n,dtype,d,t", [(2, "bf16", 5120, 1000), (8, "bf16", 2048, 300),
                                         (8, "f32", 64, 129)])
def test_mixes_n_parity(n, dtype, d, t):
    w = wl.Workload(770 + n, "mixes_n", t, d, dtype, n=n)
    x = wl.streams(w)
    p = wl.params(w)
    out = mhc.mixes_n(to_dev(x), mhc.pack_wmix_n(to_dev(p["w_mix"]), dtype), to_dev(p["base"]),
                      to_dev(p["scale"]))
    torch.cuda.synchronize()
    check_mixes(dict(x=x, **p), {k: v.cpu() for k, v in out.items()}, dtype)


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("iters", [1, 2, 20])
def test_sinkhorn_n_parity(n, iters):
    rng = np.random.default_rng(780 + n + iters)
    nm = (2 + n) * n
    m = rng.normal(0, 3.0, (517, nm)).astype(np.float32)
    base = rng.normal(0, 0.1, nm).astype(np.float32)
    scale = rng.uniform(0.5, 2.0, 3).astype(np.float32)
    out = mhc.sinkhorn_n(n, to_dev(m), to_dev(base), to_dev(scale), iters, 1e-6)
    torch.cuda.synchronize()
    pre, post, comb = oracle.split_sinkhorn(m, scale, base, iters, 1e-6, n)
    check_mix_like("pre", out["pre"].cpu(), pre)
    check_mix_like("post", out["post"].cpu(), post)
    check_comb(out["comb"].cpu(), comb, 1e-6, iters)


@pytest.mark.parametrize("n", [4, 8])
def test_sinkhorn_n_worked_example(n):
    """The course page's hand-checked 2x2 example ("2A · Single-Pass mHC", §4)
    through A (x) J_b (b = n/2) with logits log of it, base 0, scale 1, eps 0:
    after one and two rounds the blocks are the printed matrices divided by b."""
    from fractions import Fraction
    g = load_golden("sinkhorn_2x2_worked_example.txt")

    def mat(key):
        return np.array([float(Fraction(v)) for v in g[key]]).reshape(2, 2)

    b = n // 2
    big = np.kron(mat("input"), np.ones((b, b)))
    nm = (2 + n) * n
    m = np.zeros((1, nm), np.float32)
    m[0, 2 * n:] = np.log(big).reshape(-1)
    for iters, key in ((1, "round1"), (2, "round2")):
        out = mhc.sinkhorn_n(n, to_dev(m), to_dev(np.zeros(nm, np.float32)),
                             to_dev(np.ones(3, np.float32)), iters, 0.0)
        torch.cuda.synchronize()
        want = np.kron(mat(key), np.ones((b, b)) / b)
        np.testing.assert_allclose(out["comb"].cpu().numpy()[0], want, rtol=0, atol=2e-7)


def test_sinkhorn_n2_eps_quarter_hand_worked():
    """The split kernel's schedule at n = 2 with eps = 1/4 ("Stream weights for
    the feed-forward", Code, the split/Sinkhorn kernel), against fractions
    worked by hand: every eps placement changes them."""
    from fractions import Fraction
    g = load_golden("sinkhorn_2x2_eps_quarter.txt")

    def vals(key):
        return np.array([float(Fraction(v)) for v in g[key]])

    l3 = np.log(3.0)
    m = np.zeros((1, 8), np.float32)
    m[0, 0:4] = [l3, -l3, -l3, l3]
    m[0, 4:8] = np.log(vals("input"))
    eps = float(g["eps"])
    for iters, key in ((1, "round1"), (2, "round2")):
        out = mhc.sinkhorn_n(2, to_dev(m), to_dev(np.zeros(8, np.float32)),
                             to_dev(np.ones(3, np.float32)), iters, eps)
        torch.cuda.synchronize()
        np.testing.assert_allclose(out["comb"].cpu().numpy()[0].reshape(-1), vals(key),
                                   rtol=0, atol=3e-7)
        np.testing.assert_allclose(out["pre"].cpu().numpy()[0], vals("pre"), rtol=0, atol=3e-7)
        np.testing.assert_allclose(out["post"].cpu().numpy()[0], vals("post"), rtol=0, atol=3e-7)


@pytest.mark.parametrize("path", ["block", "chunk"])
def test_general_n_in_place_and_repeatable(path):
    case = make_case(wl.Workload(790, "general_n_inplace", 300, 1024, "bf16", n=8))
    ref, dev = run_step_n(case, "bf16", path=path)
    again, _ = run_step_n(case, "bf16", path=path)
    for k in ref:
        assert torch.equal(ref[k], again[k]), k
    x = dev["x"].clone()
    wp = mhc.pack_wmix_n(dev["w_mix"], "bf16")
    out = mhc.fused_step_n(x, dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                           dev["scale"], dev["gamma"], x_out=x, path=path)
    torch.cuda.synchronize()
    for k in ("x_out", "y", "pre", "post", "comb", "mix"):
        assert torch.equal(out[k].cpu(), ref[k]), k


@pytest.mark.parametrize("path", ["block", "chunk"])
@pytest.mark.parametrize("n", [2, 8])
def test_general_n_guard_bands_untouched(n, path):
    t, d, gpad = 21, 256, 64
    case = make_case(wl.Workload(795 + n, "general_n_guard", t, d, "bf16", n=n))
    dev = _dev(case)
    wp = mhc.pack_wmix_n(dev["w_mix"], "bf16")

    def guarded(count, dtype):
        buf = torch.full((count + 2 * gpad,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[gpad:gpad + count]

    nm = (2 + n) * n
    bx, vx = guarded(t * n * d, torch.bfloat16)
    by, vy = guarded(t * d, torch.bfloat16)
    bp, vp = guarded(t * n, torch.float32)
    bu, vu = guarded(t * n, torch.float32)
    bc, vc = guarded(t * n * n, torch.float32)
    bm, vm = guarded(t * nm, torch.float32)
    out = mhc.fused_step_n(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp,
                           dev["base"], dev["scale"], dev["gamma"], x_out=vx.view(t, n, d),
                           y_out=vy.view(t, d), pre_out=vp.view(t, n), post_out=vu.view(t, n),
                           comb_out=vc.view(t, n, n), mix_out=vm.view(t, nm), path=path)
    torch.cuda.synchronize()
    for buf, view in ((bx, vx), (by, vy), (bp, vp), (bu, vu), (bc, vc), (bm, vm)):
        assert torch.isnan(buf[:gpad].float()).all() and torch.isnan(buf[-gpad:].float()).all()
        assert not torch.isnan(view.float()).any()
    check_step(case, {k: v.cpu() for k, v in out.items()}, "bf16")


def test_general_n_zero_tokens():
    x = torch.zeros((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros((0, 8), device="cuda")
    wp = mhc.pack_wmix_n(torch.zeros((80, 8 * 64), device="cuda"), "bf16")
    out = mhc.fused_step_n(x, f, z, z, torch.zeros((0, 8, 8), device="cuda"), wp,
                           torch.zeros(80, device="cuda"), torch.ones(3, device="cuda"),
                           torch.ones(64, device="cuda"))
    torch.cuda.synchronize()
    assert out["y"].shape == (0, 64)


@pytest.mark.timeout(900)
def test_general_n8_throughput_shape_sampled():
    """n = 8 at 65,536 tokens x d = 5120, launched as the benchmark launches it
    (prior coefficients from the oracle on the CPU); first and last blocks plus
    a seeded random sample of tokens checked in full."""
    w = wl.Workload(3, "large_prefill_n8", 65536, 5120, "bf16", batch=4, n=8)
    t_start = time.time()
    x = wl.streams(w)
    f = wl.sublayer_out(w)
    prev, cur = wl.params(w, prev=True), wl.params(w)
    _log(f"n8 large: inputs drawn in {time.time() - t_start:.1f}s")
    pre, post, comb = oracle_prior(x, prev)
    _log(f"n8 large: oracle prior done at {time.time() - t_start:.1f}s")
    case = dict(x=x, f=f, pre=pre, post=post, comb=comb, iters=w.iters, norm_eps=w.norm_eps,
                hc_eps=w.hc_eps, **cur)
    out, _ = run_step_n(case, "bf16")
    _log(f"n8 large: GPU step done at {time.time() - t_start:.1f}s")
    t = w.tokens
    rng = np.random.default_rng(54321)
    idx = np.unique(np.concatenate([np.arange(128), np.arange(t - 128, t),
                                    rng.choice(t, 256, replace=False)]))
    sub = dict(case)
    for k in ("x", "f", "pre", "post", "comb"):
        sub[k] = case[k][idx]
    check_step(sub, {k: v[idx] for k, v in out.items()}, "bf16")
    stats = comb_sum_stats(out["comb"])
    assert stats["col_dev_max"] <= 1e-5
    _log(f"n8 large: {len(idx)} sampled tokens match; comb sums {stats}")


@pytest.mark.parametrize("n,path", [(8, "chunk"), (2, "chunk"), (4, "split"), (8, "block")])
def test_general_n_replays_from_a_hip_graph(n, path):
    """Every route of the n-family sets no memory from the host: a call
    captured into a graph replays to the eager result, with eager work and
    synchronisation between the replays, and the replays follow new inputs
    copied into the captured buffers."""
    t, d = 256, 1024
    _log(f"general graph n={n} path={path}")
    cases = [make_case(wl.Workload(980 + 10 * n + i, "general_n_graph", t, d, "bf16", n=n))
             for i in range(2)]
    dev = _dev(cases[0])
    wp = mhc.pack_wmix_n(dev["w_mix"], "bf16")
    ws = torch.zeros(max(mhc.fused_step_n_workspace_bytes(n, t, d, "bf16"), 256),
                     dtype=torch.uint8, device="cuda")
    nm = (2 + n) * n
    outs = dict(x_out=torch.empty_like(dev["x"]), y_out=torch.empty_like(dev["f"]),
                pre_out=torch.empty((t, n), device="cuda"),
                post_out=torch.empty((t, n), device="cuda"),
                comb_out=torch.empty((t, n, n), device="cuda"),
                mix_out=torch.empty((t, nm), device="cuda"))

    def call():
        mhc.fused_step_n(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp,
                         dev["base"], dev["scale"], dev["gamma"], cases[0]["iters"],
                         cases[0]["norm_eps"], cases[0]["hc_eps"], path=path, workspace=ws,
                         **outs)

    def snapshot():
        return {k: v.clone() for k, v in outs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in (0, 1, 0):
        for k in ("x", "f", "pre", "post", "comb"):
            dev[k].copy_(to_dev(cases[i][k]))
        torch.cuda.synchronize()
        for o in outs.values():
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        call()                                              # the eager reference
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for k, v in snapshot().items():
            assert torch.equal(got[k], v), (i, k)
        ref = dict(cases[0])   # the captured parameters, case i's streams and coefficients
        ref.update({k: cases[i][k] for k in ("x", "f", "pre", "post", "comb")})
        check_step(ref, {"x_out": got["x_out"].cpu(), "y": got["y_out"].cpu(),
                         "pre": got["pre_out"].cpu(), "post": got["post_out"].cpu(),
                         "comb": got["comb_out"].cpu(), "mix": got["mix_out"].cpu()}, "bf16")

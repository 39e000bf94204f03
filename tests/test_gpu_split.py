"""GPU parity of the feature-split fused-step kernel (path="split").

Each compute unit owns one slice of the features; workgroups exchange per-token
partial sums through a workspace ring. The cases cover every slice geometry the
host picks on a 256-CU device (32, 40, 48 and 64 slices of 64, 96, 128 or
160 features), token counts from one token
to enough batches that every exchange slot is reused several times, ragged
batches, in-place updates, guard bands, repeated calls on one workspace, and
agreement with the tile kernel (the new streams must match bit for bit: their
arithmetic is the same; y and the coefficients differ only in summation
order). Every call's status word must read 0 (no wait gave up).
"""

import numpy as np
import pytest
import torch

import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, run_step, to_dev
from tests.parity import check_mix_like, check_step

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _run(case, **kw):
    ws = torch.zeros(mhc.fused_step_workspace_bytes(len(case["x"]), case["x"].shape[2], "bf16"),
                     dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    out, dev = run_step(case, path="split", workspace=ws, **kw)
    assert mhc.split_status(ws) == 0, "a cross-workgroup wait gave up"
    return out, dev


# slice geometry on a 256-CU device: calls of more than 40 batches of 128
# tokens take 256-feature slices on the two-term projection where d allows
# (d = 4096: 16, 5120: 20, 6144: 24 slices), else 128-byte aligned slices
# (8192 -> 64 x 128, 3072 -> 48 x 64, 2048 -> 32 x 64, 2560 -> 40 x 64) or,
# with no aligned choice, the 32-feature tail (3840 -> 40 x 96, 6400 -> 40 x
# 160); smaller calls take the geometry with the least estimated time (at
# d = 5120 32 x 160 on all 256 CUs). The tokens after the last whole round
# are shared out over the groups, so every size below exercises it
SPLIT_CASES = [
    (5120, 1),       # one token: one wave of one group works
    (5120, 37),      # ragged first batch
    (5120, 128),     # exactly one batch
    (5120, 1000),    # fewer batches than groups for some groups
    (5120, 4133),    # every group, ring not yet wrapped, ragged
    (5120, 9000),    # ring slots reused, ragged last batch
    (4096, 300),
    (3072, 257),
    (2048, 513),
    (2560, 130),
    (6144, 700),
    (8192, 260),
    (3840, 300),     # 40 x 96: one round + a 32-feature tail
    (6400, 200),     # 40 x 160: two rounds + tail
]


@pytest.mark.parametrize("d,t", SPLIT_CASES)
def test_split_parity(d, t):
    _log(f"split d={d} T={t}")
    w = wl.Workload(400 + d % 89 + t % 7, "split", t, d, "bf16")
    case = make_case(w)
    out, _ = _run(case)
    o = check_step(case, out, "bf16")
    _log(f"  ties in new streams: {o['n_ties']}")


@pytest.mark.parametrize("t", [700, 6000])   # 40 slices of 128 features; 20 of 256
def test_split_matches_tile_kernel(t):
    w = wl.Workload(450, "split_vs_tile", t, 5120, "bf16")
    case = make_case(w)
    a, _ = _run(case)
    b, _ = run_step(case, path="tile")
    assert torch.equal(a["x_out"], b["x_out"])
    ya, yb = a["y"].float(), b["y"].float()
    ulp = torch.maximum(ya.abs(), yb.abs()) * 2.0 ** -7 + 1e-30
    assert ((ya - yb).abs() <= ulp).all()
    # y and the coefficients differ in summation order and, on 256-feature
    # slices, in the projection's terms (hi + mid against hi + mid + lo of W)
    for k in ("pre", "post", "comb", "mix"):
        check_mix_like(k, a[k], b[k])


def test_split_in_place_and_deterministic():
    w = wl.Workload(451, "split_inplace", 555, 5120, "bf16")
    case = make_case(w)
    ref, dev = _run(case)
    again, _ = _run(case)
    for k in ref:
        if ref[k] is not None:
            assert torch.equal(ref[k], again[k]), k
    x_dev = dev["x"].clone()
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    ws = torch.zeros(mhc.fused_step_workspace_bytes(555, 5120, "bf16"), dtype=torch.uint8,
                     device="cuda")
    out = mhc.fused_step(x_dev, dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                         dev["scale"], dev["gamma"], x_out=x_dev, want_mix=True, path="split",
                         workspace=ws)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    for k in ("x_out", "y", "pre", "post", "comb", "mix"):
        assert torch.equal(out[k].cpu(), ref[k]), k


def test_split_guard_bands_untouched():
    t, d, gpad = 21, 2048, 64
    w = wl.Workload(452, "split_guard", t, d, "bf16")
    case = make_case(w)
    dev = {k: to_dev(case[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                        "scale", "gamma")}
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")

    def guarded(n, dtype):
        buf = torch.full((n + 2 * gpad,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[gpad:gpad + n]

    bx, vx = guarded(t * 4 * d, torch.bfloat16)
    by, vy = guarded(t * d, torch.bfloat16)
    bp, vp = guarded(t * 4, torch.float32)
    bu, vu = guarded(t * 4, torch.float32)
    bc, vc = guarded(t * 16, torch.float32)
    bm, vm = guarded(t * 24, torch.float32)
    ws = torch.zeros(mhc.fused_step_workspace_bytes(t, d, "bf16"), dtype=torch.uint8,
                     device="cuda")
    out = mhc.fused_step(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                         dev["scale"], dev["gamma"], x_out=vx.view(t, 4, d), y_out=vy.view(t, d),
                         pre_out=vp.view(t, 4), post_out=vu.view(t, 4), comb_out=vc.view(t, 4, 4),
                         mix_out=vm.view(t, 24), path="split", workspace=ws)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    for buf, view in ((bx, vx), (by, vy), (bp, vp), (bu, vu), (bc, vc), (bm, vm)):
        assert torch.isnan(buf[:gpad].float()).all() and torch.isnan(buf[-gpad:].float()).all()
        assert not torch.isnan(view.float()).any()
    check_step(case, {k: (v.cpu() if v is not None else None) for k, v in out.items()}, "bf16")


def test_split_repeated_calls_share_a_workspace():
    """Two calls in a row on one zero-filled workspace, the second smaller: each
    call leaves the header's counters as it found them, with no clearing
    launch in between."""
    ws = torch.zeros(mhc.fused_step_workspace_bytes(3000, 5120, "bf16"), dtype=torch.uint8,
                     device="cuda")
    for t, seed in ((3000, 453), (200, 454)):
        case = make_case(wl.Workload(seed, "split_repeat", t, 5120, "bf16"))
        out, _ = run_step(case, path="split", workspace=ws)
        assert mhc.split_status(ws) == 0
        check_step(case, out, "bf16")


@pytest.mark.parametrize("t", [1000, 6000])   # 32 slices of 160 features; 20 of 256
def test_split_leaves_the_header_zero(t):
    """After a feature-split call the status word, the abort word, the done
    count, the start-order ticket count (bytes 0, 4, 8, 12) and every (group,
    slot) counter (from byte 256) are back to zero: the whole 16 KB header."""
    ws = mhc.new_workspace(mhc.fused_step_workspace_bytes(t, 5120, "bf16"))
    case = make_case(wl.Workload(455, "split_header", t, 5120, "bf16"))
    out, _ = run_step(case, path="split", workspace=ws)
    words = ws[:16384].view(torch.int32).cpu().numpy()
    assert (words[:4] == 0).all(), words[:4]
    assert (words == 0).all(), np.flatnonzero(words)[:8]
    check_step(case, out, "bf16")


def test_split_status_word_is_sticky():
    """The library never clears the status word: a value written there stays
    across calls (whose outputs are unaffected, since the waits read the
    call's own abort word), check_status reports it, and clear_split_status
    resets it. The word is set from the host; no wait is made to give up."""
    t = 300
    ws = mhc.new_workspace(mhc.fused_step_workspace_bytes(t, 5120, "bf16"))
    case = make_case(wl.Workload(456, "split_sticky", t, 5120, "bf16"))
    ws[:4].view(torch.int32).fill_(1)
    out, _ = run_step(case, path="split", workspace=ws)
    assert mhc.split_status(ws) == 1
    check_step(case, out, "bf16")
    with pytest.raises(mhc.MhcError, match="gave up"):
        run_step(case, path="split", workspace=ws, check_status=True)
    assert mhc.split_status(ws) == 0
    out, _ = run_step(case, path="split", workspace=ws, check_status=True)
    check_step(case, out, "bf16")


def test_split_workspace_validation():
    t, d = 64, 2048
    x = torch.zeros((t, 4, d), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros((t, d), dtype=torch.bfloat16, device="cuda")
    wp = mhc.pack_wmix(torch.zeros((24, 4 * d), device="cuda"), "bf16")
    z = torch.zeros((t, 4), device="cuda")
    need = mhc.fused_step_workspace_bytes(t, d, "bf16")
    args = (x, f, z, z, torch.zeros((t, 4, 4), device="cuda"), wp, torch.zeros(24, device="cuda"),
            torch.ones(3, device="cuda"), torch.ones(d, device="cuda"))
    small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mhc.MhcError, match="workspace holds"):
        mhc.fused_step(*args, path="split", workspace=small)
    big = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(mhc.MhcError, match="256-byte aligned"):
        mhc.fused_step(*args, path="split", workspace=big[16:])
    # f32 streams: only the chunked kernels (chunks of 8 steps) take a workspace
    assert mhc.fused_step_workspace_bytes(t, 5120, "f32") == 16384 + 20 * t * 128
    assert mhc.fused_step_workspace_bytes(t, 7168, "bf16") == 0
    # d = 1024 has no slice geometry: only the chunked kernels take a workspace
    assert mhc.fused_step_workspace_bytes(t, 1024, "bf16") == 16384 + 2 * t * 128
    with pytest.raises(ValueError, match="does not apply"):
        mhc.fused_step_route("split", t, 1024, "bf16")
    assert mhc.fused_step_route("auto", t, 1024, "bf16") == "chunk"


@pytest.mark.parametrize("cooperative", [False, True])
def test_split_calls_on_two_streams_in_flight_together(cooperative):
    """Two feature-split calls issued on two streams before either is waited
    for (each with its own workspace). Ordinary launches may share the device:
    their groups are filled in start order, so each call's running groups
    finish and free compute units for the rest; cooperative launches run one
    at a time. Either way both complete (status word 0) and match the same
    calls run one after the other, bit for bit."""
    t, d = 9000, 5120
    cases = [make_case(wl.Workload(460 + i, "split_streams", t, d, "bf16")) for i in range(2)]
    devs = [{k: to_dev(c[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                       "scale", "gamma")} for c in cases]
    wps = [mhc.pack_wmix(dv["w_mix"], "bf16") for dv in devs]
    wss = [torch.zeros(mhc.fused_step_workspace_bytes(t, d, "bf16"), dtype=torch.uint8,
                       device="cuda") for _ in range(2)]

    def call(i):
        dv = devs[i]
        return mhc.fused_step(dv["x"], dv["f"], dv["pre"], dv["post"], dv["comb"], wps[i],
                              dv["base"], dv["scale"], dv["gamma"], want_mix=True,
                              path="split", workspace=wss[i], cooperative=cooperative)

    ref = []
    for i in range(2):
        ref.append({k: v.clone() for k, v in call(i).items()})
        torch.cuda.synchronize()
        assert mhc.split_status(wss[i]) == 0
    streams = [torch.cuda.Stream() for _ in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):                      # a few rounds of overlapping pairs
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                outs.append((i, call(i)))
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(2):
        assert mhc.split_status(wss[i]) == 0, "a cross-workgroup wait gave up"
    for i, o in outs:
        for k in ref[i]:
            assert torch.equal(o[k], ref[i][k]), (i, k)


@pytest.mark.parametrize("t", [1000, 9000])
def test_cooperative_launch_matches_the_ordinary_launch(t):
    """MHC_PATH_COOPERATIVE runs the same kernel as a cooperative launch: the
    fused step and the mixes-only mode give the ordinary launch's bits, every
    wait completes (status word 0) and the whole header is zero again. At
    1,000 tokens every token is also checked against the oracle."""
    d = 5120
    case = make_case(wl.Workload(470 + t % 11, "split_plain", t, d, "bf16"))
    ref, dev = _run(case)
    ws = mhc.new_workspace(mhc.fused_step_workspace_bytes(t, d, "bf16"))
    out, _ = run_step(case, path="split", workspace=ws, cooperative=True)
    assert mhc.split_status(ws) == 0, "a cross-workgroup wait gave up"
    assert ws[:16384].count_nonzero().item() == 0
    for k in ref:
        if ref[k] is not None:
            assert torch.equal(out[k], ref[k]), k
    if t <= 1000:
        check_step(case, out, "bf16")
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    args = (dev["x"], wp, dev["base"], dev["scale"], case["iters"], case["norm_eps"],
            case["hc_eps"])
    m_plain = mhc.mixes(*args, want_mix=True, path="split", workspace=ws)
    m_coop = mhc.mixes(*args, want_mix=True, path="split", workspace=ws, cooperative=True)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    assert ws[:16384].count_nonzero().item() == 0
    for k in ("pre", "post", "comb", "mix"):
        assert torch.equal(m_plain[k], m_coop[k]), k


def test_two_term_projection_error_bound():
    """On 256-feature slices (the large-call geometry at d = 5120) the
    projection uses the hi and mid bf16 terms of W: |w - hi - mid| <=
    2^-16 |w|. Every mix must then lie within r * sum_f |w_jf x'_f| *
    (2^-16 + 64 * 2^-24) of the exact value on the validated new streams (the
    dropped term, plus float32 accumulation over at most 64 sequential
    roundings per output: the MFMA steps of a slice, the slices, the terms).
    Reports the largest fraction of that bound used and of the 1e-4 parity
    bar."""
    t, d = 6000, 5120
    assert mhc.fused_step_route("auto", t, d, "bf16") == "split"
    w = wl.Workload(455, "two_term", t, d, "bf16")
    case = make_case(w)
    out, _ = _run(case)
    o = check_step(case, out, "bf16")
    xp = np.asarray(o["xprime"], dtype=np.float64).reshape(t, -1)
    wabs = np.abs(np.asarray(case["w_mix"], dtype=np.float64))
    r = 1.0 / np.sqrt(np.mean(xp * xp, axis=1) + case["norm_eps"])
    err = np.abs(out["mix"].numpy().astype(np.float64) - o["m"])
    worst, worst_bar = 0.0, 0.0
    for t0 in range(0, t, 1000):
        sl = slice(t0, t0 + 1000)
        mag = (np.abs(xp[sl]) @ wabs.T) * r[sl, None]
        bound = mag * (2.0 ** -16 + 64 * 2.0 ** -24)
        assert (err[sl] <= bound).all(), "a mix outside the two-term error bound"
        worst = max(worst, float((err[sl] / bound).max()))
        worst_bar = max(worst_bar, float((err[sl] / (1e-4 * np.maximum(np.abs(o["m"][sl]), 1.0))).max()))
    _log(f"  mixes error: at most {worst:.3f} of the two-term bound, {worst_bar:.3f} of the parity bar")


def test_split_calls_on_four_streams_in_flight_together():
    """Four ordinary-launch feature-split calls in flight on four streams (each
    with its own workspace): every call's groups fill in start order, so all
    complete however the device interleaves them (status word 0), with the
    bits of the same calls run one after the other."""
    t, d = 6000, 5120
    cases = [make_case(wl.Workload(480 + i, "split_streams4", t, d, "bf16")) for i in range(4)]
    devs = [{k: to_dev(c[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                       "scale", "gamma")} for c in cases]
    wps = [mhc.pack_wmix(dv["w_mix"], "bf16") for dv in devs]
    wss = [torch.zeros(mhc.fused_step_workspace_bytes(t, d, "bf16"), dtype=torch.uint8,
                       device="cuda") for _ in range(4)]

    def call(i):
        dv = devs[i]
        return mhc.fused_step(dv["x"], dv["f"], dv["pre"], dv["post"], dv["comb"], wps[i],
                              dv["base"], dv["scale"], dv["gamma"], want_mix=True,
                              path="split", workspace=wss[i])

    ref = []
    for i in range(4):
        ref.append({k: v.clone() for k, v in call(i).items()})
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(2):
        for i in range(4):
            with torch.cuda.stream(streams[i]):
                outs.append((i, call(i)))
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(4):
        assert mhc.split_status(wss[i]) == 0, "a cross-workgroup wait gave up"
        assert wss[i][:16384].count_nonzero().item() == 0
    for i, o in outs:
        for k in ref[i]:
            assert torch.equal(o[k], ref[i][k]), (i, k)

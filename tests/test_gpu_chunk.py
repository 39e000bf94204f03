"""GPU parity of the chunked small-batch kernels (path="chunk").

Workgroups of 16 tokens x 512 features write per-token partial sums to the
workspace; a second kernel finishes every token. The cases cover one token,
ragged 16-token tiles, every chunk count from one (d = 64) to ten (d = 5120),
a ragged last chunk (d = 5056: 79 pairs of steps in chunks of 8), the largest
call the path takes (8,192 tokens), the mixes-only mode, in-place updates,
guard bands, repeated calls on one workspace, agreement with the tile kernel
(the new streams must match bit for bit: their arithmetic is the same) and the
size limits. Every call's status word must read 0.
"""

import numpy as np
import pytest
import torch

import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, run_step, to_dev
from tests.parity import check_mix_like, check_mixes, check_step

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _ws_dt(t, d, dtype):
    return torch.zeros(mhc.fused_step_workspace_bytes(t, d, dtype), dtype=torch.uint8,
                       device="cuda")


def _ws(t, d):
    return _ws_dt(t, d, "bf16")


def _run(case, **kw):
    ws = _ws(len(case["x"]), case["x"].shape[2])
    out, dev = run_step(case, path="chunk", workspace=ws, **kw)
    assert mhc.split_status(ws) == 0
    return out, dev


CHUNK_CASES = [
    (5120, 1),       # one token: one tile, 15 empty rows
    (5120, 15),
    (5120, 17),      # a second tile with one token
    (5120, 256),     # the decode shape
    (5120, 1000),
    (5120, 8192),    # the largest call the path takes
    (5056, 77),      # 79 pairs: nine chunks of 8 and one of 7
    (64, 33),        # one pair of steps: one chunk, one busy wave
    (192, 20),       # three pairs: one chunk, waves 3..7 idle
    (1024, 100),     # two chunks
    (2048, 513),
    (2560, 130),     # five chunks
    (3072, 257),
    (4096, 300),
]


@pytest.mark.parametrize("d,t", CHUNK_CASES)
def test_chunk_parity(d, t):
    _log(f"chunk d={d} T={t}")
    w = wl.Workload(700 + d % 83 + t % 5, "chunk", t, d, "bf16")
    case = make_case(w)
    out, _ = _run(case)
    o = check_step(case, out, "bf16")
    _log(f"  ties in new streams: {o['n_ties']}")


# f32 streams: chunks of 8 steps, one per wave
CHUNK_CASES_F32 = [
    (5120, 64),      # the tiny workload's shape: twenty chunks
    (5120, 1),
    (5120, 17),
    (96, 10),        # three steps: one chunk, waves 3..7 idle
    (544, 33),       # 17 steps: two chunks of 8 and a chunk of one
    (2048, 300),
    (5120, 8192),    # the largest call the path takes
]


@pytest.mark.parametrize("d,t", CHUNK_CASES_F32)
def test_chunk_parity_f32(d, t):
    _log(f"chunk f32 d={d} T={t}")
    w = wl.Workload(740 + d % 83 + t % 5, "chunk_f32", t, d, "f32")
    case = make_case(w)
    ws = _ws_dt(t, d, "f32")
    out, _ = run_step(case, dtype="f32", path="chunk", workspace=ws)
    assert mhc.split_status(ws) == 0
    check_step(case, out, "f32")


def test_chunk_f32_matches_tile_kernel():
    t, d = 70, 1024
    case = make_case(wl.Workload(747, "chunk_f32_vs_tile", t, d, "f32"))
    a, _ = run_step(case, dtype="f32", path="chunk", workspace=_ws_dt(t, d, "f32"))
    b, _ = run_step(case, dtype="f32", path="tile")
    assert torch.equal(a["x_out"], b["x_out"])   # same per-element arithmetic
    np.testing.assert_allclose(a["y"].numpy(), b["y"].numpy(), rtol=1e-5, atol=1e-6)
    for k in ("pre", "post", "comb", "mix"):
        np.testing.assert_allclose(a[k].numpy(), b[k].numpy(), rtol=0, atol=2e-5)


def test_auto_route_by_size():
    assert mhc.fused_step_route("auto", 256, 5120, "bf16") == "chunk"
    assert mhc.fused_step_route("auto", 896, 5120, "bf16") == "chunk"
    assert mhc.fused_step_route("auto", 897, 5120, "bf16") == "split"
    assert mhc.fused_step_route("auto", 65536, 5120, "bf16") == "split"
    assert mhc.fused_step_route("auto", 256, 5120, "bf16", with_workspace=False) == "tile"
    assert mhc.fused_step_route("auto", 256, 5120, "f32") == "chunk"
    assert mhc.fused_step_route("auto", 2049, 5120, "f32") == "tile"
    assert mhc.fused_step_route("auto", 64, 96, "f32") == "chunk"
    # launched cooperatively the feature-split route costs more per call, and
    # auto switches to it above 2,048 tokens
    assert mhc.fused_step_route("auto", 2048, 5120, "bf16", cooperative=True) == "chunk"
    assert mhc.fused_step_route("auto", 2049, 5120, "bf16", cooperative=True) == "split"
    assert mhc.fused_step_route("auto", 2049, 5120, "f32", cooperative=True) == "tile"
    assert mhc.fused_step_route("split", 256, 5120, "bf16", cooperative=True) == "split"
    # bf16 widths without a slice geometry take the tile kernel above 2,048 tokens
    assert mhc.fused_step_route("auto", 4096, 1024, "bf16") == "tile"
    # d = 6144 has a slice geometry but is beyond the chunked kernels' 5120
    assert mhc.fused_step_route("auto", 256, 6144, "bf16") == "split"
    assert mhc.fused_step_route("chunk", 8192, 5120, "bf16") == "chunk"
    for args in ((8193, 5120, "bf16"), (64, 6144, "bf16"), (8193, 64, "f32"), (64, 96, "bf16")):
        with pytest.raises(ValueError, match="does not apply"):
            mhc.fused_step_route("chunk", *args)


def test_chunk_matches_tile_kernel():
    w = wl.Workload(760, "chunk_vs_tile", 300, 5120, "bf16")
    case = make_case(w)
    a, _ = _run(case)
    b, _ = run_step(case, path="tile")
    assert torch.equal(a["x_out"], b["x_out"])
    ya, yb = a["y"].float(), b["y"].float()
    ulp = torch.maximum(ya.abs(), yb.abs()) * 2.0 ** -7 + 1e-30
    assert ((ya - yb).abs() <= ulp).all()
    # the chunked kernels take the hi + mid terms of W (20 Sinkhorn rounds
    # here), the tile kernel all three: the mixes agree at the parity bar
    for k in ("pre", "post", "comb", "mix"):
        check_mix_like(k, a[k], b[k])


def test_chunk_in_place_and_deterministic():
    t, d = 333, 5120
    case = make_case(wl.Workload(761, "chunk_inplace", t, d, "bf16"))
    ref, dev = _run(case)
    again, _ = _run(case)
    for k in ref:
        if ref[k] is not None:
            assert torch.equal(ref[k], again[k]), k
    x_dev = dev["x"].clone()
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    ws = _ws(t, d)
    out = mhc.fused_step(x_dev, dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                         dev["scale"], dev["gamma"], x_out=x_dev, want_mix=True, path="chunk",
                         workspace=ws)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    for k in ("x_out", "y", "pre", "post", "comb", "mix"):
        assert torch.equal(out[k].cpu(), ref[k]), k


def test_chunk_guard_bands_untouched():
    t, d, gpad = 21, 1024, 64
    case = make_case(wl.Workload(762, "chunk_guard", t, d, "bf16"))
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
    ws = _ws(t, d)
    out = mhc.fused_step(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                         dev["scale"], dev["gamma"], x_out=vx.view(t, 4, d), y_out=vy.view(t, d),
                         pre_out=vp.view(t, 4), post_out=vu.view(t, 4), comb_out=vc.view(t, 4, 4),
                         mix_out=vm.view(t, 24), path="chunk", workspace=ws)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    for buf, view in ((bx, vx), (by, vy), (bp, vp), (bu, vu), (bc, vc), (bm, vm)):
        assert torch.isnan(buf[:gpad].float()).all() and torch.isnan(buf[-gpad:].float()).all()
        assert not torch.isnan(view.float()).any()
    check_step(case, {k: (v.cpu() if v is not None else None) for k, v in out.items()}, "bf16")


def test_chunk_repeated_calls_share_a_workspace():
    """Two calls in a row on one workspace, the second smaller, then the split
    kernel on the same workspace (its counters are cleared by its own call)."""
    ws = _ws(3000, 5120)
    for t, seed, path in ((2000, 763, "chunk"), (300, 764, "chunk"), (3000, 765, "split"),
                          (100, 766, "chunk")):
        case = make_case(wl.Workload(seed, "chunk_repeat", t, 5120, "bf16"))
        out, _ = run_step(case, path=path, workspace=ws)
        assert mhc.split_status(ws) == 0
        check_step(case, out, "bf16")


def test_chunk_workspace_validation():
    t, d = 64, 1024
    x = torch.zeros((t, 4, d), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros((t, d), dtype=torch.bfloat16, device="cuda")
    wp = mhc.pack_wmix(torch.zeros((24, 4 * d), device="cuda"), "bf16")
    z = torch.zeros((t, 4), device="cuda")
    need = mhc.fused_step_workspace_bytes(t, d, "bf16")
    assert need == 16384 + 2 * t * 128
    args = (x, f, z, z, torch.zeros((t, 4, 4), device="cuda"), wp, torch.zeros(24, device="cuda"),
            torch.ones(3, device="cuda"), torch.ones(d, device="cuda"))
    small = torch.zeros(need - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(mhc.MhcError, match="workspace holds"):
        mhc.fused_step(*args, path="chunk", workspace=small)
    big = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(mhc.MhcError, match="256-byte aligned"):
        mhc.fused_step(*args, path="chunk", workspace=big[16:])


@pytest.mark.parametrize("dtype,d,t", [("bf16", 5120, 256), ("bf16", 5120, 2000),
                                        ("bf16", 1024, 37), ("bf16", 5056, 19),
                                        ("f32", 5120, 64), ("f32", 544, 21)])
def test_mixes_chunk_mode_parity(dtype, d, t):
    w = wl.Workload(770 + t % 11, "mixes_chunk", t, d, dtype)
    x = wl.streams(w)
    p = wl.params(w)
    wp = mhc.pack_wmix(to_dev(p["w_mix"]), dtype)
    ws = _ws_dt(t, d, dtype)
    dx = to_dev(x)
    out = mhc.mixes(dx, wp, to_dev(p["base"]), to_dev(p["scale"]), want_mix=True, path="chunk",
                    workspace=ws)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    check_mixes(dict(x=x, **p), {k: v.cpu() for k, v in out.items()}, dtype)
    tile = mhc.mixes(dx, wp, to_dev(p["base"]), to_dev(p["scale"]), want_mix=True, path="tile")
    for k in ("pre", "post", "comb", "mix"):
        if dtype == "bf16":   # two terms of W against three: at the parity bar
            check_mix_like(k, out[k].cpu(), tile[k].cpu())
        else:                 # the same f32 arithmetic in another order
            np.testing.assert_allclose(out[k].cpu().numpy(), tile[k].cpu().numpy(), rtol=0,
                                       atol=2e-5)


@pytest.mark.parametrize("path", ["chunk", "split"])
def test_path_replays_from_a_hip_graph(path):
    """Both workspace routes set no memory from the host (the split route's
    counters are cleared by a kernel): a call captured into a graph replays to
    the eager result, with eager work and synchronisation between the replays,
    and the replays follow new inputs copied into the captured buffers."""
    t, d = 256, 5120
    cases = [make_case(wl.Workload(780 + i, "chunk_graph", t, d, "bf16")) for i in range(2)]
    dev = {k: to_dev(cases[0][k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                            "scale", "gamma")}
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    ws = _ws(t, d)
    outs = dict(x_out=torch.empty_like(dev["x"]), y_out=torch.empty_like(dev["f"]),
                pre_out=torch.empty((t, 4), device="cuda"),
                post_out=torch.empty((t, 4), device="cuda"),
                comb_out=torch.empty((t, 4, 4), device="cuda"),
                mix_out=torch.empty((t, 24), device="cuda"))

    def call():
        mhc.fused_step(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
                       dev["scale"], dev["gamma"], path=path, workspace=ws, **outs)

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
        src = {k: to_dev(cases[i][k]) for k in ("x", "f", "pre", "post", "comb")}
        for k, v in src.items():
            dev[k].copy_(v)
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
        assert mhc.split_status(ws) == 0
        ref = dict(cases[0])   # the captured parameters, case i's streams and coefficients
        ref.update({k: cases[i][k] for k in ("x", "f", "pre", "post", "comb")})
        check_step(ref, {"x_out": got["x_out"].cpu(), "y": got["y_out"].cpu(),
                              "pre": got["pre_out"].cpu(), "post": got["post_out"].cpu(),
                              "comb": got["comb_out"].cpu(), "mix": got["mix_out"].cpu()}, "bf16")


def test_chunk_without_mix_out():
    """mix_out is optional: without it the chunked route writes every other
    output exactly as with it."""
    t, d = 100, 5120
    case = make_case(wl.Workload(790, "chunk_nomix", t, d, "bf16"))
    a, _ = _run(case)
    b, _ = _run(case, want_mix=False)
    assert b["mix"] is None
    for k in ("x_out", "y", "pre", "post", "comb"):
        assert torch.equal(a[k], b[k]), k

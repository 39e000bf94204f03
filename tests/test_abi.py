"""CPU-side checks of the C ABI: the library loads, exports every function that
include/mhc.h declares, and rejects bad arguments before any HIP call (fake,
never dereferenced device addresses are used; nothing is launched)."""

import ctypes
import os
import re

import pytest

from stream_hyper_connections_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libmhc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ("mhc_fused_step", "mhc_mixes", "mhc_sinkhorn4", "mhc_pack_wmix",
               "mhc_wmix_packed_bytes", "mhc_status_string", "mhc_last_error",
               "mhc_abi_version", "mhc_d_granule", "mhc_fused_step_workspace_bytes",
               "mhc_hc_post", "mhc_hc_pre", "mhc_rmsnorm", "mhc_wmix_packed_bytes_n",
               "mhc_pack_wmix_n", "mhc_fused_step_n", "mhc_mixes_n", "mhc_sinkhorn_n",
               "mhc_fused_step_n_workspace_bytes", "mhc_fused_step_route",
               "mhc_fused_step_route_n",
               "mhc_fused_step_backward_n", "mhc_fused_step_backward_workspace_bytes_n",
               "mhc_fused_step_noalloc"):
        assert fn in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for fn in declared_functions():
        assert hasattr(lib, fn), fn
    assert set(declared_functions()) == set(binding._SIGS)


def test_version_granule_and_status_strings():
    assert binding.abi_version() == 11
    assert binding.d_granule() == 32
    lib = binding.load()
    assert lib.mhc_status_string(0) == b"MHC_OK"
    assert lib.mhc_status_string(1) == b"MHC_ERR_INVALID_ARG"
    assert lib.mhc_status_string(2) == b"MHC_ERR_UNSUPPORTED"
    assert lib.mhc_status_string(3) == b"MHC_ERR_HIP"
    assert lib.mhc_status_string(99) == b"unknown status"


def test_packed_bytes():
    lib = binding.load()
    assert lib.mhc_wmix_packed_bytes(5120, binding.MHC_BF16) == 160 * 4 * 5 * 64 * 16
    assert lib.mhc_wmix_packed_bytes(5120, binding.MHC_F32) == 160 * 4 * 2 * 64 * 32
    assert lib.mhc_wmix_packed_bytes(100, binding.MHC_BF16) == -1
    assert lib.mhc_wmix_packed_bytes(0, binding.MHC_BF16) == -1
    assert lib.mhc_wmix_packed_bytes(64, 7) == -1


# ---- validation of mhc_fused_step with fake addresses ----------------------------------

T, D = 64, 256
ES = 2
A = 1 << 40          # fake, aligned, never dereferenced


def _layout():
    """Non-overlapping fake buffers for every argument."""
    sizes = {
        "x": T * 4 * D * ES, "f": T * D * ES, "pre_in": T * 16, "post_in": T * 16,
        "comb_in": T * 64, "w_packed": (D // 32) * 4 * 5 * 64 * 16, "base": 96, "scale": 12,
        "gamma": D * 4, "x_out": T * 4 * D * ES, "y_out": T * D * ES, "pre_out": T * 16,
        "post_out": T * 16, "comb_out": T * 64, "mix_out": T * 96,
    }
    addr, p = A, {}
    for k, n in sizes.items():
        p[k] = addr
        addr += (n + 4095) // 4096 * 4096
    return p


def _call(**over):
    p = _layout()
    args = dict(x=p["x"], f=p["f"], dtype=binding.MHC_BF16, tokens=T, d=D, pre_in=p["pre_in"],
                post_in=p["post_in"], comb_in=p["comb_in"], w_packed=p["w_packed"],
                base=p["base"], scale=p["scale"], gamma=p["gamma"], iters=20, norm_eps=1e-6,
                hc_eps=1e-6, x_out=p["x_out"], y_out=p["y_out"], pre_out=p["pre_out"],
                post_out=p["post_out"], comb_out=p["comb_out"], mix_out=p["mix_out"],
                path=binding.PATHS["auto"], workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    lib = binding.load()
    return lib.mhc_fused_step(*args.values())


@pytest.mark.parametrize("over,needle", [
    (dict(dtype=5), "dtype"),
    (dict(tokens=-1), "tokens"),
    (dict(d=0), "multiple"),
    (dict(d=48), "multiple"),
    (dict(iters=0), "sinkhorn_iters"),
    (dict(norm_eps=-1.0), "norm_eps"),
    (dict(norm_eps=float("nan")), "norm_eps"),
    (dict(hc_eps=float("inf")), "hc_eps"),
    (dict(x=None), "x is NULL"),
    (dict(gamma=None), "gamma is NULL"),
    (dict(comb_out=None), "comb_out is NULL"),
    (dict(f=A + 8), "not 16-byte aligned"),
    (dict(y_out=_layout()["x_out"] + 64), "overlap"),
    (dict(x_out=_layout()["x"] + 16), "overlaps input"),
    (dict(pre_out=_layout()["pre_in"]), "overlaps input"),
    (dict(mix_out=_layout()["comb_out"]), "overlap"),
])
def test_fused_step_rejects_bad_arguments(over, needle):
    st = _call(**over)
    assert st == binding.MHC_ERR_INVALID_ARG
    assert needle in binding.last_error()


def test_fused_step_rejects_unknown_path():
    both = binding.PLAIN_LAUNCH | binding.COOPERATIVE   # the two launch flags at once
    for path in (-1, 4, 9, 4 | binding.PLAIN_LAUNCH, 4 | binding.COOPERATIVE, 64, both,
                 2 | both):
        assert _call(path=path) == binding.MHC_ERR_INVALID_ARG
        assert "unknown path" in binding.last_error()


def test_route_query_without_a_device_query():
    """Routes that need no device attribute: the tile kernel without a
    workspace, and bad arguments."""
    lib = binding.load()
    for path in ("auto", "tile"):
        assert lib.mhc_fused_step_route(binding.PATHS[path], 64, 5120, binding.MHC_BF16, 0) == 1
    assert lib.mhc_fused_step_route(binding.PATHS["tile"], 64, 5120, binding.MHC_BF16, 1) == 1
    # neither launch flag changes these routes
    for path in ("auto", "tile"):
        for flag in (binding.PLAIN_LAUNCH, binding.COOPERATIVE):
            code = binding.PATHS[path] | flag
            assert lib.mhc_fused_step_route(code, 64, 5120, binding.MHC_BF16, 0) == 1
    assert lib.mhc_fused_step_route(7, 64, 5120, binding.MHC_BF16, 0) == -1
    assert "unknown path" in binding.last_error()
    assert lib.mhc_fused_step_route(0, -1, 5120, binding.MHC_BF16, 0) == -1
    assert "bad tokens" in binding.last_error()


def _chunk_n_bytes(n, tokens, chunks=80):
    row = ((2 + n) * n + 2 + 3) // 4 * 4
    return 16384 + chunks * tokens * row * 4


def test_route_query_n_family_without_a_device_query():
    """n = 8 and float32 streams have no feature-split kernel, so their routes
    need no device attribute: the chunks wherever they apply (up to 8192
    tokens) under "auto" with a workspace, the block kernel otherwise."""
    lib = binding.load()
    route = lib.mhc_fused_step_route_n
    bf, f32 = binding.MHC_BF16, binding.MHC_F32
    assert route(8, 0, 256, 5120, bf, 1) == 3
    assert route(8, 0, 2048, 5120, bf, 1) == 3
    assert route(8, 0, 8192, 5120, bf, 1) == 3
    assert route(8, 0, 8193, 5120, bf, 1) == 1
    assert route(8, 0, 256, 5120, bf, 0) == 1
    assert route(2, 0, 256, 5120, f32, 1) == 3
    assert route(8, 1, 256, 5120, bf, 1) == 1
    assert route(8, 3, 8192, 5120, bf, 1) == 3
    assert route(8, 3 | binding.PLAIN_LAUNCH, 8192, 5120, bf, 1) == 3
    assert route(8, binding.PLAIN_LAUNCH, 8193, 5120, bf, 1) == 1
    assert route(8, 3 | binding.COOPERATIVE, 8192, 5120, bf, 1) == 3
    assert route(8, binding.COOPERATIVE, 8193, 5120, bf, 1) == 1
    assert route(8, 3, 8193, 5120, bf, 1) == -1
    assert "chunked kernel does not apply" in binding.last_error()
    assert route(8, 2, 256, 5120, bf, 1) == -1
    assert "feature-split kernel does not apply" in binding.last_error()
    assert route(8, 3, 256, 5120, bf, 0) == -1
    assert "needs a workspace" in binding.last_error()
    assert route(3, 0, 256, 5120, bf, 1) == -1
    assert route(8, 5, 256, 5120, bf, 1) == -1
    assert "unknown path" in binding.last_error()
    # chunk workspace: 16,384-byte header, then 80 chunks of R floats per token
    assert lib.mhc_fused_step_n_workspace_bytes(8, 256, 5120, bf) == _chunk_n_bytes(8, 256)
    assert lib.mhc_fused_step_n_workspace_bytes(2, 100, 5120, f32) == _chunk_n_bytes(2, 100)
    assert lib.mhc_fused_step_n_workspace_bytes(4, 64, 5120, f32) == _chunk_n_bytes(4, 64)
    # 7 units of 32 features: one unit per chunk
    assert lib.mhc_fused_step_n_workspace_bytes(8, 10, 224, bf) == _chunk_n_bytes(8, 10, 7)
    assert lib.mhc_fused_step_n_workspace_bytes(8, 8193, 5120, bf) == 0


def test_fused_step_n_chunk_path_checks_its_workspace():
    need = _chunk_n_bytes(8, T, D // 32)
    assert _call_n(8, path=3) == binding.MHC_ERR_INVALID_ARG
    assert "needs a workspace" in binding.last_error()
    ws = A + (1 << 34)
    assert _call_n(8, path=3, workspace=ws, workspace_bytes=256) == binding.MHC_ERR_INVALID_ARG
    assert "needed" in binding.last_error()
    assert _call_n(8, path=3, workspace=ws + 64, workspace_bytes=1 << 30) == \
        binding.MHC_ERR_INVALID_ARG
    assert "aligned" in binding.last_error()
    p = _layout_n(8)
    assert _call_n(8, path=3, workspace=p["y_out"], workspace_bytes=1 << 30) == \
        binding.MHC_ERR_INVALID_ARG
    assert "overlap" in binding.last_error()
    assert _call_n(8, path=2, workspace=ws, workspace_bytes=need) == binding.MHC_ERR_UNSUPPORTED
    assert _call_n(8, path=6) == binding.MHC_ERR_INVALID_ARG


def test_workspace_bytes_rejects_bad_arguments():
    lib = binding.load()
    for args in ((-1, 5120, binding.MHC_BF16), (64, 48, binding.MHC_BF16), (64, 5120, 9)):
        assert lib.mhc_fused_step_workspace_bytes(*args) == -1
        assert "bad tokens" in binding.last_error()


def test_fused_step_zero_tokens_is_a_no_op():
    assert _call(tokens=0) == binding.MHC_OK
    assert binding.last_error() == ""


def test_fused_step_in_place_streams_pass_validation_with_zero_tokens():
    p = _layout()
    assert _call(tokens=0, x_out=p["x"]) == binding.MHC_OK


def test_mixes_and_sinkhorn_validation():
    lib = binding.load()
    p = _layout()
    st = lib.mhc_mixes(p["x"], binding.MHC_BF16, T, D, p["w_packed"], p["base"], p["scale"], 0,
                       1e-6, 1e-6, p["pre_out"], p["post_out"], p["comb_out"], None, 0, None, 0, None)
    assert st == binding.MHC_ERR_INVALID_ARG
    st = lib.mhc_mixes(p["x"], binding.MHC_BF16, 0, D, p["w_packed"], p["base"], p["scale"], 20,
                       1e-6, 1e-6, p["pre_out"], p["post_out"], p["comb_out"], None, 0, None, 0, None)
    assert st == binding.MHC_OK
    st = lib.mhc_sinkhorn4(p["mix_out"], T, p["base"], p["scale"], 20, -1.0, p["pre_out"],
                           p["post_out"], p["comb_out"], None)
    assert st == binding.MHC_ERR_INVALID_ARG
    st = lib.mhc_sinkhorn4(p["mix_out"], T, p["base"], p["scale"], 20, 1e-6, p["pre_out"],
                           p["pre_out"], p["comb_out"], None)
    assert st == binding.MHC_ERR_INVALID_ARG and "overlap" in binding.last_error()
    st = lib.mhc_sinkhorn4(p["mix_out"], 0, p["base"], p["scale"], 20, 1e-6, p["pre_out"],
                           p["post_out"], p["comb_out"], None)
    assert st == binding.MHC_OK


def test_pack_validation():
    lib = binding.load()
    p = _layout()
    need = lib.mhc_wmix_packed_bytes(D, binding.MHC_BF16)
    assert lib.mhc_pack_wmix(p["x"], D, binding.MHC_BF16, p["w_packed"], need - 16,
                             None) == binding.MHC_ERR_INVALID_ARG
    assert "bytes" in binding.last_error()
    assert lib.mhc_pack_wmix(p["x"], 40, binding.MHC_BF16, p["w_packed"], need,
                             None) == binding.MHC_ERR_INVALID_ARG
    assert lib.mhc_pack_wmix(None, D, binding.MHC_BF16, p["w_packed"], need,
                             None) == binding.MHC_ERR_INVALID_ARG


def test_unfused_entry_points_validate():
    lib = binding.load()
    p = _layout()
    # NULL input, bad width, overlapping output, zero tokens
    assert lib.mhc_hc_post(None, p["f"], binding.MHC_BF16, T, D, p["post_in"], p["comb_in"],
                           p["x_out"], None) == binding.MHC_ERR_INVALID_ARG
    assert "x is NULL" in binding.last_error()
    assert lib.mhc_hc_post(p["x"], p["f"], binding.MHC_BF16, T, 48, p["post_in"], p["comb_in"],
                           p["x_out"], None) == binding.MHC_ERR_INVALID_ARG
    assert lib.mhc_hc_post(p["x"], p["f"], binding.MHC_BF16, T, D, p["post_in"], p["comb_in"],
                           p["f"], None) == binding.MHC_ERR_INVALID_ARG
    assert "overlaps" in binding.last_error()
    assert lib.mhc_hc_post(p["x"], p["f"], binding.MHC_BF16, 0, D, p["post_in"], p["comb_in"],
                           p["x"], None) == binding.MHC_OK
    assert lib.mhc_hc_pre(p["x"], binding.MHC_BF16, T, D, p["pre_in"], p["x"] + 64,
                          None) == binding.MHC_ERR_INVALID_ARG
    assert lib.mhc_hc_pre(p["x"], 3, T, D, p["pre_in"], p["y_out"], None) == binding.MHC_ERR_INVALID_ARG
    assert lib.mhc_rmsnorm(p["y_out"], binding.MHC_BF16, T, D, None, 1e-6, p["y_out"],
                           None) == binding.MHC_ERR_INVALID_ARG
    assert "gamma is NULL" in binding.last_error()
    assert lib.mhc_rmsnorm(p["y_out"], binding.MHC_BF16, T, D, p["gamma"], -1.0, p["y_out"],
                           None) == binding.MHC_ERR_INVALID_ARG
    assert lib.mhc_rmsnorm(p["y_out"], binding.MHC_BF16, 0, D, p["gamma"], 1e-6, p["y_out"],
                           None) == binding.MHC_OK


# ---- the general-n family --------------------------------------------------------------

def test_packed_bytes_n():
    lib = binding.load()
    # bf16: three terms, each padded to ceil((2+n)n / 16) tiles of 16 columns
    for n, tiles in ((2, 3), (4, 6), (8, 15)):
        assert lib.mhc_wmix_packed_bytes_n(n, 5120, binding.MHC_BF16) == 160 * n * tiles * 64 * 16
    for n, tiles in ((2, 1), (4, 2), (8, 5)):
        assert lib.mhc_wmix_packed_bytes_n(n, 5120, binding.MHC_F32) == 160 * n * tiles * 64 * 32
    for args in ((3, 5120, binding.MHC_BF16), (8, 40, binding.MHC_BF16), (2, 64, 5)):
        assert lib.mhc_wmix_packed_bytes_n(*args) == -1


def _layout_n(n):
    nm = (2 + n) * n
    sizes = {
        "x": T * n * D * ES, "f": T * D * ES, "pre_in": T * n * 4, "post_in": T * n * 4,
        "comb_in": T * n * n * 4, "w_packed": 1 << 24, "base": nm * 4, "scale": 12,
        "gamma": D * 4, "x_out": T * n * D * ES, "y_out": T * D * ES, "pre_out": T * n * 4,
        "post_out": T * n * 4, "comb_out": T * n * n * 4, "mix_out": T * nm * 4,
    }
    addr, p = A, {}
    for k, sz in sizes.items():
        p[k] = addr
        addr += (sz + 4095) // 4096 * 4096
    return p


def _call_n(n_layout, **over):
    p = _layout_n(n_layout)
    args = dict(n=n_layout, x=p["x"], f=p["f"], dtype=binding.MHC_BF16, tokens=T, d=D,
                pre_in=p["pre_in"], post_in=p["post_in"], comb_in=p["comb_in"],
                w_packed=p["w_packed"], base=p["base"], scale=p["scale"], gamma=p["gamma"],
                iters=20, norm_eps=1e-6, hc_eps=1e-6, x_out=p["x_out"], y_out=p["y_out"],
                pre_out=p["pre_out"], post_out=p["post_out"], comb_out=p["comb_out"],
                mix_out=p["mix_out"], path=0, workspace=None, workspace_bytes=0, stream=None)
    args.update(over)
    return binding.load().mhc_fused_step_n(*args.values())


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("over,needle", [
    (dict(d=48), "multiple"),
    (dict(iters=0), "sinkhorn_iters"),
    (dict(mix_out=None), "mix_out is NULL"),
    (dict(comb_in=None), "comb_in is NULL"),
    (dict(post_out=A + 4), "not 16-byte aligned"),
    (dict(x_out="x+16"), "overlaps input"),
    (dict(mix_out="comb_out"), "overlap"),
])
def test_fused_step_n_rejects_bad_arguments(n, over, needle):
    p = _layout_n(n)
    over = {k: (p[v.split("+")[0]] + int(v.split("+")[1]) if isinstance(v, str) and "+" in v
                else p[v] if isinstance(v, str) else v) for k, v in over.items()}
    assert _call_n(n, **over) == binding.MHC_ERR_INVALID_ARG
    assert needle in binding.last_error()


def test_fused_step_n_stream_counts_and_zero_tokens():
    for n in (1, 3, 5, 16):
        assert _call_n(4, n=n) == binding.MHC_ERR_UNSUPPORTED
        assert "streams" in binding.last_error()
    for n in (2, 4, 8):
        assert _call_n(n, tokens=0) == binding.MHC_OK
        assert _call_n(n, tokens=0, x_out=_layout_n(n)["x"]) == binding.MHC_OK


def test_fused_step_n_workspace_bytes_validation():
    lib = binding.load()
    for args in ((3, 100, 512, binding.MHC_BF16), (4, -1, 512, binding.MHC_BF16),
                 (2, 100, 48, binding.MHC_BF16), (8, 100, 512, 7)):
        assert lib.mhc_fused_step_n_workspace_bytes(*args) == -1
        assert "bad" in binding.last_error()


def test_mixes_n_sinkhorn_n_pack_n_validation():
    lib = binding.load()
    p = _layout_n(8)
    st = lib.mhc_mixes_n(8, p["x"], binding.MHC_BF16, T, D, p["w_packed"], p["base"], p["scale"],
                         20, 1e-6, 1e-6, p["pre_out"], p["post_out"], p["comb_out"], None, 0, None,
                         0, None)
    assert st == binding.MHC_ERR_INVALID_ARG and "mix_out is NULL" in binding.last_error()
    st = lib.mhc_mixes_n(6, p["x"], binding.MHC_BF16, T, D, p["w_packed"], p["base"], p["scale"],
                         20, 1e-6, 1e-6, p["pre_out"], p["post_out"], p["comb_out"], p["mix_out"],
                         0, None, 0, None)
    assert st == binding.MHC_ERR_UNSUPPORTED
    st = lib.mhc_sinkhorn_n(8, p["mix_out"], T, p["base"], p["scale"], 20, 1e-6, p["pre_out"],
                            p["pre_out"], p["comb_out"], None)
    assert st == binding.MHC_ERR_INVALID_ARG and "overlap" in binding.last_error()
    st = lib.mhc_sinkhorn_n(2, p["mix_out"], T, p["base"], p["scale"], 0, 1e-6, p["pre_out"],
                            p["post_out"], p["comb_out"], None)
    assert st == binding.MHC_ERR_INVALID_ARG
    st = lib.mhc_sinkhorn_n(4, p["mix_out"], 0, p["base"], p["scale"], 20, 1e-6, p["pre_out"],
                            p["post_out"], p["comb_out"], None)
    assert st == binding.MHC_OK
    need = lib.mhc_wmix_packed_bytes_n(8, D, binding.MHC_BF16)
    assert lib.mhc_pack_wmix_n(8, p["x"], D, binding.MHC_BF16, p["w_packed"], need - 16,
                               None) == binding.MHC_ERR_INVALID_ARG
    assert lib.mhc_pack_wmix_n(5, p["x"], D, binding.MHC_BF16, p["w_packed"], need,
                               None) == binding.MHC_ERR_UNSUPPORTED


# ---- backward --------------------------------------------------------------------------

def _call_bwd(n=4, **over):
    p = _layout_n(n)
    ws_addr = A + (1 << 36)
    args = dict(n=n, x=p["x"], f=p["f"], dtype=binding.MHC_BF16, tokens=T, d=D,
                pre_in=p["pre_in"], post_in=p["post_in"], comb_in=p["comb_in"],
                x_out=p["x_out"], mix=p["mix_out"], w_mix=p["w_packed"], base=p["base"],
                scale=p["scale"], gamma=p["gamma"], iters=20, norm_eps=1e-6, hc_eps=1e-6,
                d_x_out=A + (1 << 37), d_y=A + (1 << 37) + (1 << 30), d_pre=p["pre_out"],
                d_post=p["post_out"], d_comb=p["comb_out"], d_x=A + (1 << 38),
                d_f=A + (1 << 38) + (1 << 30), d_pre_in=A + (1 << 39),
                d_post_in=A + (1 << 39) + (1 << 20), d_comb_in=A + (1 << 39) + (2 << 20),
                d_w_mix=A + (1 << 39) + (4 << 20), d_base=A + (1 << 39) + (64 << 20),
                d_scale=A + (1 << 39) + (65 << 20), d_gamma=A + (1 << 39) + (66 << 20),
                workspace=ws_addr,
                workspace_bytes=binding.load().mhc_fused_step_backward_workspace_bytes_n(n, T, D),
                stream=None)
    args.update(over)
    return binding.load().mhc_fused_step_backward_n(*args.values())


def test_backward_workspace_bytes():
    lib = binding.load()
    assert lib.mhc_fused_step_backward_workspace_bytes_n(4, 1000, 5120) > 0
    assert lib.mhc_fused_step_backward_workspace_bytes_n(8, 1000, 5120) == -1
    assert lib.mhc_fused_step_backward_workspace_bytes_n(4, -1, 5120) == -1
    assert lib.mhc_fused_step_backward_workspace_bytes_n(2, 10, 48) == -1


@pytest.mark.parametrize("over,status,needle", [
    (dict(n=8), binding.MHC_ERR_UNSUPPORTED, "streams"),
    (dict(iters=0), binding.MHC_ERR_INVALID_ARG, "sinkhorn_iters"),
    (dict(workspace_bytes=1024), binding.MHC_ERR_INVALID_ARG, "workspace holds"),
    (dict(workspace=A + (1 << 36) + 16), binding.MHC_ERR_INVALID_ARG, "256-byte"),
    (dict(mix=None), binding.MHC_ERR_INVALID_ARG, "mix is NULL"),
    (dict(d_gamma=None), binding.MHC_ERR_INVALID_ARG, "d_gamma is NULL"),
    (dict(d_x="x"), binding.MHC_ERR_INVALID_ARG, "overlaps input"),
])
def test_backward_rejects_bad_arguments(over, status, needle):
    p = _layout_n(4)
    over = {k: (p[v] if isinstance(v, str) else v) for k, v in over.items()}
    assert _call_bwd(**over) == status
    assert needle in binding.last_error()


def test_backward_zero_tokens():
    assert _call_bwd(tokens=0) == binding.MHC_OK


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mhc.h"

int main(void) {
  if (mhc_abi_version() != MHC_ABI_VERSION) return 1;
  if (strcmp(mhc_status_string(MHC_OK), "MHC_OK") != 0) return 2;
  if (mhc_wmix_packed_bytes(5120, MHC_BF16) != 160LL * 4 * 5 * 64 * 16) return 3;
  if (mhc_fused_step_workspace_bytes(-1, 5120, MHC_BF16) != -1) return 4;
  if (strstr(mhc_last_error(), "bad tokens") == NULL) return 5;
  mhc_path p = MHC_PATH_CHUNK;
  if (mhc_fused_step_route(9, 64, 5120, MHC_BF16, 0) != -1 || p != 3) return 6;
  printf("ok %d\n", mhc_abi_version());
  return 0;
}
"""


def test_header_is_c_and_links(tmp_path):
    """include/mhc.h compiles as C99 and a C program linked against libmhc.so
    calls the entry points that need no device."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(binding.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.dirname(HEADER),
           str(src), "-o", str(exe), "-L", libdir, "-l:libmhc.so", f"-Wl,-rpath,{libdir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stderr)
    assert run.stdout.strip() == f"ok {binding.abi_version()}"


# ---- property-based check of the validation (fake addresses, no device) --------------

from hypothesis import given, settings, strategies as st  # noqa: E402

_PTRS = ("x", "f", "pre_in", "post_in", "comb_in", "w_packed", "base", "scale", "gamma",
         "x_out", "y_out", "pre_out", "post_out", "comb_out")
_OUTS = ("x_out", "y_out", "pre_out", "post_out", "comb_out", "mix_out")


def _defects():
    """Each defect makes the call invalid on its own; (kind, key, value)."""
    p = _layout()
    out = [("dtype", "dtype", v) for v in (-1, 2, 5, 100)]
    out += [("tokens", "tokens", v) for v in (-1, -(1 << 40))]
    out += [("d", "d", v) for v in (0, -32, 31, 48, 100)]
    out += [("iters", "iters", v) for v in (0, -5)]
    for k in ("norm_eps", "hc_eps"):
        out += [(k, k, v) for v in (-1e-3, float("nan"), float("inf"), float("-inf"))]
    out += [("null", k, None) for k in _PTRS]
    out += [("align", k, p[k] + off) for k in _PTRS for off in (4, 8)]
    # an output that starts inside another buffer (never the exact in-place x_out == x)
    out += [("overlap", o, p[b] + 16) for o in _OUTS for b in ("x", "f", "comb_in", "y_out")
            if o != b]
    out += [("path", "path", v) for v in (-1, 4, 99)]
    return out


DEFECTS = _defects()


@settings(max_examples=300, deadline=None)
@given(st.lists(st.sampled_from(range(len(DEFECTS))), min_size=1, max_size=3, unique=True))
def test_fused_step_rejects_any_invalid_combination(picks):
    over = {}
    for i in picks:
        _, key, value = DEFECTS[i]
        if key not in over:   # the first defect on a field wins
            over[key] = value
    st_code = _call(**over)
    assert st_code == binding.MHC_ERR_INVALID_ARG, (over, st_code, binding.last_error())
    assert binding.last_error() != ""


@settings(max_examples=100, deadline=None)
@given(st.integers(min_value=(1 << 35) + 1, max_value=1 << 50))
def test_fused_step_rejects_token_counts_beyond_the_limit(tokens):
    assert _call(tokens=tokens) == binding.MHC_ERR_UNSUPPORTED
    assert "2^35" in binding.last_error()


def _defects_n(n):
    p = _layout_n(n)
    ptrs = _PTRS + ("mix_out",)
    out = [("dtype", "dtype", v) for v in (-1, 2, 5)]
    out += [("tokens", "tokens", v) for v in (-1, -(1 << 40))]
    out += [("d", "d", v) for v in (0, 31, 48)]
    out += [("iters", "iters", v) for v in (0, -5)]
    for k in ("norm_eps", "hc_eps"):
        out += [(k, k, v) for v in (-1.0, float("nan"), float("inf"))]
    out += [("null", k, None) for k in ptrs]
    out += [("align", k, p[k] + 8) for k in ptrs]
    out += [("overlap", o, p[b] + 16) for o in _OUTS for b in ("x", "f", "comb_in", "y_out")
            if o != b]
    return out


@settings(max_examples=150, deadline=None)
@given(st.sampled_from([2, 4, 8]), st.data())
def test_fused_step_n_rejects_any_invalid_combination(n, data):
    defects = _defects_n(n)
    picks = data.draw(st.lists(st.sampled_from(range(len(defects))), min_size=1, max_size=3,
                               unique=True))
    over = {}
    for i in picks:
        _, key, value = defects[i]
        over.setdefault(key, value)
    st_code = _call_n(n, **over)
    assert st_code == binding.MHC_ERR_INVALID_ARG, (n, over, st_code, binding.last_error())
    assert binding.last_error() != ""

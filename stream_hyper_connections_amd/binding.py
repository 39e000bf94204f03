"""Thin ctypes binding of libmhc (include/mhc.h) for torch tensors.

Argument marshalling only: every computation runs in the HIP kernels of
libmhc.so. Tensors must be CUDA (HIP) tensors, contiguous, with the layouts of
mhc.h; outputs are allocated with torch when not given. Work is enqueued on
torch's current stream. There is no CPU fallback: if the library is missing
the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MHC_LIBRARY names another build of the same library (the CPU sanitizer test
# loads an AddressSanitizer build this way); by default the in-tree one.
LIB_PATH = os.environ.get("MHC_LIBRARY") or os.path.join(_PKG, "libmhc.so")

MHC_OK, MHC_ERR_INVALID_ARG, MHC_ERR_UNSUPPORTED, MHC_ERR_HIP = 0, 1, 2, 3
MHC_F32, MHC_BF16 = 0, 1
N_STREAMS, N_MIX = 4, 24

_c_void_p, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float

_SIGS = {
    "mhc_abi_version": ([], _i32),
    "mhc_status_string": ([_i32], ctypes.c_char_p),
    "mhc_last_error": ([], ctypes.c_char_p),
    "mhc_d_granule": ([], _i32),
    "mhc_wmix_packed_bytes": ([_i32, _i32], _i64),
    "mhc_pack_wmix": ([_c_void_p, _i32, _i32, _c_void_p, _i64, _c_void_p], _i32),
    "mhc_fused_step_workspace_bytes": ([_i64, _i32, _i32], _i64),
    "mhc_fused_step": ([_c_void_p, _c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p, _c_void_p,
                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _f32, _f32,
                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                        _i32, _c_void_p, _i64, _c_void_p], _i32),
    "mhc_fused_step_noalloc": ([_c_void_p, _c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p,
                                _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _f32,
                                _f32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p, _i32, _c_void_p], _i32),
    "mhc_mixes": ([_c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _f32, _f32,
                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p, _i64, _c_void_p],
                  _i32),
    "mhc_fused_step_route": ([_i32, _i64, _i32, _i32, _i32], _i32),
    "mhc_hc_post": ([_c_void_p, _c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p, _c_void_p,
                     _c_void_p], _i32),
    "mhc_hc_pre": ([_c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p, _c_void_p], _i32),
    "mhc_rmsnorm": ([_c_void_p, _i32, _i64, _i32, _c_void_p, _f32, _c_void_p, _c_void_p], _i32),
    "mhc_sinkhorn4": ([_c_void_p, _i64, _c_void_p, _c_void_p, _i32, _f32, _c_void_p, _c_void_p,
                       _c_void_p, _c_void_p], _i32),
    "mhc_wmix_packed_bytes_n": ([_i32, _i32, _i32], _i64),
    "mhc_pack_wmix_n": ([_i32, _c_void_p, _i32, _i32, _c_void_p, _i64, _c_void_p], _i32),
    "mhc_fused_step_n_workspace_bytes": ([_i32, _i64, _i32, _i32], _i64),
    "mhc_fused_step_n": ([_i32, _c_void_p, _c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p,
                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _f32, _f32,
                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                          _i32, _c_void_p, _i64, _c_void_p], _i32),
    "mhc_mixes_n": ([_i32, _c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p, _c_void_p, _i32,
                     _f32, _f32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p,
                     _i64, _c_void_p], _i32),
    "mhc_fused_step_route_n": ([_i32, _i32, _i64, _i32, _i32, _i32], _i32),
    "mhc_sinkhorn_n": ([_i32, _c_void_p, _i64, _c_void_p, _c_void_p, _i32, _f32, _c_void_p,
                        _c_void_p, _c_void_p, _c_void_p], _i32),
    "mhc_fused_step_backward_workspace_bytes_n": ([_i32, _i64, _i32], _i64),
    "mhc_fused_step_backward_n": ([_i32, _c_void_p, _c_void_p, _i32, _i64, _i32]
                                  + [_c_void_p] * 9 + [_i32, _f32, _f32]
                                  + [_c_void_p] * 15 + [_i64, _c_void_p], _i32),
}

_lib = None


class MhcError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}: {detail}")


def load():
    """Load libmhc.so (once) and declare the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; build it with "
                               "`python -m stream_hyper_connections_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().mhc_status_string(status).decode()


def last_error() -> str:
    return load().mhc_last_error().decode()


def abi_version() -> int:
    return load().mhc_abi_version()


def d_granule() -> int:
    return load().mhc_d_granule()


def _check(fn, status):
    if status != MHC_OK:
        raise MhcError(fn, status, last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MHC_BF16
    if t.dtype == torch.float32:
        return MHC_F32
    raise TypeError(f"stream tensors must be bfloat16 or float32, got {t.dtype}")


def _dtype_name_code(dtype) -> int:
    if dtype in ("bf16", torch.bfloat16, MHC_BF16):
        return MHC_BF16
    if dtype in ("f32", torch.float32, MHC_F32):
        return MHC_F32
    raise TypeError(f"unknown stream dtype {dtype!r}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _f32_out(shape, like, out):
    if out is not None:
        return out
    return torch.empty(shape, dtype=torch.float32, device=like.device)


def wmix_packed_bytes(d: int, dtype) -> int:
    return load().mhc_wmix_packed_bytes(d, _dtype_name_code(dtype))


def pack_wmix(w_mix: torch.Tensor, dtype, out: torch.Tensor | None = None) -> torch.Tensor:
    """mhc_pack_wmix: float32 W [24, 4d] -> packed operand buffer (uint8)."""
    code = _dtype_name_code(dtype)
    d = w_mix.shape[1] // N_STREAMS
    nbytes = load().mhc_wmix_packed_bytes(d, code)
    if nbytes < 0:
        raise ValueError(f"width {d} is not a positive multiple of {d_granule()}")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w_mix.device)
    _check("mhc_pack_wmix", load().mhc_pack_wmix(_ptr(w_mix), d, code, _ptr(out),
                                                 out.numel() * out.element_size(), _stream()))
    return out


# mhc_path codes by name
PATHS = {"auto": 0, "tile": 1, "split": 2, "chunk": 3}
_PATH_NAMES = {v: k for k, v in PATHS.items()}
# MHC_PATH_COOPERATIVE: OR-ed into a path code, the feature-split kernel is
# launched cooperatively instead of as an ordinary kernel (see mhc.h)
COOPERATIVE = 32
# MHC_PATH_PLAIN_LAUNCH: the ordinary launch, the default; accepted, changes nothing
PLAIN_LAUNCH = 16

_workspaces = {}


def fused_step_route(path: str, tokens: int, d: int, dtype, with_workspace=True,
                     cooperative=False) -> str:
    """mhc_fused_step_route: the kernel family ("tile", "split" or "chunk") that
    fused_step / mixes run for `path` (and cooperative); ValueError if that
    path cannot run these arguments."""
    if path not in PATHS:
        raise ValueError(f"unknown path {path!r}")
    r = load().mhc_fused_step_route(PATHS[path] | (COOPERATIVE if cooperative else 0), tokens,
                                    d, _dtype_name_code(dtype), 1 if with_workspace else 0)
    if r < 0:
        raise ValueError(f"path {path!r}, d={d}, {dtype}: {last_error()}")
    return _PATH_NAMES[r]


def fused_step_workspace_bytes(tokens: int, d: int, dtype) -> int:
    """mhc_fused_step_workspace_bytes: the workspace both workspace kernel
    families need (0 when neither applies to (tokens, d, dtype) on the current
    device)."""
    n = load().mhc_fused_step_workspace_bytes(tokens, d, _dtype_name_code(dtype))
    if n < 0:
        raise MhcError("mhc_fused_step_workspace_bytes", MHC_ERR_INVALID_ARG, last_error())
    return n


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of nbytes (the library requires its header to
    be zero before first use and leaves it so after every call)."""
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def workspace_for(device, nbytes: int) -> torch.Tensor:
    """A workspace of at least nbytes, cached per (device, current stream):
    calls that share it are ordered by their stream."""
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(nbytes, device)
        _workspaces[key] = ws
    return ws


def split_status(workspace: torch.Tensor) -> int:
    """The status word of a workspace (synchronises): 0, or 1 if a
    cross-workgroup wait of any feature-split call since the last
    clear_split_status gave up (that call's outputs are invalid)."""
    return int(workspace[:4].view(torch.int32).item())


def clear_split_status(workspace: torch.Tensor) -> None:
    """Write 0 to the status word (on the current stream; the library never
    clears it)."""
    workspace[:4].zero_()


def _raise_on_status(fn, workspace):
    if workspace is not None and split_status(workspace) != 0:
        clear_split_status(workspace)
        raise MhcError(fn, MHC_ERR_HIP, "a cross-workgroup wait of the feature-split kernel "
                       "gave up; the outputs of this call are invalid")


def fused_step(x, f, pre_in, post_in, comb_in, w_packed, base, scale, gamma, iters=20,
               norm_eps=1e-6, hc_eps=1e-6, x_out=None, y_out=None, pre_out=None, post_out=None,
               comb_out=None, mix_out=None, want_mix=False, path="auto", workspace=None,
               check_status=False, cooperative=False) -> dict:
    """mhc_fused_step on tensors. x [T,4,d], f [T,d] (bf16 or f32); coefficients
    and parameters float32. Returns dict(x_out, y, pre, post, comb, mix).

    path: "tile" (no workspace), "split" (feature-split kernel), "chunk" (chunked
    kernels; both raise ValueError where they do not apply), or "auto" (the
    library's choice by size, with a workspace where one applies). workspace:
    optional zero-initialised uint8 tensor (new_workspace; a cached one is used
    otherwise). check_status: synchronise after the call and raise MhcError if
    the workspace's status word is set (it is cleared then). cooperative: OR
    MHC_PATH_COOPERATIVE into the path (a cooperative launch of the
    feature-split kernel instead of an ordinary one)."""
    t, n, d = x.shape
    if n != N_STREAMS:
        raise ValueError("x must be [T, 4, d]")
    code, ws_ptr, ws_bytes, ws = _workspace_arg(x, t, d, path, workspace)
    code |= COOPERATIVE if cooperative else 0
    x_out = torch.empty_like(x) if x_out is None else x_out
    y_out = torch.empty_like(f) if y_out is None else y_out
    pre_out = _f32_out((t, N_STREAMS), x, pre_out)
    post_out = _f32_out((t, N_STREAMS), x, post_out)
    comb_out = _f32_out((t, N_STREAMS, N_STREAMS), x, comb_out)
    if want_mix and mix_out is None:
        mix_out = _f32_out((t, N_MIX), x, None)
    st = load().mhc_fused_step(
        _ptr(x), _ptr(f), _dtype_code(x), t, d, _ptr(pre_in), _ptr(post_in), _ptr(comb_in),
        _ptr(w_packed), _ptr(base), _ptr(scale), _ptr(gamma), iters, norm_eps, hc_eps,
        _ptr(x_out), _ptr(y_out), _ptr(pre_out), _ptr(post_out), _ptr(comb_out), _ptr(mix_out),
        code, ws_ptr, ws_bytes, _stream())
    _check("mhc_fused_step", st)
    if check_status:
        _raise_on_status("mhc_fused_step", ws)
    return {"x_out": x_out, "y": y_out, "pre": pre_out, "post": post_out, "comb": comb_out,
            "mix": mix_out}


def fused_step_noalloc(x, f, pre_in, post_in, comb_in, w_packed, base, scale, gamma, iters=20,
                       norm_eps=1e-6, hc_eps=1e-6, x_out=None, y_out=None, pre_out=None,
                       post_out=None, comb_out=None, mix_out=None, want_mix=False,
                       path="auto", cooperative=False) -> dict:
    """mhc_fused_step_noalloc on tensors: fused_step with the library's static
    scratch as the workspace (no device allocation by the library; outputs
    not given are allocated here by torch). cooperative as for fused_step."""
    t, n, d = x.shape
    if n != N_STREAMS:
        raise ValueError("x must be [T, 4, d]")
    if path not in PATHS:
        raise ValueError(f"unknown path {path!r}")
    x_out = torch.empty_like(x) if x_out is None else x_out
    y_out = torch.empty_like(f) if y_out is None else y_out
    pre_out = _f32_out((t, N_STREAMS), x, pre_out)
    post_out = _f32_out((t, N_STREAMS), x, post_out)
    comb_out = _f32_out((t, N_STREAMS, N_STREAMS), x, comb_out)
    if want_mix and mix_out is None:
        mix_out = _f32_out((t, N_MIX), x, None)
    st = load().mhc_fused_step_noalloc(
        _ptr(x), _ptr(f), _dtype_code(x), t, d, _ptr(pre_in), _ptr(post_in), _ptr(comb_in),
        _ptr(w_packed), _ptr(base), _ptr(scale), _ptr(gamma), iters, norm_eps, hc_eps,
        _ptr(x_out), _ptr(y_out), _ptr(pre_out), _ptr(post_out), _ptr(comb_out), _ptr(mix_out),
        PATHS[path] | (COOPERATIVE if cooperative else 0), _stream())
    _check("mhc_fused_step_noalloc", st)
    return {"x_out": x_out, "y": y_out, "pre": pre_out, "post": post_out, "comb": comb_out,
            "mix": mix_out}


def _workspace_arg(x, t, d, path, workspace):
    """(mhc_path code, workspace pointer, workspace bytes, workspace tensor or
    None) for path "auto" / "tile" / "split" / "chunk"."""
    if path not in PATHS:
        raise ValueError(f"unknown path {path!r}")
    if path == "tile":
        return PATHS["tile"], None, 0, None
    if path != "auto":
        fused_step_route(path, t, d, _dtype_code(x))   # raises where the path does not apply
    need = fused_step_workspace_bytes(t, d, _dtype_code(x))
    if need == 0:
        return PATHS[path], None, 0, None
    if workspace is None:
        workspace = workspace_for(x.device, need)
    return (PATHS[path], _ptr(workspace), workspace.numel() * workspace.element_size(),
            workspace)


def mixes(x, w_packed, base, scale, iters=20, norm_eps=1e-6, hc_eps=1e-6, pre_out=None,
          post_out=None, comb_out=None, mix_out=None, want_mix=False, path="auto",
          workspace=None, check_status=False, cooperative=False) -> dict:
    """mhc_mixes on tensors. Returns dict(pre, post, comb, mix). path,
    workspace, check_status and cooperative as for fused_step."""
    t, n, d = x.shape
    if n != N_STREAMS:
        raise ValueError("x must be [T, 4, d]")
    code, ws_ptr, ws_bytes, ws = _workspace_arg(x, t, d, path, workspace)
    code |= COOPERATIVE if cooperative else 0
    pre_out = _f32_out((t, N_STREAMS), x, pre_out)
    post_out = _f32_out((t, N_STREAMS), x, post_out)
    comb_out = _f32_out((t, N_STREAMS, N_STREAMS), x, comb_out)
    if want_mix and mix_out is None:
        mix_out = _f32_out((t, N_MIX), x, None)
    st = load().mhc_mixes(_ptr(x), _dtype_code(x), t, d, _ptr(w_packed), _ptr(base), _ptr(scale),
                          iters, norm_eps, hc_eps, _ptr(pre_out), _ptr(post_out), _ptr(comb_out),
                          _ptr(mix_out), code, ws_ptr, ws_bytes, _stream())
    _check("mhc_mixes", st)
    if check_status:
        _raise_on_status("mhc_mixes", ws)
    return {"pre": pre_out, "post": post_out, "comb": comb_out, "mix": mix_out}


def sinkhorn4(mix, base, scale, iters=20, hc_eps=1e-6, pre_out=None, post_out=None,
              comb_out=None) -> dict:
    """mhc_sinkhorn4 on tensors: mix [T, 24] float32. Returns dict(pre, post, comb)."""
    t = mix.shape[0]
    pre_out = _f32_out((t, N_STREAMS), mix, pre_out)
    post_out = _f32_out((t, N_STREAMS), mix, post_out)
    comb_out = _f32_out((t, N_STREAMS, N_STREAMS), mix, comb_out)
    st = load().mhc_sinkhorn4(_ptr(mix), t, _ptr(base), _ptr(scale), iters, hc_eps,
                              _ptr(pre_out), _ptr(post_out), _ptr(comb_out), _stream())
    _check("mhc_sinkhorn4", st)
    return {"pre": pre_out, "post": post_out, "comb": comb_out}


def hc_post(x, f, post_in, comb_in, x_out=None):
    """mhc_hc_post: new streams x_out [T,4,d] = S(comb^T x + post * f)."""
    t, n, d = x.shape
    x_out = torch.empty_like(x) if x_out is None else x_out
    _check("mhc_hc_post", load().mhc_hc_post(_ptr(x), _ptr(f), _dtype_code(x), t, d, _ptr(post_in),
                                             _ptr(comb_in), _ptr(x_out), _stream()))
    return x_out


def hc_pre(x, pre_in, h_out=None):
    """mhc_hc_pre: h [T,d] = S(sum_k pre_k x_k)."""
    t, n, d = x.shape
    h_out = torch.empty((t, d), dtype=x.dtype, device=x.device) if h_out is None else h_out
    _check("mhc_hc_pre", load().mhc_hc_pre(_ptr(x), _dtype_code(x), t, d, _ptr(pre_in),
                                           _ptr(h_out), _stream()))
    return h_out


def rmsnorm(h, gamma, norm_eps=1e-6, y_out=None):
    """mhc_rmsnorm: y [T,d] = S(gamma * h / rms(h))."""
    t, d = h.shape
    y_out = torch.empty_like(h) if y_out is None else y_out
    _check("mhc_rmsnorm", load().mhc_rmsnorm(_ptr(h), _dtype_code(h), t, d, _ptr(gamma), norm_eps,
                                             _ptr(y_out), _stream()))
    return y_out


def three_kernel_step(x, f, pre_in, post_in, comb_in, w_packed, base, scale, gamma, iters=20,
                      norm_eps=1e-6, hc_eps=1e-6, want_mix=False, path="auto", workspace=None,
                      x_out=None, h_out=None, y_out=None) -> dict:
    """The step as the pages run it, one kernel per operation: hc_post, hc_mixes,
    hc_pre, RMSNorm. Same outputs as fused_step (plus h)."""
    xo = hc_post(x, f, post_in, comb_in, x_out=x_out)
    m = mixes(xo, w_packed, base, scale, iters, norm_eps, hc_eps, want_mix=want_mix, path=path,
              workspace=workspace)
    h = hc_pre(xo, pre_in, h_out=h_out)
    y = rmsnorm(h, gamma, norm_eps, y_out=y_out)
    return {"x_out": xo, "y": y, "pre": m["pre"], "post": m["post"], "comb": m["comb"],
            "mix": m["mix"], "h": h}


# ----- any stream count n in {2, 4, 8} (the *_n entry points) -----------------------------

def n_mix(n: int) -> int:
    return (2 + n) * n


def wmix_packed_bytes_n(n: int, d: int, dtype) -> int:
    return load().mhc_wmix_packed_bytes_n(n, d, _dtype_name_code(dtype))


def pack_wmix_n(w_mix: torch.Tensor, dtype, out: torch.Tensor | None = None) -> torch.Tensor:
    """mhc_pack_wmix_n: float32 W [(2+n)n, n*d] -> packed operand buffer (uint8)."""
    code = _dtype_name_code(dtype)
    rows, cols = w_mix.shape
    n = next((k for k in (2, 4, 8) if n_mix(k) == rows), None)
    if n is None or cols % n:
        raise ValueError(f"w_mix shape {tuple(w_mix.shape)} is not [(2+n)n, n*d] for n in 2, 4, 8")
    d = cols // n
    nbytes = load().mhc_wmix_packed_bytes_n(n, d, code)
    if nbytes < 0:
        raise ValueError(f"width {d} is not a positive multiple of {d_granule()}")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w_mix.device)
    _check("mhc_pack_wmix_n", load().mhc_pack_wmix_n(n, _ptr(w_mix), d, code, _ptr(out),
                                                     out.numel() * out.element_size(), _stream()))
    return out


def fused_step_n_workspace_bytes(n: int, tokens: int, d: int, dtype) -> int:
    """mhc_fused_step_n_workspace_bytes: the workspace both workspace routes of
    the n-family need (0 when neither applies to (n, tokens, d, dtype) on the
    current device)."""
    b = load().mhc_fused_step_n_workspace_bytes(n, tokens, d, _dtype_name_code(dtype))
    if b < 0:
        raise MhcError("mhc_fused_step_n_workspace_bytes", MHC_ERR_INVALID_ARG, last_error())
    return b


# path names of the n-family ("block" is the token-block kernel, MHC_PATH_TILE)
PATHS_N = {"auto": 0, "block": 1, "split": 2, "chunk": 3}
_PATH_NAMES_N = {v: k for k, v in PATHS_N.items()}


def fused_step_route_n(n: int, path: str, tokens: int, d: int, dtype,
                       with_workspace=True) -> str:
    """mhc_fused_step_route_n: the kernel family ("block", "split" or "chunk")
    that fused_step_n / mixes_n run for `path`; ValueError if that path cannot
    run these arguments."""
    if path not in PATHS_N:
        raise ValueError(f"unknown path {path!r}")
    r = load().mhc_fused_step_route_n(n, PATHS_N[path], tokens, d, _dtype_name_code(dtype),
                                      1 if with_workspace else 0)
    if r < 0:
        raise ValueError(f"path {path!r}, n={n}, d={d}, {dtype}: {last_error()}")
    return _PATH_NAMES_N[r]


def _workspace_arg_n(x, n, t, d, path, workspace):
    """(mhc_path code, workspace pointer, workspace bytes, workspace tensor or
    None) of the n-family for path "block" / "split" / "chunk" (both raise
    ValueError where they do not apply) / "auto"."""
    if path not in PATHS_N:
        raise ValueError(f"unknown path {path!r}")
    if path == "block":
        return PATHS_N["block"], None, 0, None
    if path != "auto":
        fused_step_route_n(n, path, t, d, _dtype_code(x))   # raises where it does not apply
    need = fused_step_n_workspace_bytes(n, t, d, _dtype_code(x))
    if need == 0:
        return PATHS_N[path], None, 0, None
    if workspace is None:
        workspace = workspace_for(x.device, need)
    return (PATHS_N[path], _ptr(workspace), workspace.numel() * workspace.element_size(),
            workspace)


def fused_step_n(x, f, pre_in, post_in, comb_in, w_packed, base, scale, gamma, iters=20,
                 norm_eps=1e-6, hc_eps=1e-6, x_out=None, y_out=None, pre_out=None, post_out=None,
                 comb_out=None, mix_out=None, path="auto", workspace=None,
                 check_status=False, cooperative=False) -> dict:
    """mhc_fused_step_n on tensors: x [T,n,d], f [T,d]; w_packed from pack_wmix_n.
    Returns dict(x_out, y, pre, post, comb, mix) (mix is always produced).
    path: "block" (no workspace), "split" (feature-split kernel: n in {2, 4},
    bf16), "chunk" (the block kernel in chunks of the features, up to 8192
    tokens) or "auto" (the library's choice by size); workspace: optional
    zero-initialised uint8 tensor (a cached one is used otherwise);
    check_status and cooperative as for fused_step."""
    t, n, d = x.shape
    code, ws_ptr, ws_bytes, ws = _workspace_arg_n(x, n, t, d, path, workspace)
    code |= COOPERATIVE if cooperative else 0
    x_out = torch.empty_like(x) if x_out is None else x_out
    y_out = torch.empty_like(f) if y_out is None else y_out
    pre_out = _f32_out((t, n), x, pre_out)
    post_out = _f32_out((t, n), x, post_out)
    comb_out = _f32_out((t, n, n), x, comb_out)
    mix_out = _f32_out((t, n_mix(n)), x, mix_out)
    st = load().mhc_fused_step_n(
        n, _ptr(x), _ptr(f), _dtype_code(x), t, d, _ptr(pre_in), _ptr(post_in), _ptr(comb_in),
        _ptr(w_packed), _ptr(base), _ptr(scale), _ptr(gamma), iters, norm_eps, hc_eps,
        _ptr(x_out), _ptr(y_out), _ptr(pre_out), _ptr(post_out), _ptr(comb_out), _ptr(mix_out),
        code, ws_ptr, ws_bytes, _stream())
    _check("mhc_fused_step_n", st)
    if check_status:
        _raise_on_status("mhc_fused_step_n", ws)
    return {"x_out": x_out, "y": y_out, "pre": pre_out, "post": post_out, "comb": comb_out,
            "mix": mix_out}


def mixes_n(x, w_packed, base, scale, iters=20, norm_eps=1e-6, hc_eps=1e-6, pre_out=None,
            post_out=None, comb_out=None, mix_out=None, path="auto", workspace=None,
            check_status=False, cooperative=False) -> dict:
    """mhc_mixes_n on tensors: x [T,n,d]. Returns dict(pre, post, comb, mix).
    path, workspace, check_status and cooperative as for fused_step_n."""
    t, n, d = x.shape
    code, ws_ptr, ws_bytes, ws = _workspace_arg_n(x, n, t, d, path, workspace)
    code |= COOPERATIVE if cooperative else 0
    pre_out = _f32_out((t, n), x, pre_out)
    post_out = _f32_out((t, n), x, post_out)
    comb_out = _f32_out((t, n, n), x, comb_out)
    mix_out = _f32_out((t, n_mix(n)), x, mix_out)
    st = load().mhc_mixes_n(n, _ptr(x), _dtype_code(x), t, d, _ptr(w_packed), _ptr(base),
                            _ptr(scale), iters, norm_eps, hc_eps, _ptr(pre_out), _ptr(post_out),
                            _ptr(comb_out), _ptr(mix_out), code, ws_ptr, ws_bytes,
                            _stream())
    _check("mhc_mixes_n", st)
    if check_status:
        _raise_on_status("mhc_mixes_n", ws)
    return {"pre": pre_out, "post": post_out, "comb": comb_out, "mix": mix_out}


def sinkhorn_n(n, mix, base, scale, iters=20, hc_eps=1e-6, pre_out=None, post_out=None,
               comb_out=None) -> dict:
    """mhc_sinkhorn_n on tensors: mix [T, (2+n)n] float32. Returns dict(pre, post, comb)."""
    t = mix.shape[0]
    pre_out = _f32_out((t, n), mix, pre_out)
    post_out = _f32_out((t, n), mix, post_out)
    comb_out = _f32_out((t, n, n), mix, comb_out)
    st = load().mhc_sinkhorn_n(n, _ptr(mix), t, _ptr(base), _ptr(scale), iters, hc_eps,
                               _ptr(pre_out), _ptr(post_out), _ptr(comb_out), _stream())
    _check("mhc_sinkhorn_n", st)
    return {"pre": pre_out, "post": post_out, "comb": comb_out}


# ----- backward of the step (n in {2, 4}) --------------------------------------------------

def fused_step_backward_workspace_bytes_n(n: int, tokens: int, d: int) -> int:
    b = load().mhc_fused_step_backward_workspace_bytes_n(n, tokens, d)
    if b < 0:
        raise MhcError("mhc_fused_step_backward_workspace_bytes_n", MHC_ERR_INVALID_ARG,
                       last_error())
    return b


def fused_step_backward_n(x, f, pre_in, post_in, comb_in, x_out, mix, w_mix, base, scale, gamma,
                          d_x_out, d_y, d_pre, d_post, d_comb, iters=20, norm_eps=1e-6,
                          hc_eps=1e-6, workspace=None) -> dict:
    """mhc_fused_step_backward_n on tensors. Forward inputs (x [T,n,d], f,
    pre_in, post_in, comb_in), the forward's saved outputs (x_out, mix), the
    float32 parameters (w_mix [(2+n)n, nd] unpacked, base, scale, gamma) and
    the upstream gradients (d_x_out, d_y in the stream dtype; d_pre, d_post,
    d_comb float32). Returns the gradients d_x, d_f (stream dtype), d_pre_in,
    d_post_in, d_comb_in, d_w_mix, d_base, d_scale, d_gamma (float32)."""
    t, n, d = x.shape
    nm = n_mix(n)
    dev = x.device
    need = fused_step_backward_workspace_bytes_n(n, t, d)
    if workspace is None:
        workspace = workspace_for(dev, need)
    out = {"d_x": torch.empty_like(x), "d_f": torch.empty_like(f),
           "d_pre_in": torch.empty((t, n), device=dev), "d_post_in": torch.empty((t, n), device=dev),
           "d_comb_in": torch.empty((t, n, n), device=dev),
           "d_w_mix": torch.empty((nm, n * d), device=dev), "d_base": torch.empty(nm, device=dev),
           "d_scale": torch.empty(3, device=dev), "d_gamma": torch.empty(d, device=dev)}
    st = load().mhc_fused_step_backward_n(
        n, _ptr(x), _ptr(f), _dtype_code(x), t, d, _ptr(pre_in), _ptr(post_in), _ptr(comb_in),
        _ptr(x_out), _ptr(mix), _ptr(w_mix), _ptr(base), _ptr(scale), _ptr(gamma), iters,
        norm_eps, hc_eps, _ptr(d_x_out), _ptr(d_y), _ptr(d_pre), _ptr(d_post), _ptr(d_comb),
        _ptr(out["d_x"]), _ptr(out["d_f"]), _ptr(out["d_pre_in"]), _ptr(out["d_post_in"]),
        _ptr(out["d_comb_in"]), _ptr(out["d_w_mix"]), _ptr(out["d_base"]), _ptr(out["d_scale"]),
        _ptr(out["d_gamma"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream())
    _check("mhc_fused_step_backward_n", st)
    return out

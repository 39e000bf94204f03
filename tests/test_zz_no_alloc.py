"""The allocation-free entry point (mhc_fused_step_noalloc) through the C ABI,
against mhc_fused_step with its own zero-filled workspace on the same inputs:
the outputs must be equal bit for bit (same kernels), on two calls in a row
with the second smaller, and on a route of each kind. A call whose route
needs more than the static scratch is rejected before any launch."""

import numpy as np
import pytest
import torch

import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, to_dev
from tests.parity import check_step

pytestmark = pytest.mark.gpu


def _dev(case):
    return {k: to_dev(case[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base",
                                         "scale", "gamma")}


def _both(case, path):
    dev = _dev(case)
    wp = mhc.pack_wmix(dev["w_mix"], "bf16")
    args = (dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp, dev["base"],
            dev["scale"], dev["gamma"], case["iters"], case["norm_eps"], case["hc_eps"])
    got = mhc.fused_step_noalloc(*args, want_mix=True, path=path)
    torch.cuda.synchronize()
    got = {k: v.cpu() for k, v in got.items()}
    ws = mhc.new_workspace(mhc.fused_step_workspace_bytes(len(case["x"]), case["x"].shape[2],
                                                          "bf16"))
    ref = mhc.fused_step(*args, want_mix=True, path=path, workspace=ws)
    torch.cuda.synchronize()
    assert mhc.split_status(ws) == 0
    return got, {k: v.cpu() for k, v in ref.items()}


@pytest.mark.parametrize("first,second", [(6000, 1500), (3000, 300)])
def test_noalloc_matches_the_workspace_entry_point(first, second):
    """Two calls in a row on the same scratch, the second smaller; the first
    pair runs the feature-split kernel twice (20 slices of 256 features, then
    32 of 160), the second pair the split then the chunked kernels (path
    auto: chunks up to 896 tokens)."""
    for i, t in enumerate((first, second)):
        case = make_case(wl.Workload(930 + i + first % 7, "noalloc", t, 5120, "bf16"))
        path = "split" if first == 5000 else "auto"
        got, ref = _both(case, path)
        for k in ("x_out", "y", "pre", "post", "comb", "mix"):
            assert torch.equal(got[k], ref[k]), (t, k)
        idx = np.unique(np.concatenate([np.arange(8), np.arange(t - 8, t)]))
        sub = dict(case)
        for k in ("x", "f", "pre", "post", "comb"):
            sub[k] = case[k][idx]
        check_step(sub, {k: v[idx] for k, v in got.items()}, "bf16")


def test_noalloc_rejects_calls_beyond_the_scratch():
    """200,000 tokens at d = 5120 need about 35 MB on the feature-split route;
    the call is refused before anything is launched (the pointers are never
    dereferenced)."""
    lib = mhc.load()
    t, d = 200_000, 5120
    fake = [0x7f0000000000 + (i << 36) for i in range(16)]
    st = lib.mhc_fused_step_noalloc(fake[0], fake[1], 1, t, d, fake[2], fake[3], fake[4],
                                    fake[5], fake[6], fake[7], fake[8], 20, 1e-6, 1e-6,
                                    fake[9], fake[10], fake[11], fake[12], fake[13], None, 2,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == mhc.binding.MHC_ERR_INVALID_ARG
    assert "static scratch" in mhc.last_error()

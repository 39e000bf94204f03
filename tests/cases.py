"""Builders of seeded test cases shared by the GPU parity tests and smoke().

Inputs come from ``stream_hyper_connections_amd.workloads``; the prior
coefficients (pre, post, comb of the previous sublayer) come from the float64
oracle's ``mixes`` on the same streams with an independent parameter set,
rounded to float32 -- never from the HIP path.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from stream_hyper_connections_amd import workloads as wl


def oracle_prior(x_cpu, prev, iters=20, norm_eps=1e-6, hc_eps=1e-6, chunk=1024):
    """Oracle mixes of the streams with parameters ``prev``, as float32 numpy."""
    t, n = x_cpu.shape[0], x_cpu.shape[1]
    pre = np.empty((t, n), np.float32)
    post = np.empty((t, n), np.float32)
    comb = np.empty((t, n, n), np.float32)
    for t0 in range(0, t, chunk):
        xs = x_cpu[t0:t0 + chunk].double().numpy()
        _, p, u, c = oracle.mixes(xs, prev["w_mix"], prev["base"], prev["scale"], iters,
                                  norm_eps, hc_eps)
        pre[t0:t0 + chunk], post[t0:t0 + chunk], comb[t0:t0 + chunk] = p, u, c
    return pre, post, comb


def make_case(w: wl.Workload, step: int = 0, tokens=None):
    """CPU inputs of one fused step of workload ``w``."""
    x = wl.streams(w, step, tokens)
    f = wl.sublayer_out(w, step, tokens)
    prev = wl.params(w, step, prev=True)
    cur = wl.params(w, step)
    pre, post, comb = oracle_prior(x, prev, w.iters, w.norm_eps, w.hc_eps)
    return dict(x=x, f=f, pre=pre, post=post, comb=comb, iters=w.iters, norm_eps=w.norm_eps,
                hc_eps=w.hc_eps, **cur)


def to_dev(a, dev="cuda"):
    if isinstance(a, torch.Tensor):
        return a.to(dev).contiguous()
    return torch.as_tensor(np.ascontiguousarray(a)).to(dev)


def run_step(case, want_mix=True, dtype="bf16", **kw):
    """Pack the case's projection and run mhc_fused_step on the GPU; returns
    (dict of CPU outputs, dict of device inputs)."""
    import stream_hyper_connections_amd as mhc
    dev = {k: to_dev(case[k]) for k in ("x", "f", "pre", "post", "comb", "w_mix", "base", "scale",
                                        "gamma")}
    wp = mhc.pack_wmix(dev["w_mix"], dtype)
    out = mhc.fused_step(dev["x"], dev["f"], dev["pre"], dev["post"], dev["comb"], wp,
                         dev["base"], dev["scale"], dev["gamma"], case["iters"],
                         case["norm_eps"], case["hc_eps"], want_mix=want_mix, **kw)
    torch.cuda.synchronize()
    return {k: (v.cpu() if v is not None else None) for k, v in out.items()}, dev

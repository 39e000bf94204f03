"""GPU parity for a call whose stream tensors pass 4 GiB (n = 4, d = 5120, bf16).

131,072 tokens: X and X' are 5.37 GB each, so the rows of tokens from 104,858
on start beyond 2^32 bytes, and the 32-bit buffer offsets of the kernels only
ever cover one wave's rows from a 64-bit base. Checked here, on the route that
path "auto" takes at that size (the feature-split kernel and its tail):

* the oracle on every token around the 2^32-byte boundary of X, the last
  tokens and a seeded sample of the upper half;
* the same library on the last 32,768 tokens alone (a call whose base
  pointers sit 4.03 GB into the same tensors, its first token on a 128-token
  batch boundary, so every token keeps its place in its batch): every output
  of those tokens equal bit for bit;
* the comb column sums of every token;
* hc_mixes on the input streams at the same size, sampled against the oracle;
* the general-n entry point at n = 4 on the same inputs, sampled against the
  oracle.

Inputs: streams and sublayer output drawn as every workload's (id 5 of the
seed tree), the prior coefficients from the oracle's mixes of the first 1,024
tokens with an independent parameter set, token t taking those of token
t mod 1,024.
"""

import time

import numpy as np
import pytest
import torch

import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import oracle_prior, to_dev
from tests.parity import check_mixes, check_step, comb_sum_stats
from tests.test_gpu_backward import check_token_grads

pytestmark = pytest.mark.gpu

BIG = wl.Workload(5, "beyond_4gib", 131072, 5120, "bf16", batch=8)   # id 5 of the seed tree
SUFFIX = 32768


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def big():
    """The 131,072-token inputs on the GPU, the CPU rows of the sampled tokens
    and the prior coefficients (numpy, per token of the first chunk)."""
    w = BIG
    t, d = w.tokens, w.d
    row_x = w.n * d * 2
    first_high = (1 << 32) // row_x + 1          # first token whose X row starts past 2^32
    assert t * row_x > (1 << 32) and (first_high - 1) * row_x < (1 << 32)
    rng = np.random.default_rng(5150)
    idx = np.unique(np.concatenate([np.arange(4), np.arange(first_high - 24, first_high + 24),
                                    np.arange(t - 48, t),
                                    rng.choice(np.arange(t // 2, t), 96, replace=False)]))
    t_start = time.time()
    x = torch.empty((t, w.n, d), dtype=torch.bfloat16, device="cuda")
    f = torch.empty((t, d), dtype=torch.bfloat16, device="cuda")
    xs_cpu = torch.empty((len(idx), w.n, d), dtype=torch.bfloat16)
    fs_cpu = torch.empty((len(idx), d), dtype=torch.bfloat16)
    first_x = None
    for (t0, bx), (_, bf) in zip(wl.token_tensor_chunks(w, wl.X), wl.token_tensor_chunks(w, wl.F)):
        cx = wl.to_dtype(bx, "bf16").reshape(-1, w.n, d)
        cf = wl.to_dtype(bf, "bf16")
        x[t0:t0 + len(cx)].copy_(cx)
        f[t0:t0 + len(cf)].copy_(cf)
        if first_x is None:
            first_x = cx
        sel = np.nonzero((idx >= t0) & (idx < t0 + len(cx)))[0]
        xs_cpu[sel] = cx[idx[sel] - t0]
        fs_cpu[sel] = cf[idx[sel] - t0]
    _log(f"beyond_4gib: {t} tokens drawn in {time.time() - t_start:.1f}s")
    pre1, post1, comb1 = oracle_prior(first_x, wl.params(w, prev=True), w.iters, w.norm_eps,
                                      w.hc_eps)
    rep = np.arange(t) % wl.CHUNK
    yield dict(w=w, idx=idx, x=x, f=f, xs_cpu=xs_cpu, fs_cpu=fs_cpu,
               prior=(pre1, post1, comb1),
               dev_prior=(to_dev(pre1[rep]), to_dev(post1[rep]), to_dev(comb1[rep])))
    torch.cuda.empty_cache()


def _sampled_case(b, p):
    w, idx = b["w"], b["idx"]
    pre1, post1, comb1 = b["prior"]
    return dict(x=b["xs_cpu"], f=b["fs_cpu"], pre=pre1[idx % wl.CHUNK],
                post=post1[idx % wl.CHUNK], comb=comb1[idx % wl.CHUNK], iters=w.iters,
                norm_eps=w.norm_eps, hc_eps=w.hc_eps, **p)


@pytest.mark.timeout(900)
def test_step_beyond_4gib(big):
    w, idx, x, f = big["w"], big["idx"], big["x"], big["f"]
    t, d = w.tokens, w.d
    assert mhc.fused_step_route("auto", t, d, "bf16") == "split"
    t_start = time.time()
    pre, post, comb = big["dev_prior"]
    p = wl.params(w)
    base, scale, gamma = to_dev(p["base"]), to_dev(p["scale"]), to_dev(p["gamma"])
    wp = mhc.pack_wmix(to_dev(p["w_mix"]), "bf16")
    ws = mhc.new_workspace(mhc.fused_step_workspace_bytes(t, d, "bf16"))

    out = mhc.fused_step(x, f, pre, post, comb, wp, base, scale, gamma, w.iters, w.norm_eps,
                         w.hc_eps, want_mix=True, workspace=ws, check_status=True)
    torch.cuda.synchronize()
    _log(f"beyond_4gib: fused step done at {time.time() - t_start:.1f}s")

    didx = torch.as_tensor(idx, device="cuda")
    check_step(_sampled_case(big, p), {k: v.index_select(0, didx).cpu() for k, v in out.items()}, "bf16")
    _log(f"beyond_4gib: {len(idx)} sampled tokens (from token {idx[0]} to {idx[-1]}) match "
         "the oracle")

    stats = comb_sum_stats(out["comb"].cpu())
    assert stats["col_dev_max"] <= 1e-5, stats

    s0 = t - SUFFIX
    assert s0 % 128 == 0 and mhc.fused_step_route("auto", SUFFIX, d, "bf16") == "split"
    tail = mhc.fused_step(x[s0:], f[s0:], pre[s0:], post[s0:], comb[s0:], wp, base, scale,
                          gamma, w.iters, w.norm_eps, w.hc_eps, want_mix=True, workspace=ws,
                          check_status=True)
    torch.cuda.synchronize()
    for k in ("x_out", "y", "pre", "post", "comb", "mix"):
        assert torch.equal(tail[k], out[k][s0:]), k
    _log(f"beyond_4gib: the last {SUFFIX} tokens on their own equal the full call bit for bit")
    del out, tail

    mx = mhc.mixes(x, wp, base, scale, w.iters, w.norm_eps, w.hc_eps, want_mix=True,
                   workspace=ws, check_status=True)
    torch.cuda.synchronize()
    check_mixes(dict(x=big["xs_cpu"], iters=w.iters, norm_eps=w.norm_eps, hc_eps=w.hc_eps, **p),
                {k: v.index_select(0, didx).cpu() for k, v in mx.items()}, "bf16")
    _log(f"beyond_4gib: hc_mixes on the input streams matches the oracle on the "
         f"{len(idx)} sampled tokens ({time.time() - t_start:.1f}s)")
    del mx

    # the general-n entry point at n = 4 (its own feature-split kernel)
    route = mhc.fused_step_route_n(4, "auto", t, d, "bf16")
    wpn = mhc.pack_wmix_n(to_dev(p["w_mix"]), "bf16")
    on = mhc.fused_step_n(x, f, pre, post, comb, wpn, base, scale, gamma, w.iters, w.norm_eps,
                          w.hc_eps, check_status=True)
    torch.cuda.synchronize()
    check_step(_sampled_case(big, p), {k: v.index_select(0, didx).cpu() for k, v in on.items()},
               "bf16")
    _log(f"beyond_4gib: fused_step_n (n = 4, route {route}) matches the oracle on the "
         f"{len(idx)} sampled tokens")


@pytest.mark.timeout(900)
def test_backward_beyond_4gib(big):
    """The backward on the same 131,072 tokens: the per-token gradients of the
    sampled tokens against the backward oracle (on the new streams validated
    against the forward oracle); the backward of the upper half alone (base
    pointers 2.7 GB into X, its first token on a workgroup boundary of every
    kernel) equal bit for bit on those tokens; and the parameter gradients of
    the whole call equal to the sums of the two halves' within float32
    regrouping (a misplaced row would move them by its own size)."""
    w, idx, x, f = big["w"], big["idx"], big["x"], big["f"]
    t, d = w.tokens, w.d
    pre, post, comb = big["dev_prior"]
    p = wl.params(w)
    dev_p = {k: to_dev(v) for k, v in p.items()}
    wp = mhc.pack_wmix(dev_p["w_mix"], "bf16")
    fwd = mhc.fused_step(x, f, pre, post, comb, wp, dev_p["base"], dev_p["scale"],
                         dev_p["gamma"], w.iters, w.norm_eps, w.hc_eps, want_mix=True,
                         check_status=True)
    didx = torch.as_tensor(idx, device="cuda")
    o = check_step(_sampled_case(big, p),
                   {k: v.index_select(0, didx).cpu() for k, v in fwd.items()}, "bf16")
    del fwd["y"]
    gen = torch.Generator(device="cuda").manual_seed(5151)
    up = {"d_xprime": torch.randn((t, w.n, d), generator=gen, device="cuda").to(torch.bfloat16),
          "d_y": torch.randn((t, d), generator=gen, device="cuda").to(torch.bfloat16),
          "d_pre": torch.randn((t, w.n), generator=gen, device="cuda"),
          "d_post": torch.randn((t, w.n), generator=gen, device="cuda"),
          "d_comb": torch.randn((t, w.n, w.n), generator=gen, device="cuda")}

    def backward(lo, hi):
        g = mhc.fused_step_backward_n(x[lo:hi], f[lo:hi], pre[lo:hi], post[lo:hi], comb[lo:hi],
                                      fwd["x_out"][lo:hi], fwd["mix"][lo:hi], dev_p["w_mix"],
                                      dev_p["base"], dev_p["scale"], dev_p["gamma"],
                                      *(up[k][lo:hi] for k in ("d_xprime", "d_y", "d_pre",
                                                                "d_post", "d_comb")),
                                      w.iters, w.norm_eps, w.hc_eps)
        torch.cuda.synchronize()
        return g

    t_start = time.time()
    full = backward(0, t)
    _log(f"beyond_4gib backward: {t} tokens in one call ({time.time() - t_start:.1f}s)")
    up_s = {k: v.index_select(0, didx).cpu().double().numpy() for k, v in up.items()}
    got_s = {k: full[k].index_select(0, didx).cpu()
             for k in ("d_x", "d_f", "d_comb_in", "d_post_in", "d_pre_in")}
    _, used = check_token_grads(_sampled_case(big, p), got_s, up_s, o["xprime"], w.iters, "bf16")
    _log(f"beyond_4gib backward: {len(idx)} sampled tokens match the oracle "
         + ", ".join(f"{k} {v:.1e}" for k, v in used.items()))

    half = t // 2
    parts = []
    for lo, hi in ((0, half), (half, t)):
        parts.append({k: v for k, v in backward(lo, hi).items()
                      if k in ("d_w_mix", "d_gamma", "d_base", "d_scale")
                      or (lo == half and k in ("d_x", "d_f", "d_comb_in", "d_post_in",
                                               "d_pre_in"))})
    for k in ("d_x", "d_f", "d_comb_in", "d_post_in", "d_pre_in"):
        assert torch.equal(parts[1][k], full[k][half:]), k
    for k in ("d_w_mix", "d_gamma", "d_base", "d_scale"):
        a, b = parts[0][k].double(), parts[1][k].double()
        tol = 1e-3 * (a.abs() + b.abs()) + 1e-5 * b.abs().max()
        diff = (full[k].double() - (a + b)).abs()
        assert bool((diff <= tol).all()), (k, float((diff / tol).max()))
    _log("beyond_4gib backward: the upper half alone equals the full call per token bit for "
         "bit; parameter gradients = lower + upper half")

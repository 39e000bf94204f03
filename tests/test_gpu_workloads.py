"""GPU parity on the five synthetic workloads (n = 4, d = 5120):

* tiny (64 tokens, f32) and decode (256 tokens, bf16, 1% outlier tokens x30):
  every output of every token against the oracle;
* prefill (4,096 tokens): every token;
* large prefill (65,536 tokens, the throughput shape, launched exactly as the
  benchmark launches it): every token, in 1,024-token chunks;
* chain (8,192 tokens x 80 sublayer steps, fresh parameters per step, each
  step's outputs feeding the next): at steps 1, 40 and 80 every token against
  the oracle applied to exactly the inputs the GPU consumed; at every step
  sampled tokens against the oracle carried alongside, comb column sums of
  every token, the workspace status word, and drift statistics of a
  free-running oracle chain (reported).
"""

import time

import numpy as np
import pytest
import torch

import oracle
import stream_hyper_connections_amd as mhc
from stream_hyper_connections_amd import workloads as wl
from tests.cases import make_case, oracle_prior, run_step, to_dev
from tests.parity import check_step, coef_gap, comb_sum_stats

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _sub(case, idx):
    out = dict(case)
    for k in ("x", "f", "pre", "post", "comb"):
        out[k] = case[k][idx]
    return out


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_workload_full(name):
    w = wl.WORKLOADS[name]
    _log(f"workload {name}: T={w.tokens} dtype={w.dtype}")
    case = make_case(w)
    out, _ = run_step(case, dtype=w.dtype)
    for t0 in range(0, w.tokens, 512):
        sl = slice(t0, t0 + 512)
        check_step(_sub(case, sl), {k: (v[sl] if v is not None else None) for k, v in out.items()},
                   w.dtype)
    _log(f"  comb sums: {comb_sum_stats(out['comb'])}")


def _check_chunked(case, out, dtype, chunk=1024):
    t = len(case["x"])
    for t0 in range(0, t, chunk):
        sl = slice(t0, min(t, t0 + chunk))
        check_step(_sub(case, sl), {k: (v[sl] if v is not None else None) for k, v in out.items()},
                   dtype)


@pytest.mark.timeout(900)
def test_workload_large_prefill_full():
    w = wl.WORKLOADS["large_prefill"]
    t = w.tokens
    t_start = time.time()
    x = wl.streams(w)
    f = wl.sublayer_out(w)
    prev, cur = wl.params(w, prev=True), wl.params(w)
    _log(f"large_prefill: inputs drawn in {time.time() - t_start:.1f}s")
    pre, post, comb = oracle_prior(x, prev)
    _log(f"large_prefill: oracle prior done at {time.time() - t_start:.1f}s")
    case = dict(x=x, f=f, pre=pre, post=post, comb=comb, iters=w.iters, norm_eps=w.norm_eps,
                hc_eps=w.hc_eps, **cur)
    ws = mhc.new_workspace(mhc.fused_step_workspace_bytes(t, w.d, "bf16"))
    out, _ = run_step(case, workspace=ws)
    assert mhc.split_status(ws) == 0, "a cross-workgroup wait gave up"
    _log(f"large_prefill: GPU step done at {time.time() - t_start:.1f}s")
    _check_chunked(case, out, "bf16")
    stats = comb_sum_stats(out["comb"])
    assert stats["col_dev_max"] <= 1e-5
    _log(f"large_prefill: all {t} tokens match the oracle at {time.time() - t_start:.1f}s; "
         f"comb sums {stats}")
    # the same inputs cut to a ragged last batch (511 whole 128-token batches
    # and 37 tokens), in the same launch configuration
    t2 = 511 * 128 + 37
    sub = dict(case, x=case["x"][:t2], f=case["f"][:t2], pre=pre[:t2], post=post[:t2],
               comb=comb[:t2])
    out2, _ = run_step(sub, workspace=ws)
    assert mhc.split_status(ws) == 0, "a cross-workgroup wait gave up"
    rng = np.random.default_rng(12345)
    idx2 = np.unique(np.concatenate([np.arange(8), np.arange(t2 - 64, t2),
                                     rng.choice(t2, 120, replace=False)]))
    check_step(_sub(sub, idx2), {k: (v[idx2] if v is not None else None)
                                 for k, v in out2.items()}, "bf16")
    for k in ("x_out", "y", "pre", "post", "comb", "mix"):   # tokens before the cut unchanged
        assert torch.equal(out2[k][:t2 - 37], out[k][:t2 - 37]), k
    _log(f"large_prefill cut to {t2} tokens: {len(idx2)} sampled tokens match, the whole "
         "batches equal the full run bit for bit")


@pytest.mark.timeout(900)
def test_workload_chain():
    w = wl.WORKLOADS["chain"]
    t = w.tokens
    rng = np.random.default_rng(777)
    idx = np.unique(np.concatenate([[0, t - 1], rng.choice(t, 62, replace=False)]))
    x0 = wl.streams(w, 0)
    pre, post, comb = oracle_prior(x0, wl.params(w, 0, prev=True))
    dev_x = to_dev(x0)
    dev_c = {"pre": to_dev(pre), "post": to_dev(post), "comb": to_dev(comb)}
    # oracle state on the sampled tokens: teacher-forced (tie choices as on the
    # GPU) and free-running
    tf = {"x": x0[idx].double().numpy(), "pre": pre[idx].astype(np.float64),
          "post": post[idx].astype(np.float64), "comb": comb[idx].astype(np.float64)}
    free = {k: v.copy() for k, v in tf.items()}
    gap = np.zeros(len(idx))
    max_ties = 0
    ws = mhc.new_workspace(mhc.fused_step_workspace_bytes(t, w.d, "bf16"))
    full_steps = (0, 39, w.steps - 1)     # steps 1, 40 and 80: every token
    for s in range(w.steps):
        p = wl.params(w, s)
        f_cpu = wl.sublayer_out(w, s)
        wp = mhc.pack_wmix(to_dev(p["w_mix"]), "bf16")
        if s in full_steps:   # exactly the inputs the GPU consumes at this step
            consumed = dict(x=dev_x.cpu(), f=f_cpu, pre=dev_c["pre"].cpu().numpy(),
                            post=dev_c["post"].cpu().numpy(), comb=dev_c["comb"].cpu().numpy(),
                            iters=w.iters, norm_eps=w.norm_eps, hc_eps=w.hc_eps, **p)
        out = mhc.fused_step(dev_x, to_dev(f_cpu), dev_c["pre"], dev_c["post"], dev_c["comb"], wp,
                             to_dev(p["base"]), to_dev(p["scale"]), to_dev(p["gamma"]),
                             w.iters, w.norm_eps, w.hc_eps, want_mix=True, workspace=ws)
        assert mhc.split_status(ws) == 0, f"step {s}: a cross-workgroup wait gave up"
        if s in full_steps:
            _check_chunked(consumed, {k: (v.cpu() if v is not None else None)
                                      for k, v in out.items()}, "bf16")
            _log(f"chain step {s + 1}: all {t} tokens match the oracle on the inputs consumed")
        didx = torch.as_tensor(idx, device="cuda")
        g = {k: v.index_select(0, didx).cpu() for k, v in out.items() if v is not None}
        col = out["comb"].sum(dim=1)
        assert (col - 1).abs().max().item() <= 1e-5, f"step {s}: column sums"
        inputs = dict(x=tf["x"], f=f_cpu[idx], pre=tf["pre"], post=tf["post"], comb=tf["comb"],
                      iters=w.iters, norm_eps=w.norm_eps, hc_eps=w.hc_eps, **p)
        o = check_step(inputs, g, "bf16", coef_abs=gap)
        max_ties = max(max_ties, o["n_ties"])
        gap = coef_gap(g, o)
        tf = {"x": o["xprime"], "pre": o["pre"], "post": o["post"], "comb": o["comb"]}
        fo = oracle.fused_step(free["x"], f_cpu[idx].double().numpy(), free["pre"], free["post"],
                               free["comb"], p["w_mix"], p["base"], p["scale"], p["gamma"],
                               w.iters, w.norm_eps, w.hc_eps, "bf16")
        free = {"x": fo["xprime"], "pre": fo["pre"], "post": fo["post"], "comb": fo["comb"]}
        dev_x = out["x_out"]
        dev_c = {k: out[k] for k in ("pre", "post", "comb")}
        if s % 10 == 9 or s == w.steps - 1:
            gx = g["x_out"].double().numpy()
            drift = np.linalg.norm(gx - free["x"]) / np.linalg.norm(free["x"])
            rms = float(np.sqrt(np.mean(gx ** 2)))
            _log(f"chain step {s + 1}: sampled parity ok, max coef gap {gap.max():.2e}, "
                 f"ties {o['n_ties']}, stream rms {rms:.3f}, free-running drift {drift:.2e}, "
                 f"comb {comb_sum_stats(out['comb'])}")
    torch.cuda.synchronize()

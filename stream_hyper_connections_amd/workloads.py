"""Seeded synthetic inputs for the mHC step.

This module only draws random numbers and converts dtypes; it holds none of the
step's arithmetic, so the HIP path, the tests and the float64 oracle can all
use it. Every draw comes from ``numpy.random.default_rng`` seeded with
``SeedSequence([20261202, workload_id, tensor_id, step, chunk])``; token-indexed
tensors are drawn in chunks of ``CHUNK`` tokens so that any token's inputs can
be regenerated on its own.

Workloads (n = 4 streams, d = 5120):

====  =================  ==========  ======  =========================================
id    name               tokens      dtype   notes
====  =================  ==========  ======  =========================================
0     tiny               64          f32     correctness case
1     prefill            4096        bf16
2     decode             256         bf16    1% of tokens (3) scaled by 30
3     large_prefill      65536       bf16    4 x 16384; the throughput workload
4     chain              8192 x 80   bf16    80 sublayer steps, fresh params per step
====  =================  ==========  ======  =========================================

Id 5 is a test case past 4 GiB of streams (131,072 tokens, bf16), drawn the
same way. Other stream counts n (2 or 8) use the same recipe with n streams and
(2+n)*n mixes; at n = 4 the draws are those of the table above.

Distributions: streams X and sublayer output F ~ N(0, 1); W_mix [(2+n)n, nd]
~ N(0, 0.02); base [(2+n)n] ~ N(0, 0.1); scale [3] ~ U(0.5, 2); gamma [d] ~ 1 +
N(0, 0.05). N(mu, s) names the standard deviation s. Values are drawn in
float32 and rounded to bf16 (round-to-nearest-even) where the workload is bf16.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED = 20261202
CHUNK = 1024
N_STREAMS = 4
N_MIX = 24

# tensor ids of the seed tree
X, F, W, BASE, SCALE, GAMMA, W_PREV, BASE_PREV, SCALE_PREV, OUTLIERS = range(10)


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    tokens: int
    d: int
    dtype: str            # "bf16" or "f32"
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    steps: int = 1
    iters: int = 20
    norm_eps: float = 1e-6
    hc_eps: float = 1e-6
    batch: int = 1
    n: int = N_STREAMS

    @property
    def n_mix(self) -> int:
        return (2 + self.n) * self.n

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.tokens))


WORKLOADS = {
    "tiny": Workload(0, "tiny", 64, 5120, "f32"),
    "prefill": Workload(1, "prefill", 4096, 5120, "bf16"),
    "decode": Workload(2, "decode", 256, 5120, "bf16", outlier_frac=0.01, outlier_scale=30.0,
                       batch=256),
    "large_prefill": Workload(3, "large_prefill", 65536, 5120, "bf16", batch=4),
    "chain": Workload(4, "chain", 8192, 5120, "bf16", steps=80),
}


def _rng(wid: int, tensor: int, step: int = 0, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, wid, tensor, step, chunk]))


def to_dtype(a32: np.ndarray, dtype: str):
    """float32 array -> torch CPU tensor of the stream dtype (RNE for bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def outlier_tokens(wl: Workload) -> np.ndarray:
    """Sorted token indices scaled by ``outlier_scale`` (a seeded permutation)."""
    if wl.n_outliers == 0:
        return np.zeros(0, dtype=np.int64)
    perm = _rng(wl.wid, OUTLIERS).permutation(wl.tokens)
    return np.sort(perm[: wl.n_outliers])


def _token_chunk(wl: Workload, tensor: int, step: int, c: int, width: int) -> np.ndarray:
    t0 = c * CHUNK
    t1 = min(wl.tokens, t0 + CHUNK)
    a = _rng(wl.wid, tensor, step, c).standard_normal((t1 - t0, width), dtype=np.float32)
    if wl.n_outliers:
        out = outlier_tokens(wl)
        sel = out[(out >= t0) & (out < t1)] - t0
        a[sel] *= np.float32(wl.outlier_scale)
    return a


def token_rows(wl: Workload, tensor: int, tokens, step: int = 0) -> np.ndarray:
    """float32 rows of a token-indexed tensor (X: width n*d, F: width d) for the
    given token indices, drawn exactly as the full tensor would be."""
    width = wl.n * wl.d if tensor == X else wl.d
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.empty((len(tokens), width), dtype=np.float32)
    for c in np.unique(tokens // CHUNK):
        blk = _token_chunk(wl, tensor, step, int(c), width)
        sel = np.nonzero(tokens // CHUNK == c)[0]
        out[sel] = blk[tokens[sel] - c * CHUNK]
    return out


def token_tensor_chunks(wl: Workload, tensor: int, step: int = 0):
    """Yield (t0, float32 block) over the whole token range."""
    width = wl.n * wl.d if tensor == X else wl.d
    nchunks = (wl.tokens + CHUNK - 1) // CHUNK
    for c in range(nchunks):
        yield c * CHUNK, _token_chunk(wl, tensor, step, c, width)


def streams(wl: Workload, step: int = 0, tokens=None):
    """X as a torch CPU tensor [T, n, d] in the workload dtype."""
    if tokens is None:
        tokens = np.arange(wl.tokens)
    a = token_rows(wl, X, tokens, step)
    return to_dtype(a, wl.dtype).reshape(len(tokens), wl.n, wl.d)


def sublayer_out(wl: Workload, step: int = 0, tokens=None):
    """F as a torch CPU tensor [T, d] in the workload dtype."""
    if tokens is None:
        tokens = np.arange(wl.tokens)
    a = token_rows(wl, F, tokens, step)
    return to_dtype(a, wl.dtype)


def params(wl: Workload, step: int = 0, prev: bool = False) -> dict:
    """fp32 parameters (numpy) of one sublayer: w_mix [(2+n)n, nd], base
    [(2+n)n], scale [3], gamma [d]. ``prev`` selects the independent set used to make the
    prior coefficients."""
    tw, tb, ts = (W_PREV, BASE_PREV, SCALE_PREV) if prev else (W, BASE, SCALE)
    d = wl.d
    w = (_rng(wl.wid, tw, step).standard_normal((wl.n_mix, wl.n * d), dtype=np.float32)
         * np.float32(0.02))
    b = _rng(wl.wid, tb, step).standard_normal(wl.n_mix, dtype=np.float32) * np.float32(0.1)
    s = _rng(wl.wid, ts, step).uniform(0.5, 2.0, size=3).astype(np.float32)
    g = (np.float32(1.0)
         + _rng(wl.wid, GAMMA, step).standard_normal(d, dtype=np.float32) * np.float32(0.05))
    return {"w_mix": w, "base": b, "scale": s, "gamma": g.astype(np.float32)}

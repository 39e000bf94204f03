"""Pin of the step's composition against the block's forward pass.

"DeepSeek V4.1 · MoE RMSNorm", Code (``Block.forward``) runs, per block:
attention's coefficients from the streams entering the block; the attention
input read with the ``pre_mix`` handed in by the previous block; attention;
``hc_post`` with attention's write weights and comb; then the same for the
feed-forward, whose input is read with ATTENTION's read weights, and the block
hands the feed-forward's read weights to the next block.

The fused step claims to be exactly what happens at one sublayer boundary.
This file writes the block out as its own float64 program (the pages' ``.float()``
arithmetic taken exactly, casts back to the stream dtype), with attention and
the feed-forward replaced by fixed functions, runs two blocks, and checks
``oracle.fused_step`` at both boundaries of the first block's feed-forward:

* attention -> feed-forward: new streams, the feed-forward's normalised input
  and its coefficients;
* feed-forward -> next block's attention: the block's output, the next
  attention's normalised input (read with the weights the block returned) and
  the next attention's coefficients.

The transcription shares nothing with the oracle: library routines (scipy's
softmax and logistic, NumPy/torch casts) stand in for the pages' torch calls.
Feeding the fused step's hc_pre with the new read weights instead of the
previous sublayer's, or computing the mixes on the old streams, fails here.
"""

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

from oracle import fused_step

NORM_EPS = 1e-6
HC_EPS = 1e-6
ITERS = 20


def _cast(v, dtype):
    """Cast float64 values to the stream dtype and back (torch's conversion)."""
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).to(tdt).double().numpy()


class _Block:
    """Parameters of one block: two ``hc_mixes`` instances and two norms."""

    def __init__(self, rng, n, d):
        nm = (2 + n) * n
        self.fn = {s: rng.normal(0, 0.02, (nm, n * d)) for s in ("attn", "ffn")}
        self.base = {s: rng.normal(0, 0.1, nm) for s in ("attn", "ffn")}
        self.scale = {s: rng.uniform(0.5, 2, 3) for s in ("attn", "ffn")}
        self.gain = {s: 1 + rng.normal(0, 0.05, d) for s in ("attn", "ffn")}
        # the fixed stand-ins for attention and the feed-forward
        self.a = rng.normal(0, 1 / np.sqrt(d), (d, d))
        self.b = rng.normal(0, 1 / np.sqrt(d), (d, d))


def _coefficients(streams, fn, scale, base, n):
    """The block's ``hc_mixes``: per token one RMS over all n*d stream values,
    the projection, then pre / post and the comb schedule (row softmax + eps,
    column division, then alternating row and column divisions)."""
    t = streams.shape[0]
    flat = streams.reshape(t, -1)
    inv = 1 / np.sqrt((flat ** 2).mean(axis=1, keepdims=True) + NORM_EPS)
    mix = flat @ fn.T * inv
    pre = expit(mix[:, :n] * scale[0] + base[:n]) + HC_EPS
    post = 2 * expit(mix[:, n:2 * n] * scale[1] + base[n:2 * n])
    c = softmax((mix[:, 2 * n:] * scale[2] + base[2 * n:]).reshape(t, n, n), axis=2) + HC_EPS
    c = c / (c.sum(axis=1, keepdims=True) + HC_EPS)
    for _ in range(ITERS - 1):
        c = c / (c.sum(axis=2, keepdims=True) + HC_EPS)
        c = c / (c.sum(axis=1, keepdims=True) + HC_EPS)
    return pre, post, c


def _read(streams, weights, dtype):
    """The block's ``hc_pre``: weighted sum over the stream axis, cast back."""
    return _cast((weights[:, :, None] * streams).sum(axis=1), dtype)


def _write(out, residual, post, comb, dtype):
    """The block's ``hc_post``: out broadcast into every stream with post,
    plus residual stream j sent through comb row j, summed over j."""
    spread = post[:, :, None] * out[:, None, :]
    mixed = (comb[:, :, :, None] * residual[:, :, None, :]).sum(axis=1)
    return _cast(spread + mixed, dtype)


def _norm(h, gain, dtype):
    inv = 1 / np.sqrt((h ** 2).mean(axis=1, keepdims=True) + NORM_EPS)
    return _cast(gain * (h * inv), dtype)


def _block(streams, pre_mix, blk, n, dtype):
    """Both halves of one block; returns the block output, the read weights it
    hands on, and every value the boundary checks need."""
    rec = {"x_in": streams}
    residual = streams
    a_pre, a_post, a_comb = _coefficients(streams, blk.fn["attn"], blk.scale["attn"],
                                          blk.base["attn"], n)
    a_in = _norm(_read(streams, pre_mix, dtype), blk.gain["attn"], dtype)
    a_out = _cast(np.tanh(a_in @ blk.a), dtype)
    streams = _write(a_out, residual, a_post, a_comb, dtype)
    rec.update(a_in=a_in, a_out=a_out, a_pre=a_pre, a_post=a_post, a_comb=a_comb,
               x_mid=streams)

    residual = streams
    f_pre, f_post, f_comb = _coefficients(streams, blk.fn["ffn"], blk.scale["ffn"],
                                          blk.base["ffn"], n)
    f_in = _norm(_read(streams, a_pre, dtype), blk.gain["ffn"], dtype)
    f_out = _cast((f_in * expit(f_in)) @ blk.b, dtype)
    streams = _write(f_out, residual, f_post, f_comb, dtype)
    rec.update(f_in=f_in, f_out=f_out, f_pre=f_pre, f_post=f_post, f_comb=f_comb,
               x_out=streams)
    return streams, f_pre, rec


def _check_stream(got, want, dtype):
    # both sides round the same exact value; float64 evaluation order may differ
    # in the last bits, which can move a value by one ulp of the stream dtype
    ulp = {"f32": 2.0 ** -23, "bf16": 2.0 ** -7}[dtype]
    mag = np.maximum(np.abs(want), 2.0 ** -126)
    err = np.abs(got - want) / mag
    assert np.mean(err > 0) < 1e-3, np.mean(err > 0)
    assert np.max(err) <= ulp * 1.0001


@pytest.mark.parametrize("n,d", [(4, 16), (2, 8), (4, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_step_is_the_block_at_both_boundaries(n, d, dtype):
    rng = np.random.default_rng(1000 + 10 * n + d)
    t = 7
    blocks = [_Block(rng, n, d), _Block(rng, n, d)]
    x0 = _cast(rng.standard_normal((t, n, d)), dtype)
    pre_mix0 = rng.uniform(0.2, 1.0, (t, n))
    x1, hand_on, r0 = _block(x0, pre_mix0, blocks[0], n, dtype)
    _, _, r1 = _block(x1, hand_on, blocks[1], n, dtype)

    # attention -> feed-forward of block 0
    b = blocks[0]
    got = fused_step(r0["x_in"], r0["a_out"], r0["a_pre"], r0["a_post"], r0["a_comb"],
                     b.fn["ffn"], b.base["ffn"], b.scale["ffn"], b.gain["ffn"], ITERS,
                     NORM_EPS, HC_EPS, dtype)
    _check_stream(got["xprime"], r0["x_mid"], dtype)
    _check_stream(got["y"], r0["f_in"], dtype)
    np.testing.assert_allclose(got["pre"], r0["f_pre"], rtol=1e-9)
    np.testing.assert_allclose(got["post"], r0["f_post"], rtol=1e-9)
    np.testing.assert_allclose(got["comb"], r0["f_comb"], rtol=1e-9, atol=1e-15)

    # feed-forward of block 0 -> attention of block 1, read with the weights
    # block 0 handed on
    nb = blocks[1]
    got = fused_step(r0["x_mid"], r0["f_out"], r0["f_pre"], r0["f_post"], r0["f_comb"],
                     nb.fn["attn"], nb.base["attn"], nb.scale["attn"], nb.gain["attn"], ITERS,
                     NORM_EPS, HC_EPS, dtype)
    _check_stream(got["xprime"], r0["x_out"], dtype)
    np.testing.assert_array_equal(r1["x_in"], r0["x_out"])
    _check_stream(got["y"], r1["a_in"], dtype)
    np.testing.assert_allclose(got["pre"], r1["a_pre"], rtol=1e-9)
    np.testing.assert_allclose(got["post"], r1["a_post"], rtol=1e-9)
    np.testing.assert_allclose(got["comb"], r1["a_comb"], rtol=1e-9, atol=1e-15)


def test_previous_read_weights_differ_from_new_ones():
    """The check above would not see a swapped read weight if the two weight
    sets happened to agree: make sure they do not on this data."""
    rng = np.random.default_rng(7)
    n, d, t = 4, 16, 7
    blk = _Block(rng, n, d)
    x0 = _cast(rng.standard_normal((t, n, d)), "f32")
    _, _, r = _block(x0, rng.uniform(0.2, 1.0, (t, n)), blk, n, "f32")
    assert np.min(np.abs(r["a_pre"] - r["f_pre"])) > 1e-4
    y_swapped = _norm(_read(r["x_mid"], r["f_pre"], "f32"), blk.gain["ffn"], "f32")
    assert np.max(np.abs(y_swapped - r["f_in"])) > 1e-3

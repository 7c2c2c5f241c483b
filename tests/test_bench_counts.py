"""The training step's algorithmic counts in bench.py, recounted from the weight manifest
(CPU only): every [out, in] matrix costs 2 * rows * out * in flops per product, the step
runs three products per matrix (forward, weight gradient, input gradient) except the input
gradients of action_in (its input is data) and of the time-embedding half of time_in; the
bytes are the bf16 weights read three times, the fp32 gradients written once and the valid
prefix K/V read twice."""
import os
import sys

import numpy as np

import synth

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _recount(L, B, lengths):
    rows = B * synth.CHUNK
    fl = 0
    for name, shape, kind in synth.manifest(L):
        if kind != "w":
            continue
        out_, in_ = shape
        n_products = 3
        if name == "action_in.w":
            n_products = 2
        fl += n_products * 2 * rows * out_ * in_
        if name == "time_in.w":
            fl -= 2 * rows * out_ * (in_ - synth.D_MODEL)  # no input gradient for the e(t) half
    # attention: per row, query head and allowed key, 4 x 64 forward + 8 x 64 backward
    C = synth.CHUNK
    for nb in lengths:
        for l in range(L):
            keys = C * nb + (C * (C + 1) // 2 if synth.is_self_layer(l) else 0)
            fl += 15 * keys * 12 * 64
    n_w = synth.weight_count(L)
    byt = 3 * 2 * n_w + 4 * n_w + 2 * L * sum(lengths) * 5 * 64 * 2 * 2
    return byt, fl


def test_train_counts_match_a_recount_from_the_manifest():
    for L, B, lengths in ((16, 64, [257] * 64), (4, 3, [70, 33, 1]), (2, 1, [0])):
        assert bench.train_algorithmic(L, B, lengths) == _recount(L, B, lengths), (L, B)


def _recount_denoise(L, B, lengths, n_steps):
    """Per call: every manifest tensor the loop reads, once per step at 2 bytes per element,
    except what the weight load folds away (RMSNorm gains into the following matrices;
    action_in and its bias into a [720, 32] matrix and the bias of time_in; the time-embedding
    half of time_in into one time vector per step, which stands in for time_in.b), plus each
    layer's valid prefix K/V; flops 2 per multiply-add per chunk row for every matrix as the
    loop applies it (the folded [720, 32] matrix for action_in and the action half of time_in),
    attention over the unmasked keys."""
    rows = B * synth.CHUNK
    el = fl = 0
    for name, shape, kind in synth.manifest(L):
        if kind == "g" or name.startswith("action_in."):
            continue
        n = int(np.prod(shape))
        if name == "time_in.w":
            out_, _ = shape
            el += out_ * synth.ACTION_DIM      # the folded [720, 32] matrix
            fl += 2 * rows * out_ * synth.ACTION_DIM
            continue
        el += n
        if kind == "w":
            fl += 2 * rows * n
    kv = L * 5 * 64 * 2 * 2 * sum(lengths)
    C = synth.CHUNK
    for nb in lengths:
        for l in range(L):
            keys = C * nb + (C * (C + 1) // 2 if synth.is_self_layer(l) else 0)
            fl += 15 * keys * 4 * 64
    return n_steps * (2 * el + kv), n_steps * fl


def test_denoise_counts_match_a_recount_from_the_manifest():
    for L, B, lengths in ((16, 1, [177]), (16, 64, [257] * 64), (4, 16, list(range(150, 166))), (2, 3, [70, 0, 1])):
        byt, fl = bench.loop_algorithmic(L, B, lengths, 10)
        rb, rf = _recount_denoise(L, B, lengths, 10)
        assert byt == rb and abs(fl - rf) <= 1e-9 * rf, (L, B, byt, rb, fl, rf)
    # per step at batch 1, prefix 177: 194.3 MB of parameters and 3.6 MB of valid K/V
    byt, _ = bench.loop_algorithmic(16, 1, [177], 1)
    assert byt == 2 * 97_149_632 + 16 * 1280 * 177


def test_denoise_counts_with_8bit_weights():
    """8-bit weights: every streamed matrix costs 1 byte per element plus a 4-byte row scale
    instead of 2 bytes per element; K/V, biases, time vectors and flops are unchanged."""
    rows = elems = 0
    for name, shape, kind in synth.manifest(16):
        if kind != "w" or name == "action_in.w":
            continue
        out_, in_ = shape
        if name == "time_in.w":
            in_ = synth.ACTION_DIM  # the folded [720, 32] matrix
        rows += out_
        elems += out_ * in_
    b16, f16 = bench.loop_algorithmic(16, 1, [177], 1)
    b8, f8 = bench.loop_algorithmic(16, 1, [177], 1, w8=True)
    assert f8 == f16
    assert b16 - b8 == elems - 4 * rows


class _FakeLib:
    """The two library calls kernel_table makes, answered on the host: the library's query-group
    split (two groups from 64 queries on, one per 64 from 192 on) and a constant kernel time."""

    def smolexp_batch_groups(self, cfg, B):
        G = B // 64 if B >= 192 else 2 if B >= 64 else 1
        base = ((B + G - 1) // G + 7) // 8 * 8
        return [base] * (G - 1) + [B - (G - 1) * base]

    def smolexp_time_kernel(self, h, kid, reps):
        return 1.0


def test_launch_counts_per_call_match_the_kernel_traces():
    """Launches per call of the 16-layer, 10-step loop as bench.py counts them (the prologue, then
    every timed kernel's launches per call), against the dispatches per call the rocprofv3 traces
    of the library show: batch 1 733 (the step boundary, with both time-MLP layers of the next
    step, one launch from the first step to the last; the cross layers' Q projection inside
    attention), batch 64 1643 (two groups of 32, each
    with its step boundary in one launch; the cross layers' Q projection a launch of its own),
    batch 128 1643 (two groups of 64 at 3200 rows, the boundary still one launch)."""
    import types
    cfg = types.SimpleNamespace(n_steps=10)
    for B, want in ((1, 733), (64, 1643), (128, 1643)):
        kern = bench.kernel_table(_FakeLib(), None, cfg, 16, B, [177] * B, 177, 1)
        assert 1 + sum(v["launches_per_call"] for v in kern.values()) == want, B

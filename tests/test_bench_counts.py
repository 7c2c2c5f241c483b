"""The training step's algorithmic counts in bench.py, recounted from the weight manifest
(CPU only): every [out, in] matrix costs 2 * rows * out * in flops per product, the step
runs three products per matrix (forward, weight gradient, input gradient) except the input
gradients of action_in (its input is data) and of the time-embedding half of time_in; the
bytes are the bf16 weights read three times, the fp32 gradients written once and the valid
prefix K/V read twice."""
import os
import sys

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

"""GPU parity at the library's limits: the largest prefix a handle takes (max_prefix 4096) and
the largest batch (max_batch 1024), against the oracle on sampled queries, at the tolerances
of tests/gpu_util.py.  Two layers (one self, one cross) keep the oracle to seconds; the
kernels and their launch configurations are those of any depth."""
import numpy as np
import pytest

import synth
from gpu_util import Expert, to_device, run_gpu, run_oracle, compare

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def _workload(L, B, P, lengths, seed_shift=0):
    kv = synth.draw_prefix_kv(L, B, P, seed=synth.gen.SEED_KV + seed_shift)
    mask = synth.make_mask(B, P, lengths)
    for b, p in zip(*np.nonzero(mask == 0)):
        kv[:, :, b, :, p, :] = 0x7FC0  # bf16 NaN in every masked slot: pads must never be read as keys
    return {"prefix_kv": kv, "mask": mask, "noise": synth.draw_noise(B), "prev_actions": None}


def test_largest_prefix_4096_both_attention_families():
    """P = 4096 = max_prefix: at batch 9 the register-staged streamed attention (4146 keys in the
    self layers fill its key-kind array exactly), at batch 1 the staged kernels (13 key rounds in the
    self layers, 13 in the cross layers' fused Q-projection kernel), with ragged valid lengths
    (all, most, one token) and NaN pads."""
    L, P = 2, 4096
    ex = Expert(L, max_batch=9, max_prefix=P)
    try:
        lengths = [4096, 3999, 1, 4096, 2048, 4095, 64, 4096, 3000]
        wl = _workload(L, 9, P, lengths)
        _say("P = 4096, batch 9 (streamed attention)")
        gpu = run_gpu(ex, to_device(wl))
        q = [0, 1, 2, 8]
        compare(gpu, run_oracle(ex, wl, q), q, wl["noise"], "P=4096 batch 9")
        _say("P = 4096, batch 1 (staged attention)")
        wl1 = {k: (v[:, :, :1] if k == "prefix_kv" else v[:1]) if v is not None else None for k, v in wl.items()}
        wl1["prefix_kv"] = np.ascontiguousarray(wl1["prefix_kv"])
        gpu1 = run_gpu(ex, to_device(wl1))
        compare(gpu1, run_oracle(ex, wl1, [0]), [0], wl1["noise"], "P=4096 batch 1")
        # the same query gives the same chunk in both launch configurations up to rounding
        assert np.abs(gpu1["out"][0] - gpu["out"][0]).max() < 2e-2
    finally:
        ex.close()


def test_largest_batch_1024():
    """B = 1024 = max_batch at a short ragged prefix: eight concurrent query groups of 128,
    sampled queries at the groups' edges against the oracle."""
    L, B, P = 2, 1024, 16
    ex = Expert(L, max_batch=B, max_prefix=P)
    try:
        lengths = synth.draw_lengths(B, 1, P)
        wl = _workload(L, B, P, lengths, seed_shift=11)
        _say("batch 1024, P = 16 (eight query groups)")
        gpu = run_gpu(ex, to_device(wl))
        q = [0, 127, 128, 511, 896, 1023]
        compare(gpu, run_oracle(ex, wl, q), q, wl["noise"], "batch 1024")
        assert np.isfinite(gpu["out"]).all()
    finally:
        ex.close()


def test_largest_prefix_4096_ring_attention():
    """P = 4096 at batch 25: the streamed attention of direct global->LDS loads through an LDS ring
    (the kernel of 25-32, 49-64 and more than 96 queries per group), ragged lengths from all to
    one valid token, NaN pads."""
    L, P, B = 2, 4096, 25
    ex = Expert(L, max_batch=B, max_prefix=P)
    try:
        lengths = [4096, 1, 3999, 2048, 4095] + [64 * (i + 1) for i in range(B - 5)]
        wl = _workload(L, B, P, lengths, seed_shift=5)
        _say("P = 4096, batch 25 (ring attention)")
        gpu = run_gpu(ex, to_device(wl))
        q = [0, 1, 2, 24]
        compare(gpu, run_oracle(ex, wl, q), q, wl["noise"], "P=4096 batch 25")
    finally:
        ex.close()

"""GPU parity of the 8-bit weight path (config.weight_format = SMOLEXP_WEIGHTS_E4M3): the HIP
kernels reading E4M3 codes with row scales, called through the C ABI, against the oracle's
8-bit model (oracle.quant.streamed_weights: the same matrices quantized by the same rule), at
the tolerances of the fp16 path.  The difference between the 8-bit and the dense model is
printed (the price of the rounded weights), not asserted against a page's figure: the pages
give none."""
import numpy as np
import pytest
import torch

import flow_matching_action_step_amd as fm
import oracle
import synth
from gpu_util import Expert, to_device, run_gpu, run_oracle, compare, VEL_RTOL

pytestmark = pytest.mark.gpu

E4M3 = fm.SMOLEXP_WEIGHTS_E4M3


def _say(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def ex16_w8():
    _say("create 16-layer expert with 8-bit weights (max_batch 8)")
    e = Expert(16, max_batch=8, max_prefix=512, weight_format=E4M3)
    yield e
    e.close()


def test_fp8_denoise_16_layers_batch1(ex16_w8):
    _say("8-bit weights: denoise expert16_b1_p177")
    wl = synth.make_workload("expert16_b1_p177", with_weights=False)
    gpu = run_gpu(ex16_w8, to_device(wl))
    orc = run_oracle(ex16_w8, wl, [0])
    compare(gpu, orc, [0], wl["noise"], "8-bit expert16_b1_p177")
    # the price of the 8-bit weights: the dense float64 model on the same inputs
    dense = oracle.denoise_batch(oracle.decode_weights(ex16_w8.named), ex16_w8.ocfg, wl["prefix_kv"], wl["mask"],
                                 wl["noise"], n_steps=10, record=True, queries=[0])
    rel = [float(np.linalg.norm(orc["vel"][k] - dense[1][k]) / np.linalg.norm(dense[1][k])) for k in range(10)]
    print(f"[fp8] 8-bit against dense model: velocity rel {min(rel):.3e} .. {max(rel):.3e}, "
          f"action max-abs {np.abs(orc['out'] - dense[0]).max():.3e}", flush=True)


def test_fp8_denoise_batch8_overwrite_full_batch(ex16_w8):
    """The largest batch the 8-bit path takes (400 chunk rows: the two-row-block kernels),
    with 7 overwritten rows, sampled queries against the oracle."""
    _say("8-bit weights: denoise expert16_b128_p177_ow7 at batch 8")
    wl = synth.make_workload("expert16_b128_p177_ow7", batch=8, with_weights=False)
    gpu = run_gpu(ex16_w8, to_device(wl), d=7)
    q = [0, 5, 7]
    compare(gpu, run_oracle(ex16_w8, wl, q, d=7), q, wl["noise"], "8-bit b8 overwrite 7", d=7)


def test_fp8_denoise_batch1_overwrite(ex16_w8):
    """Batch 1 with 8-bit weights and 7 overwritten rows: the step-boundary launch with both
    time-MLP layers of the next step reads the 8-bit codes of action_out and of both layers."""
    _say("8-bit weights: denoise at batch 1 with 7 overwritten rows")
    wl = synth.make_workload("expert16_b128_p177_ow7", batch=1, with_weights=False)
    gpu = run_gpu(ex16_w8, to_device(wl), d=7)
    compare(gpu, run_oracle(ex16_w8, wl, [0], d=7), [0], wl["noise"], "8-bit b1 overwrite 7", d=7)


def test_fp8_velocity_ragged_batch3_two_layers():
    """One velocity evaluation through a self and a cross layer, batch 3 with ragged prefixes,
    at t = 1 and an off-schedule t, gains drawn away from 1 (the fold into the quantized rows)."""
    _say("8-bit weights: velocity, 2 layers, batch 3, ragged prefixes")
    ex = Expert(2, max_batch=3, max_prefix=130, gain_seed=synth.gen.SEED_GAINS, weight_format=E4M3)
    try:
        B, P = 3, 130
        kv = synth.draw_prefix_kv(2, B, P)
        mask = synth.make_mask(B, P, [130, 64, 1])
        rng = np.random.default_rng(77)
        x_np = rng.standard_normal((B, 50, 32)).astype(np.float32)
        kv_d = torch.from_numpy(kv.view(np.int16)).cuda()
        mask_d = torch.from_numpy(mask).cuda()
        for t in (1.0, 0.37):
            x = torch.from_numpy(x_np).cuda()
            v = torch.empty_like(x)
            fm.smolexp_velocity(ex.h, ex.cfg, kv_d, mask_d, x, t, v)
            torch.cuda.synchronize()
            got = v.cpu().numpy()
            for b in range(B):
                want = oracle.velocity(ex.W, ex.ocfg, x_np[b].astype(np.float64), np.float32(t),
                                       oracle.bf16_bits_to_float(kv[:, 0, b]), oracle.bf16_bits_to_float(kv[:, 1, b]),
                                       mask[b].astype(bool))
                rel = np.linalg.norm(got[b] - want) / np.linalg.norm(want)
                print(f"[parity] 8-bit velocity t={t} query {b}: rel {rel:.3e}", flush=True)
                assert rel <= VEL_RTOL
    finally:
        ex.close()


def test_fp8_graphs_match_direct_launches_and_repeat_bitwise():
    _say("8-bit weights: graph replay against direct launches, 4 layers, batch 2")
    wl = synth.make_workload("expert4_b1_p177", batch=2, with_weights=False)
    outs = []
    for use_graphs in (1, 0):
        ex = Expert(4, max_batch=2, max_prefix=256, use_graphs=use_graphs, with_oracle=False, weight_format=E4M3)
        try:
            dev = to_device(wl)
            a = run_gpu(ex, dev)["out"]
            b = run_gpu(ex, dev)["out"]
            np.testing.assert_array_equal(a, b)
            outs.append(a)
        finally:
            ex.close()
    np.testing.assert_array_equal(outs[0], outs[1])
    assert np.isfinite(outs[0]).all()


def test_fp8_noalloc_matches_denoise():
    """The entry point that allocates nothing, on a handle with 8-bit weights: bitwise equal to
    smolexp_denoise on the same handle (the same kernels, the workspace in the library's
    fixed array)."""
    import ctypes
    _say("8-bit weights: no-alloc denoise against denoise, 4 layers, batch 5")
    ex = Expert(4, max_batch=8, max_prefix=200, with_oracle=False, weight_format=E4M3)
    try:
        wl = synth.make_workload("expert16_b16_pvar241", batch=5, with_weights=False)
        B, P = 5, 200
        kv = torch.from_numpy(np.ascontiguousarray(synth.draw_prefix_kv(4, B, P)).view(np.int16)).cuda()
        mask = torch.from_numpy(synth.make_mask(B, P, [200, 150, 1, 77, 199])).cuda()
        noise = torch.from_numpy(wl["noise"]).cuda()
        ref = torch.full((B, 50, 32), float("nan"), device="cuda")
        got = torch.full((B, 50, 32), float("nan"), device="cuda")
        fm.smolexp_denoise(ex.h, ex.cfg, kv, mask, noise, ref)
        rc = fm.raw().smolexp_denoise_noalloc(ex.h, ctypes.c_void_p(kv.data_ptr()), ctypes.c_void_p(mask.data_ptr()),
                                              P, ctypes.c_void_p(noise.data_ptr()), ctypes.c_void_p(got.data_ptr()),
                                              B, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, fm.smolexp_last_error(ex.h)
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.isfinite(r).all()
        np.testing.assert_array_equal(g, r)
    finally:
        ex.close()


def test_fp8_key_round_boundaries_three_steps_overwrite():
    """8-bit weights on a 4-layer expert with three Euler steps and 7 overwritten rows, at prefix
    lengths on either side of a staged key round: P = 270 (self layers 320 keys, one whole round)
    and 321 (cross layers 321 keys: the second round holds one key); the second query's valid
    prefix is shorter and every masked slot holds NaN."""
    ex = Expert(4, n_steps=3, max_batch=2, max_prefix=512, weight_format=E4M3)
    try:
        for P, lens in ((270, [270, 135]), (321, [321, 160])):
            _say(f"8-bit weights: P = {P}, 3 Euler steps, d = 7")
            wl = synth.make_workload("expert4_b1_p177", batch=2, with_weights=False)
            wl["prefix_kv"] = synth.draw_prefix_kv(4, 2, P, seed=97 + P)
            wl["prefix_len"] = P
            wl["mask"] = synth.make_mask(2, P, lens)
            wl["lengths"] = wl["mask"].sum(axis=1)
            wl["prev_actions"] = synth.draw_prev_actions(2, 7)
            for b, p in zip(*np.nonzero(wl["mask"] == 0)):
                wl["prefix_kv"][:, :, b, :, p, :] = 0x7FC0   # bf16 NaN in every masked slot
            gpu = run_gpu(ex, to_device(wl), d=7)
            compare(gpu, run_oracle(ex, wl, [0, 1], d=7), [0, 1], wl["noise"], f"8-bit P={P} n=3 d=7", d=7)
    finally:
        ex.close()

"""smolexp_denoise_noalloc (the entry point that allocates nothing: its per-call workspace is a
fixed device array of the library) against smolexp_denoise on the same handle, through the C
ABI: two calls in a row, the second with a smaller batch and prefix, each bitwise equal to the
handle's own path (the same kernels in the same launch configuration), plus its size limit."""
import ctypes

import numpy as np
import pytest
import torch

import flow_matching_action_step_amd as fm
import synth

pytestmark = pytest.mark.gpu


def _inputs(L, B, P, lengths, seed):
    kv = synth.draw_prefix_kv(L, B, P, seed=seed)
    mask = synth.make_mask(B, P, lengths)
    noise = synth.draw_noise(B, seed=seed + 1)
    return (torch.from_numpy(kv.view(np.int16)).cuda(), torch.from_numpy(mask).cuda(),
            torch.from_numpy(noise).cuda())


def test_noalloc_matches_denoise_twice_then_smaller():
    L = 16
    cfg = fm.smolexp_default_config(n_layers=L, max_batch=32, max_prefix=256)
    h = fm.smolexp_create(cfg, 0)
    try:
        fm.smolexp_load_weights(h, synth.pack_weights(synth.draw_weights(L), L))
        lib = fm.raw()
        cases = [
            (16, 241, [int(x) for x in synth.draw_lengths(16, 150, 241)], 21),  # every query, ragged prefixes
            (3, 100, [100, 37, 1], 31),                                           # then a smaller call
        ]
        for B, P, lengths, seed in cases:
            print(f"\n[gpu-test] no-alloc denoise, 16 layers, batch {B}, prefix {P}", flush=True)
            kv, mask, noise = _inputs(L, B, P, lengths, seed)
            ref = torch.full((B, 50, 32), float("nan"), device="cuda")
            got = torch.full((B, 50, 32), float("nan"), device="cuda")
            fm.smolexp_denoise(h, cfg, kv, mask, noise, ref)
            rc = lib.smolexp_denoise_noalloc(h, ctypes.c_void_p(kv.data_ptr()), ctypes.c_void_p(mask.data_ptr()), P,
                                             ctypes.c_void_p(noise.data_ptr()), ctypes.c_void_p(got.data_ptr()), B,
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert rc == 0, fm.smolexp_last_error(h)
            torch.cuda.synchronize()
            r, g = ref.cpu().numpy(), got.cpu().numpy()
            assert np.isfinite(r).all()
            np.testing.assert_array_equal(g, r)
            assert np.abs(r - noise.cpu().numpy()).max() > 0.2  # the expert moved the chunk
        # beyond the array's size: a clear error, nothing enqueued
        kv, mask, noise = _inputs(L, 17, 8, [8] * 17, 41)
        out = torch.zeros((17, 50, 32), device="cuda")
        rc = lib.smolexp_denoise_noalloc(h, ctypes.c_void_p(kv.data_ptr()), ctypes.c_void_p(mask.data_ptr()), 8,
                                         ctypes.c_void_p(noise.data_ptr()), ctypes.c_void_p(out.data_ptr()), 17, None)
        assert rc == fm.SMOLEXP_E_INVAL
        assert "no-alloc" in fm.smolexp_last_error(h)
        torch.cuda.synchronize()
        assert (out == 0).all()
    finally:
        fm.smolexp_destroy(h)

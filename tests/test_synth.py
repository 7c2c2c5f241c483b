"""The seeded input generators: determinism, bf16 encoding, shapes and masks."""
import numpy as np

import synth


def test_bf16_rounding_is_nearest_even_and_exact_on_bf16_values():
    # exact bf16 values pass through unchanged
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000], np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(f), bits)
    # halfway cases round to even; just above halfway rounds up
    one = np.float32(1.0).view(np.uint32)
    cases = np.array([one + 0x8000, one + 0x18000, one + 0x8001, one + 0x7FFF], np.uint32).view(np.float32)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(cases), np.array([0x3F80, 0x3F82, 0x3F81, 0x3F80], np.uint16))


def test_draws_are_deterministic_and_shaped():
    a = synth.draw_weights(2)
    b = synth.draw_weights(2)
    assert list(a) == [n for n, _, _ in synth.manifest(2)]
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    flat = synth.pack_weights(a, 2)
    assert flat.dtype == np.uint16 and flat.size == synth.weight_count(2)
    assert np.all(a["layers.0.norm1.g"] == 0x3F80)          # unit gains
    w = (a["layers.1.gate.w"].astype(np.uint32) << 16).view(np.float32)
    assert abs(w.std() - 0.02) < 5e-4 and abs(w.mean()) < 5e-4
    kv = synth.draw_prefix_kv(2, 3, 9)
    assert kv.shape == (2, 2, 3, 5, 9, 64)
    np.testing.assert_array_equal(kv, synth.draw_prefix_kv(2, 3, 9))
    n = synth.draw_noise(4)
    assert n.shape == (4, 50, 32) and n.dtype == np.float32
    np.testing.assert_array_equal(synth.draw_noise(2), n[:2])     # row-wise stream
    p = synth.draw_prev_actions(3, 7)
    assert p.shape == (3, 7, 32) and abs(p.std() - 0.5) < 0.05


def test_lengths_and_masks():
    L = synth.draw_lengths(16, 150, 241)
    assert L.min() >= 150 and L.max() <= 241
    m = synth.make_mask(16, 241, L)
    np.testing.assert_array_equal(m.sum(1), L)
    for b in range(16):
        assert m[b, :L[b]].all() and not m[b, L[b]:].any()
    wl = synth.make_workload("expert16_b16_pvar241", with_weights=False)
    np.testing.assert_array_equal(wl["mask"].sum(1), wl["lengths"])
    assert wl["prev_actions"] is None
    wl = synth.make_workload("expert16_b128_p177_ow7", batch=2, with_weights=False)
    assert wl["prev_actions"].shape == (2, 7, 32) and wl["mask"].all()

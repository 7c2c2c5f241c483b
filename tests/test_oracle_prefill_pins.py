"""Pins for the oracle's prefix prefill (oracle/prefill.py): each function is
fixed by something other than itself -- a composition of torch library
routines, closed forms, and invariants the method's definition implies.  CPU only.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.prefill import PrefillConfig, prefill, prefill_layer, prefill_batch, prefix_positions, round_to_bf16_bits
import synth


def _rope_complex(x, pos, theta):
    """Rotary embedding as multiplication by a unit complex number (pairs (d, d + D/2))."""
    D = x.shape[-1]
    z = torch.complex(x[..., : D // 2], x[..., D // 2:])
    freqs = theta ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones(len(pos), D // 2, dtype=torch.float64), pos[:, None] * freqs[None, :])
    zr = z * rot
    return torch.cat([zr.real, zr.imag], dim=-1)


def _torch_lm_layer(W, cfg, l, h, pmask):
    """The layer as torch library routines; positions from torch's cumulative sum."""
    p = f"lm.{l}."
    t = {k: torch.from_numpy(v) for k, v in W.items() if k.startswith(p)}
    h = torch.from_numpy(h)
    P = h.shape[0]
    m = torch.from_numpy(pmask.astype(np.int64))
    pos = (torch.cumsum(m, 0) - m).to(torch.float64)
    n1 = F.rms_norm(h, (cfg.d_model,), weight=t[p + "norm1.g"], eps=cfg.rms_eps)
    q = _rope_complex(F.linear(n1, t[p + "q.w"]).view(P, 15, 64).transpose(0, 1), pos, cfg.rope_theta)
    k = _rope_complex(F.linear(n1, t[p + "k.w"]).view(P, 5, 64).transpose(0, 1), pos, cfg.rope_theta)
    v = F.linear(n1, t[p + "v.w"]).view(P, 5, 64).transpose(0, 1)
    mask = torch.from_numpy(pmask)[None, :].expand(P, P)
    o = F.scaled_dot_product_attention(q[None], k[None].contiguous(), v[None].contiguous(),
                                       attn_mask=mask, enable_gqa=True)[0]
    h = h + F.linear(o.transpose(0, 1).reshape(P, 960), t[p + "o.w"])
    n2 = F.rms_norm(h, (cfg.d_model,), weight=t[p + "norm2.g"], eps=cfg.rms_eps)
    h = h + F.linear(F.silu(F.linear(n2, t[p + "gate.w"])) * F.linear(n2, t[p + "up.w"]), t[p + "down.w"])
    return h.numpy(), k.numpy(), v.numpy()


@pytest.fixture(scope="module")
def lm():
    L = 2
    W = oracle.decode_weights(synth.draw_lm_weights(L, gain_seed=synth.gen.SEED_GAINS))
    cfg = PrefillConfig(n_layers=L)
    P = 29
    emb = synth.draw_prefix_embeddings(2, P)
    mask = np.ones((2, P), np.uint8)
    mask[1, [3, 4, 10, 27, 28]] = 0  # interleaved and trailing pads
    return W, cfg, emb, mask


def test_prefix_positions_closed_values():
    m = np.array([1, 0, 1, 1, 0, 0, 1], np.uint8)
    np.testing.assert_array_equal(prefix_positions(m), [0, 1, 1, 2, 3, 3, 3])
    np.testing.assert_array_equal(prefix_positions(np.ones(5, bool)), np.arange(5))


@pytest.mark.parametrize("layer", [0, 1])
@pytest.mark.parametrize("query", [0, 1])
def test_prefill_layer_matches_torch_library_composition(lm, layer, query):
    W, cfg, emb, mask = lm
    h = oracle.bf16_bits_to_float(emb[query]) * (1.0 + 0.5 * layer)
    pm = mask[query].astype(bool)
    got = prefill_layer(W, cfg, layer, h, pm)
    want = _torch_lm_layer(W, cfg, layer, h, pm)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12)


def test_prefill_pad_invariance_with_nan_pads(lm):
    W, cfg, emb, mask = lm
    pm = mask[1].astype(bool)
    e = oracle.bf16_bits_to_float(emb[1])
    k0, v0 = prefill(W, cfg, e, pm)
    e2 = e.copy()
    e2[~pm] = np.nan
    k1, v1 = prefill(W, cfg, e2, pm)
    np.testing.assert_array_equal(k1[:, :, pm], k0[:, :, pm])
    np.testing.assert_array_equal(v1[:, :, pm], v0[:, :, pm])


def test_prefill_pads_do_not_advance_positions(lm):
    """With the pads removed, the valid tokens' keys and values are the same: positions are
    ranks among valid tokens and the keys form a set."""
    W, cfg, emb, mask = lm
    pm = mask[1].astype(bool)
    e = oracle.bf16_bits_to_float(emb[1])
    k0, v0 = prefill(W, cfg, e, pm)
    kc, vc = prefill(W, cfg, e[pm], np.ones(int(pm.sum()), bool))
    np.testing.assert_allclose(k0[:, :, pm], kc, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(v0[:, :, pm], vc, rtol=1e-11, atol=1e-12)


def test_prefill_is_bidirectional_within_the_prefix(lm):
    """The prefix is one block of the block mask: token 0's layer-1 keys depend on the last
    token, while layer 0's keys/values are per-token (no attention before them)."""
    W, cfg, emb, mask = lm
    e = oracle.bf16_bits_to_float(emb[0])
    pm = mask[0].astype(bool)
    k0, v0 = prefill(W, cfg, e, pm)
    e2 = e.copy()
    e2[-1] += 2.0
    k1, v1 = prefill(W, cfg, e2, pm)
    np.testing.assert_array_equal(k1[0, :, :-1], k0[0, :, :-1])
    np.testing.assert_array_equal(v1[0, :, :-1], v0[0, :, :-1])
    assert np.abs(k1[1, :, 0] - k0[1, :, 0]).max() > 1e-6
    assert np.abs(v1[1, :, 0] - v0[1, :, 0]).max() > 1e-6


def test_prefill_single_token_closed_form(lm):
    """One valid token: every query head's attention returns its KV head's V row, so the
    layer is h + concat_h(v[h // 3]) W_o^T followed by the MLP (no softmax)."""
    W, cfg, emb, _ = lm
    e = oracle.bf16_bits_to_float(emb[0, :3])
    pm = np.array([False, True, False])
    h1, k, v = prefill_layer(W, cfg, 0, e, pm)
    p = "lm.0."
    x = e[1:2]
    n1 = oracle.rms_norm(x, W[p + "norm1.g"], cfg.rms_eps)
    vv = (n1 @ W[p + "v.w"].T).reshape(5, 64)
    o = np.concatenate([vv[hq // 3] for hq in range(15)])[None, :]
    hh = x + o @ W[p + "o.w"].T
    n2 = oracle.rms_norm(hh, W[p + "norm2.g"], cfg.rms_eps)
    want = hh + (oracle.silu(n2 @ W[p + "gate.w"].T) * (n2 @ W[p + "up.w"].T)) @ W[p + "down.w"].T
    np.testing.assert_allclose(h1[1:2], want, rtol=1e-12, atol=1e-13)
    # its key sits at position 0: no rotation
    np.testing.assert_allclose(k[:, 1], (n1 @ W[p + "k.w"].T).reshape(5, 64), rtol=1e-13, atol=1e-14)


def test_prefill_batch_layout_and_independence(lm):
    W, cfg, emb, mask = lm
    kv = prefill_batch(W, cfg, emb, mask)
    assert kv.shape == (cfg.n_layers, 2, 2, 5, emb.shape[1], 64)
    for b in range(2):
        k, v = prefill(W, cfg, oracle.bf16_bits_to_float(emb[b]), mask[b].astype(bool))
        np.testing.assert_array_equal(kv[:, 0, b], k)
        np.testing.assert_array_equal(kv[:, 1, b], v)
    np.testing.assert_array_equal(prefill_batch(W, cfg, emb, mask, queries=[1])[:, :, 0], kv[:, :, 1])


def test_round_to_bf16_bits_closed_values():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -2.5, 0.0, 2.0 ** -130])
    got = round_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 0x3F80 and 0x3F81 -> even; 1 + 3 * 2^-9 rounds up; 2^-130 is
    # the subnormal 8 x 2^-133
    np.testing.assert_array_equal(got, np.array([0x3F80, 0x3F80, 0x3F81, 0xC020, 0x0000, 0x0008], np.uint16))
    # exact bf16 values come back unchanged
    y = oracle.bf16_bits_to_float(synth.f32_to_bf16_bits(np.linspace(-3, 3, 17, dtype=np.float32)))
    np.testing.assert_array_equal(oracle.bf16_bits_to_float(round_to_bf16_bits(y)), y)

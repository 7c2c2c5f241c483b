"""Pins for the oracle's 8-bit weights (oracle/quant.py): the E4M3 code points of the OCP
8-bit floating-point format, an exhaustive nearest-value search, torch's float8_e4m3fn cast,
the rounding error bound, the row-scale definition, and the algebra of the streamed weights
(the fp8 model without rounding is the float64 expert).  CPU only."""
import numpy as np
import pytest
import torch

import oracle
from oracle import ExpertConfig
from oracle import quant
import synth


# ---------------------------------------------------------------- the E4M3 format

def test_e4m3_code_points_of_the_format():
    # sign | 4 exponent bits (bias 7) | 3 mantissa bits; no infinities, S.1111.111 = NaN
    d = quant.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0            # largest finite: 1.75 x 2^8
    assert d(0x08) == 2.0 ** -6                              # smallest normal
    assert d(0x07) == 0.875 * 2.0 ** -6                      # largest subnormal
    assert d(0x01) == 2.0 ** -9                              # smallest subnormal
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert d(0x3C) == 1.5 and d(0x39) == 1.125
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert not np.isnan(quant.e4m3_decode(np.arange(256))[[0x77, 0x78, 0x7E]]).any()


def test_e4m3_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    finite = ~np.isnan(quant.e4m3_decode(codes))
    vals = quant.e4m3_decode(codes[finite])
    back = quant.e4m3_encode(vals)
    want = codes[finite].copy()
    want[want == 0x80] = 0x00  # -0 encodes as +0
    np.testing.assert_array_equal(back, want)


def _nearest_by_search(v):
    """Brute force: the finite code whose value is nearest; among two, the even mantissa."""
    codes = np.arange(256, dtype=np.uint8)
    vals = quant.e4m3_decode(codes)
    ok = ~np.isnan(vals) & (codes != 0x80)
    codes, vals = codes[ok], vals[ok]
    out = []
    for x in np.ravel(v):
        dist = np.abs(vals - x)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:
            best = [b for b in best if codes[b] % 2 == 0] or list(best)
        out.append(codes[best[0]])
    return np.array(out, np.uint8).reshape(np.shape(v))


def test_e4m3_encode_is_the_nearest_value_ties_to_even():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.uniform(-448, 448, 300),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 300),                   # subnormals and the first binades
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 300)) * rng.choice([-1, 1], 300),
        # midpoints between neighbouring codes (ties) and just beside them
        [1 + 1 / 16, 1 + 3 / 16, 1 + 5 / 16, 0.5 * 2 ** -9, 1.5 * 2 ** -9, 7.5 * 2 ** -9, 416.0,
         432.0, 15.5 * 2 ** -6 / 8, (1 + 1 / 16) * (1 + 1e-12), (1 + 1 / 16) * (1 - 1e-12)],
    ])
    np.testing.assert_array_equal(quant.e4m3_encode(v), _nearest_by_search(v))


def test_e4m3_encode_matches_torch_float8_cast():
    rng = np.random.default_rng(1)
    v32 = np.concatenate([
        rng.uniform(-448, 448, 20000),
        np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 20000)) * rng.choice([-1, 1], 20000),
        quant.e4m3_decode(np.arange(256))[~np.isnan(quant.e4m3_decode(np.arange(256)))],
    ]).astype(np.float32)  # float32 inputs: torch rounds once, from float32
    t = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = quant.e4m3_encode(v32.astype(np.float64))
    # torch keeps the sign of a value that rounds to zero; the encoder writes +0 for it
    t = np.where((t & 0x7F) == 0, 0, t).astype(np.uint8)
    np.testing.assert_array_equal(got, t)


def test_e4m3_rounding_error_bound():
    rng = np.random.default_rng(2)
    v = np.exp(rng.uniform(np.log(2.0 ** -14), np.log(448.0), 50000)) * rng.choice([-1, 1], 50000)
    err = np.abs(quant.e4m3_decode(quant.e4m3_encode(v)) - v)
    normal = np.abs(v) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(v[normal]))   # half a unit of the 3-bit mantissa
    assert np.all(err[~normal] <= 2.0 ** -10)                       # half the subnormal spacing


def test_e4m3_encode_rejects_out_of_range():
    for bad in (449.0, -1000.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            quant.e4m3_encode(np.array([bad]))


# ---------------------------------------------------------------- rows and scales

def test_row_scales_put_each_row_max_in_the_top_binades():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((64, 100)) * np.exp(rng.uniform(-20, 10, 64))[:, None]
    W[5] = 0.0
    W[6] = 0.0
    W[6, 3] = 448.0 * 2.0 ** -20         # a row whose max is exactly 448 x 2^k
    W[7] = 0.0
    W[7, 0] = -224.0 * 2.0 ** -3         # 224 x 2^k = 448 x 2^(k-1): it maps to -448, not to -224
    s = quant.row_scales(W)
    e = np.log2(s)
    assert np.all(e == np.round(e))
    r = np.max(np.abs(W), axis=1) / s
    nz = np.arange(64) != 5
    assert np.all((r[nz] > 224.0) & (r[nz] <= 448.0))
    assert s[5] == 1.0 and s[6] == 2.0 ** -20 and s[7] == 2.0 ** -4
    codes, s2 = quant.quantize_rows(W)
    np.testing.assert_array_equal(s, s2)
    assert codes[6, 3] == 0x7E and codes[7, 0] == 0xFE    # 448 and -448
    dq = quant.dequantize_rows(codes, s)
    assert np.all(np.abs(dq - W) <= 2.0 ** -4 * np.abs(W) + 2.0 ** -10 * s[:, None])


# ---------------------------------------------------------------- the streamed model

@pytest.fixture(scope="module")
def tiny_model():
    L = 2
    W = oracle.decode_weights(synth.draw_weights(L, gain_seed=synth.gen.SEED_GAINS))
    cfg = ExpertConfig(n_layers=L)
    P = 23
    kv = synth.draw_prefix_kv(L, 2, P)
    mask = synth.make_mask(2, P, [23, 15])
    noise = synth.draw_noise(2)
    return W, cfg, kv, mask, noise


def _velocity(W, cfg, kv, mask, x, t, b):
    pk = oracle.bf16_bits_to_float(kv[:, 0, b])
    pv = oracle.bf16_bits_to_float(kv[:, 1, b])
    return oracle.velocity(W, cfg, x, t, pk, pv, mask[b].astype(bool))


def test_streamed_weights_without_rounding_are_the_float64_expert(tiny_model):
    W, cfg, kv, mask, noise = tiny_model
    W0 = quant.streamed_weights(W, cfg, quantize=False)
    for b, t in ((0, 1.0), (1, 0.37)):
        v = _velocity(W, cfg, kv, mask, noise[b].astype(np.float64), t, b)
        v0 = _velocity(W0, cfg, kv, mask, noise[b].astype(np.float64), t, b)
        np.testing.assert_allclose(v0, v, rtol=1e-11, atol=1e-13)


def _streamed_without_gain_fold(W, cfg, quantize=True):
    out = quant.streamed_weights(W, cfg, quantize)
    for l in range(cfg.n_layers):
        out[f"layers.{l}.gate.w"] = W[f"layers.{l}.gate.w"]  # gain set to 1 but not folded into gate
    return out


def _streamed_time_half_dropped(W, cfg, quantize=True):
    out = quant.streamed_weights(W, cfg, quantize)
    out["time_in.w"] = np.concatenate([np.eye(cfg.d_model), np.zeros((cfg.d_model, cfg.d_model))], axis=1)
    return out


@pytest.mark.parametrize("mutant", [_streamed_without_gain_fold, _streamed_time_half_dropped])
def test_streamed_weight_algebra_catches_planted_mistakes(tiny_model, mutant):
    W, cfg, kv, mask, noise = tiny_model
    W0 = mutant(W, cfg, quantize=False)
    v = _velocity(W, cfg, kv, mask, noise[0].astype(np.float64), 0.6, 0)
    v0 = _velocity(W0, cfg, kv, mask, noise[0].astype(np.float64), 0.6, 0)
    assert np.max(np.abs(v0 - v)) > 1e-6 * np.max(np.abs(v))


def test_streamed_weights_are_on_the_e4m3_grid_of_their_rows(tiny_model):
    W, cfg, _, _, _ = tiny_model
    Q = quant.streamed_weights(W, cfg)
    for name in ("action_in.w", "time_out.w", "layers.0.q.w", "layers.0.v.w", "layers.1.q.w", "layers.1.o.w",
                 "layers.1.up.w", "layers.0.down.w", "action_out.w"):
        A = Q[name]
        s = quant.row_scales(A)
        c = quant.e4m3_encode(A / s[:, None])
        np.testing.assert_array_equal(quant.e4m3_decode(c) * s[:, None], A)  # re-quantizing changes nothing
    np.testing.assert_array_equal(Q["time_in.w"][:, 720:], W["time_in.w"][:, 720:])
    np.testing.assert_array_equal(Q["time_in.w"][:, :720], np.eye(720))

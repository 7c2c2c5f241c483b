"""8-bit weights for the action expert: OCP FP8 E4M3 codes with one power-of-two scale per
output row, and the expert with its streamed matrices replaced by their quantized values.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: PyPI "mlx-smolvla", Run a checkpoint: 8-bit and 4-bit weight presets exist as
explicit opt-ins, dense bf16 stays the default and neither preset is chosen implicitly.  The
pages name no 8-bit format, grouping or rounding; the reading taken here:
  * format: OCP 8-bit floating point, E4M3 variant (sign, 4 exponent bits with bias 7, 3
    mantissa bits; subnormals below 2^-6; largest finite value 448; no infinities, only
    S.1111.111 is NaN);
  * one scale per output row (per output channel) of each matrix, the power of two
    2^ceil(log2(max|row| / 448)), so that w / scale is exact and the row's largest magnitude
    lands in (224, 448];
  * rounding to nearest, ties to even (no saturation is needed: |w / scale| <= 448);
  * what is quantized: every matrix the denoising loop streams, as the loop applies it: the
    RMSNorm gains multiplied into the columns of the matrix that follows the norm (exact:
    products of two bf16 values), and action_in composed with the action half of the time
    MLP's first layer ([720, 32]).  The time-embedding half of that layer only ever meets
    the fixed flow times, so it is not streamed and stays exact, as do the biases.
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6      # 2^-6: smallest normal magnitude
E4M3_MANT_BITS = 3


def e4m3_decode(codes):
    """Values of E4M3 codes (uint8) as float64; the NaN code gives NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    sub = sign * np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def e4m3_encode(v):
    """Nearest E4M3 code (ties to even) of float64 values with |v| <= 448.

    The quantum of a magnitude a is 2^(max(floor(log2 a), -6) - 3); a / quantum is exact
    (a power-of-two division) and is rounded to an integer, ties to even.  An integer of 16
    carries into the next binade, which the code arithmetic below does by itself."""
    v = np.asarray(v, np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values with |v| <= 448")
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = f 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    b = np.maximum(np.where(a > 0, ex - 1, E4M3_MIN_NORMAL_EXP), E4M3_MIN_NORMAL_EXP)
    n = np.rint(np.ldexp(a, E4M3_MANT_BITS - b)).astype(np.int64)   # in [0, 16]
    # code magnitude: subnormal binade (b = -6 and n < 8) is n itself; otherwise the
    # exponent field is b + 7 and the mantissa n - 8, i.e. (b + 7) * 8 + n - 8
    mag = np.where((b == E4M3_MIN_NORMAL_EXP) & (n < 8), n, (b + 7) * 8 + n - 8)
    return (mag | np.where(np.signbit(v) & (mag > 0), 0x80, 0)).astype(np.uint8)


def row_scales(W):
    """Per-row power of two 2^ceil(log2(max|row| / 448)); 1 for an all-zero row."""
    W = np.asarray(W, np.float64)
    amax = np.max(np.abs(W), axis=1)
    s = np.ones_like(amax)
    nz = amax > 0
    e = np.ceil(np.log2(amax[nz] / E4M3_MAX)).astype(np.int64)
    # log2 of an exact quotient can land one off at a power of two: fix it exactly
    e = np.where(np.ldexp(amax[nz], -e) > E4M3_MAX, e + 1, e)
    e = np.where(np.ldexp(amax[nz], -(e - 1)) <= E4M3_MAX, e - 1, e)
    s[nz] = np.ldexp(1.0, e)
    return s


def quantize_rows(W):
    """E4M3 codes [N, K] (uint8) and row scales [N] (float64) of a float64 matrix."""
    W = np.asarray(W, np.float64)
    s = row_scales(W)
    return e4m3_encode(W / s[:, None]), s


def dequantize_rows(codes, scales):
    return e4m3_decode(codes) * np.asarray(scales, np.float64)[:, None]


def _fp8(W):
    c, s = quantize_rows(W)
    return dequantize_rows(c, s)


def streamed_weights(W, cfg, quantize=True):
    """The expert's weights as the fp8 loop applies them, as a dict with the manifest's
    names and shapes, so that expert.velocity computes the fp8 model unchanged:

      action_in.w = Q(W_t1[:, :720] W_in)        [720, 32]
      action_in.b = W_t1[:, :720] b_in
      time_in.w   = [I | W_t1[:, 720:]]          (the identity passes y on; e(t)'s half exact)
      time_in.b   = b_t1
      time_out.w  = Q(W_t2)
      layers: q, k, v, gate, up = Q(W diag(g)) with their norm's gain g, norm gains = 1;
              o, down = Q(W)
      action_out.w = Q(W_out diag(g_final)), final_norm.g = 1
    so that W_t1 [y ; e] + b_t1 with y = x W_in^T + b_in equals the composed form exactly
    in real arithmetic.  quantize=False returns the same algebra without rounding (it must
    give expert.velocity's values to float64 rounding)."""
    q = _fp8 if quantize else (lambda a: np.asarray(a, np.float64))
    D = cfg.d_model
    out = dict(W)
    w_t1 = np.asarray(W["time_in.w"], np.float64)
    w_t1a, w_t1e = w_t1[:, :D], w_t1[:, D:]
    out["action_in.w"] = q(w_t1a @ np.asarray(W["action_in.w"], np.float64))
    out["action_in.b"] = w_t1a @ np.asarray(W["action_in.b"], np.float64)
    out["time_in.w"] = np.concatenate([np.eye(D), w_t1e], axis=1)
    out["time_out.w"] = q(W["time_out.w"])
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        g1 = np.asarray(W[p + "norm1.g"], np.float64)
        g2 = np.asarray(W[p + "norm2.g"], np.float64)
        names = ["q.w", "k.w", "v.w"] if l % 2 == 0 else ["q.w"]
        for n in names:
            out[p + n] = q(np.asarray(W[p + n], np.float64) * g1[None, :])
        out[p + "o.w"] = q(W[p + "o.w"])
        out[p + "gate.w"] = q(np.asarray(W[p + "gate.w"], np.float64) * g2[None, :])
        out[p + "up.w"] = q(np.asarray(W[p + "up.w"], np.float64) * g2[None, :])
        out[p + "down.w"] = q(W[p + "down.w"])
        out[p + "norm1.g"] = np.ones(D)
        out[p + "norm2.g"] = np.ones(D)
    gf = np.asarray(W["final_norm.g"], np.float64)
    out["action_out.w"] = q(np.asarray(W["action_out.w"], np.float64) * gf[None, :])
    out["final_norm.g"] = np.ones(D)
    return out

"""The action expert's velocity field v_theta(x_t, t | prefix), one query, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation follows noeira docs "SmolVLA" (Architecture): x is the 50 x 32
action chunk at flow time t, the prefix is the VLM's per-layer cached K/V,
and the expert is a stack of width-720 layers that alternate self-attention
(even layers) and cross-attention (odd layers).
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ExpertConfig:
    n_layers: int = 16
    d_model: int = 720
    n_q: int = 15
    n_kv: int = 5
    head_dim: int = 64
    ffn: int = 2048
    chunk: int = 50
    action_dim: int = 32
    # Readings where the pages are silent (no trained weights exist here, so
    # any fixed value is equally valid; these are the textbook defaults):
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    t_min_period: float = 4e-3
    t_max_period: float = 4.0


def bf16_bits_to_float(bits):
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_weights(named_bits):
    """Dict of bf16 bit arrays -> dict of float64 arrays (exact)."""
    return {k: bf16_bits_to_float(v) for k, v in named_bits.items()}


def rms_norm(h, g, eps):
    """RMSNorm over the last axis: h / sqrt(mean(h^2) + eps) * g (pre-norm, LLaMA family)."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * g


def silu(z):
    """SiLU(z) = z * sigmoid(z)."""
    return z / (1.0 + np.exp(-z))


def rope(x, pos, theta):
    """Rotary position embedding with the half-split pairing.

    x: [..., n, D]; pos: [n].  Dimension d < D/2 is paired with d + D/2 and
    the pair is rotated by the angle pos * theta^(-2d/D).  (The pages name
    RoPE without fixing the pairing or theta; this is the common form.)
    """
    D = x.shape[-1]
    half = D // 2
    inv_freq = theta ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def time_embedding(t, dim, p_min, p_max):
    """Sinusoidal embedding of the flow time t (a scalar in [0, 1]).

    e = [sin(2 pi t / p_k) for k < dim/2] ++ [cos(2 pi t / p_k) for k < dim/2],
    with periods p_k spaced geometrically from p_min to p_max.  The pages say
    only "sinusoidal"; this is the reading taken.
    """
    half = dim // 2
    frac = np.arange(half) / (half - 1)
    period = p_min * (p_max / p_min) ** frac
    ang = 2.0 * np.pi * float(t) / period
    return np.concatenate([np.sin(ang), np.cos(ang)])


def attention(q, k, v, allowed, scale):
    """Softmax attention of one head with an explicit boolean key mask.

    q [nq, D], k [nk, D], v [nk, D], allowed [nq, nk].  Keys that are not
    allowed are left out of the softmax altogether.  A query row with no
    allowed key returns 0 (empty sum).
    """
    nq = q.shape[0]
    out = np.zeros((nq, v.shape[1]), np.float64)
    if k.shape[0] == 0:
        return out
    s = (q @ k.T) * scale
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    has_key = np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(allowed, np.exp(s - m), 0.0)
    denom = p.sum(axis=1, keepdims=True)
    out[has_key] = (p[has_key] / denom[has_key]) @ v
    return out


def _identity(a):
    return a


def embed(W, cfg, x, t, act_round=_identity):
    """Action and time projections -> the residual stream h0 [chunk, d_model].

    y = x W_in^T + b_in;  h0 = W_t2 SiLU(W_t1 [y ; e(t)] + b_t1) + b_t2.
    The action embedding comes first in the concatenation; biases exist on
    these four projections only.
    """
    y = act_round(x @ W["action_in.w"].T + W["action_in.b"])
    e = time_embedding(t, cfg.d_model, cfg.t_min_period, cfg.t_max_period)
    z = np.concatenate([y, np.broadcast_to(e, (x.shape[0], e.shape[0]))], axis=1)
    s = act_round(silu(z @ W["time_in.w"].T + W["time_in.b"]))
    return s @ W["time_out.w"].T + W["time_out.b"]


def expert_layer(W, cfg, l, h, pk, pv, pmask, act_round=_identity):
    """One pre-norm transformer layer of the expert.

    h [chunk, d_model]; pk, pv [n_kv, P, head_dim] = this layer's cached
    prefix keys (already rotated at prefix positions) and values; pmask [P]
    boolean, True = valid token.  Chunk row i sits at position n_valid + i.
    Self layers (even l) attend to [valid prefix ; chunk rows j <= i]; cross
    layers (odd l) attend to the valid prefix only.  Query head hq reads KV
    head hq // (n_q / n_kv).  Scale 1/sqrt(head_dim).
    """
    p = f"layers.{l}."
    C, H, G, D = h.shape[0], cfg.n_q, cfg.n_kv, cfg.head_dim
    pmask = np.asarray(pmask, bool)
    n_valid = int(pmask.sum())
    pos = n_valid + np.arange(C)

    n1 = act_round(rms_norm(h, W[p + "norm1.g"], cfg.rms_eps))
    q = act_round(rope((n1 @ W[p + "q.w"].T).reshape(C, H, D).transpose(1, 0, 2), pos, cfg.rope_theta))
    kp = pk[:, pmask, :]
    vp = pv[:, pmask, :]
    if l % 2 == 0:
        kc = act_round(rope((n1 @ W[p + "k.w"].T).reshape(C, G, D).transpose(1, 0, 2), pos, cfg.rope_theta))
        vc = act_round((n1 @ W[p + "v.w"].T).reshape(C, G, D).transpose(1, 0, 2))
        keys = np.concatenate([kp, kc], axis=1)
        vals = np.concatenate([vp, vc], axis=1)
        allowed = np.concatenate([np.ones((C, n_valid), bool), np.tril(np.ones((C, C), bool))], axis=1)
    else:
        keys, vals = kp, vp
        allowed = np.ones((C, n_valid), bool)
    group = H // G
    o = np.stack([attention(q[hq], keys[hq // group], vals[hq // group], allowed, 1.0 / np.sqrt(D))
                  for hq in range(H)])
    o = act_round(o.transpose(1, 0, 2).reshape(C, H * D))
    h = h + o @ W[p + "o.w"].T

    n2 = act_round(rms_norm(h, W[p + "norm2.g"], cfg.rms_eps))
    u = act_round(silu(n2 @ W[p + "gate.w"].T) * (n2 @ W[p + "up.w"].T))
    return h + u @ W[p + "down.w"].T


def head(W, cfg, h, act_round=_identity):
    """Final RMSNorm and action_out: v = RMSNorm(h) W_out^T + b_out  [chunk, action_dim]."""
    n = act_round(rms_norm(h, W["final_norm.g"], cfg.rms_eps))
    return n @ W["action_out.w"].T + W["action_out.b"]


def velocity(W, cfg, x, t, pk, pv, pmask, act_round=_identity):
    """v_theta(x, t | prefix) for one query.

    W: float64 weights by manifest name; x [chunk, action_dim]; t scalar;
    pk, pv [n_layers, n_kv, P, head_dim]; pmask [P].
    """
    h = embed(W, cfg, np.asarray(x, np.float64), t, act_round)
    for l in range(cfg.n_layers):
        h = expert_layer(W, cfg, l, h, pk[l], pv[l], pmask, act_round)
    return head(W, cfg, h, act_round)

"""The prefix prefill: the language model's per-layer keys/values over one query's prefix, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

noeira docs "SmolVLA", Architecture: the language model (SmolLM2) has 16
layers of width 960 with grouped-query attention (15 query heads over 5 KV
heads of dim 64), RoPE, SwiGLU and RMSNorm.  A query runs it once over its
prefix (camera images, the tokenised instruction, one state token) and caches
each layer's keys and values; the expert then reads layer l's cache.  The
prefix and the action suffix are joined by a block attention mask, so the
prefix never sees the actions and a prefill alone yields the same prefix
activations as a joint pass.

Readings where the pages are silent (each one a parameter where it can be):
  * the prefix is one block of that mask: every prefix token attends to every
    valid prefix token, before or after it; masked (pad) tokens are left out
    as keys;
  * the token at prefix index j sits at RoPE position = the number of valid
    tokens before it, so pads do not advance positions and the expert's chunk
    row i continues at n_valid + i; the rotation form and theta are the
    expert's (``expert.rope``);
  * the SwiGLU width is 2560 (SmolLM2-360M's layer); the RMSNorm epsilon is the
    expert's; the layer's projections have no biases;
  * the cache holds, for every prefix index (pads included, never attended),
    layer l's keys after the rotation and its values.  Nothing after the last
    layer's keys/values is computed: the expert reads only the cache.
"""
from dataclasses import dataclass

import numpy as np

from .expert import rms_norm, silu, rope, attention, bf16_bits_to_float


@dataclass(frozen=True)
class PrefillConfig:
    n_layers: int = 16
    d_model: int = 960
    n_q: int = 15
    n_kv: int = 5
    head_dim: int = 64
    ffn: int = 2560
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6


def prefix_positions(pmask):
    """RoPE position of every prefix index: how many valid tokens come before it."""
    m = np.asarray(pmask, bool).astype(np.int64)
    return np.cumsum(m) - m


def prefill_layer(W, cfg, l, h, pmask, need_output=True):
    """One pre-norm language-model layer over the prefix rows h [P, d_model].

    Returns (h after the layer or None, K [n_kv, P, head_dim] rotated, V
    [n_kv, P, head_dim]).  With need_output False only K and V are formed.
    """
    p = f"lm.{l}."
    P, H, G, D = h.shape[0], cfg.n_q, cfg.n_kv, cfg.head_dim
    pmask = np.asarray(pmask, bool)
    pos = prefix_positions(pmask)
    n1 = rms_norm(h, W[p + "norm1.g"], cfg.rms_eps)
    k = rope((n1 @ W[p + "k.w"].T).reshape(P, G, D).transpose(1, 0, 2), pos, cfg.rope_theta)
    v = (n1 @ W[p + "v.w"].T).reshape(P, G, D).transpose(1, 0, 2)
    if not need_output:
        return None, k, v
    q = rope((n1 @ W[p + "q.w"].T).reshape(P, H, D).transpose(1, 0, 2), pos, cfg.rope_theta)
    # every row attends to every valid prefix token; pads are not keys at all
    keys, vals = k[:, pmask], v[:, pmask]
    allowed = np.ones((P, keys.shape[1]), bool)
    group = H // G
    o = np.stack([attention(q[hq], keys[hq // group], vals[hq // group], allowed, 1.0 / np.sqrt(D))
                  for hq in range(H)])
    h = h + o.transpose(1, 0, 2).reshape(P, H * D) @ W[p + "o.w"].T
    n2 = rms_norm(h, W[p + "norm2.g"], cfg.rms_eps)
    u = silu(n2 @ W[p + "gate.w"].T) * (n2 @ W[p + "up.w"].T)
    return h + u @ W[p + "down.w"].T, k, v


def prefill(W, cfg, emb, pmask):
    """Keys and values of every layer for one query: K, V [n_layers, n_kv, P, head_dim].

    emb [P, d_model]: the prefix token embeddings (float); pmask [P] boolean.
    """
    h = np.asarray(emb, np.float64)
    ks, vs = [], []
    for l in range(cfg.n_layers):
        h, k, v = prefill_layer(W, cfg, l, h, pmask, need_output=l < cfg.n_layers - 1)
        ks.append(k)
        vs.append(v)
    return np.stack(ks), np.stack(vs)


def prefill_batch(W, cfg, emb_bits, mask, queries=None):
    """Float64 cache [n_layers, 2 (K, V), len(queries), n_kv, P, head_dim] of the listed queries.

    emb_bits: bf16 bit patterns [B, P, d_model]; mask [B, P].
    """
    qs = range(emb_bits.shape[0]) if queries is None else queries
    out = []
    for b in qs:
        k, v = prefill(W, cfg, bf16_bits_to_float(emb_bits[b]), np.asarray(mask[b], bool))
        out.append(np.stack([k, v]))  # [2, L, G, P, D]
    return np.stack(out).transpose(2, 1, 0, 3, 4, 5)


def round_to_bf16_bits(x):
    """The cache is stored in bf16 (CSDN "SmolVLA PyTorch official-like 精度排查过程与结论",
    sections 8 and 12): float64 values rounded to float32, as a float32 accumulator holds
    them, then to the nearest bf16 (ties to even).  Bit patterns; finite inputs.
    """
    u = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32)).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)

"""Seeded generators for every input of the action-expert denoiser.

Randomness uses numpy's PCG64 (``np.random.default_rng``).  One seed per
kind of tensor, so that changing one input never shifts another:

    weights        seed 0   N(0, 0.02) for matrices and biases, drawn in
                            manifest order; RMSNorm gains are 1 (not drawn)
    noise          seed 1   N(0, 1) fp32, [B, 50, 32]  (x at t = 1)
    prefix K/V     seed 2   N(0, 1) rounded to bf16, [L, 2, B, 5, P, 64],
                            pad positions are drawn too (they must never matter)
    lengths        seed 3   valid prefix length per query, U{lo..hi}
    prev. actions  seed 4   N(0, 0.5) fp32 (std 0.5), [B, d, 32]
    gain variant   seed 5   RMSNorm gains 1 + N(0, 0.1), only when asked for
    LM weights     seed 6   the prefix language model's weights, as the
                            expert's (N(0, 0.02), gains 1), in its manifest order
    embeddings     seed 7   prefix token embeddings N(0, 1) rounded to bf16,
                            [B, P, 960] (what the vision connector and the text
                            embedding table would produce)
    actions        seed 8   training targets: action chunks N(0, 1) fp32,
                            [B, 50, 32] (normalised actions)
    flow times     seed 9   training flow times, one per query, U(0, 1) fp32

Floating-point draws are made in float32 and rounded to bf16 with
round-to-nearest-even where the tensor is stored as bf16.  Everything is
returned as plain numpy arrays; bf16 tensors are uint16 bit patterns.

Architecture constants are those of SmolVLA's action expert (noeira docs
"SmolVLA", Architecture table: 16 layers, width 720, even layers
self-attend, odd layers cross-attend; the language model's grouped-query
layout of 15 query heads over 5 KV heads of dim 64 is shared by the
expert's attention).
"""
import numpy as np

D_MODEL = 720       # expert width
N_Q = 15            # query heads
N_KV = 5            # key/value heads
HEAD_DIM = 64
FFN = 2048          # SwiGLU intermediate width
CHUNK = 50          # actions per chunk
ACTION_DIM = 32     # padded action vector width
TIME_DIM = 720      # sinusoidal time-embedding width

SEED_WEIGHTS, SEED_NOISE, SEED_KV, SEED_LENGTHS, SEED_PREV, SEED_GAINS = 0, 1, 2, 3, 4, 5
SEED_LM_WEIGHTS, SEED_EMB = 6, 7
SEED_ACTIONS, SEED_TIMES = 8, 9

# The language model that fills the prefix cache (noeira docs "SmolVLA",
# Architecture table: SmolLM2, 16 layers of width 960, the same grouped-query
# layout).  Its SwiGLU width is not on the pages; 2560 is SmolLM2-360M's.
LM_D_MODEL = 960
LM_FFN = 2560

# The five synthetic workloads.  `prefix_len` is the padded prefix length P;
# `lengths` is None (all P tokens valid) or the (lo, hi) range of valid
# lengths; `overwrite_rows` is d for prefix overwrite (0 = off).
WORKLOADS = {
    "expert4_b1_p177": dict(n_layers=4, batch=1, prefix_len=177, lengths=None, overwrite_rows=0),
    "expert16_b1_p177": dict(n_layers=16, batch=1, prefix_len=177, lengths=None, overwrite_rows=0),
    "expert16_b16_pvar241": dict(n_layers=16, batch=16, prefix_len=241, lengths=(150, 241), overwrite_rows=0),
    "expert16_b64_p257": dict(n_layers=16, batch=64, prefix_len=257, lengths=None, overwrite_rows=0),
    "expert16_b128_p177_ow7": dict(n_layers=16, batch=128, prefix_len=177, lengths=None, overwrite_rows=7),
}


def is_self_layer(layer):
    """Even layers (0-based) self-attend, odd layers cross-attend."""
    return layer % 2 == 0


def manifest(n_layers):
    """Ordered (name, shape, kind) list of every expert tensor.

    kind is "w" (matrix, [out, in]), "b" (bias) or "g" (RMSNorm gain).
    Self-attention layers own q/k/v/o projections; cross-attention layers
    attend to the cached prefix K/V as-is and own only q and o.
    """
    m = [
        ("action_in.w", (D_MODEL, ACTION_DIM), "w"),
        ("action_in.b", (D_MODEL,), "b"),
        ("time_in.w", (D_MODEL, D_MODEL + TIME_DIM), "w"),
        ("time_in.b", (D_MODEL,), "b"),
        ("time_out.w", (D_MODEL, D_MODEL), "w"),
        ("time_out.b", (D_MODEL,), "b"),
    ]
    for l in range(n_layers):
        p = f"layers.{l}."
        m.append((p + "norm1.g", (D_MODEL,), "g"))
        m.append((p + "q.w", (N_Q * HEAD_DIM, D_MODEL), "w"))
        if is_self_layer(l):
            m.append((p + "k.w", (N_KV * HEAD_DIM, D_MODEL), "w"))
            m.append((p + "v.w", (N_KV * HEAD_DIM, D_MODEL), "w"))
        m.append((p + "o.w", (D_MODEL, N_Q * HEAD_DIM), "w"))
        m.append((p + "norm2.g", (D_MODEL,), "g"))
        m.append((p + "gate.w", (FFN, D_MODEL), "w"))
        m.append((p + "up.w", (FFN, D_MODEL), "w"))
        m.append((p + "down.w", (D_MODEL, FFN), "w"))
    m += [
        ("final_norm.g", (D_MODEL,), "g"),
        ("action_out.w", (ACTION_DIM, D_MODEL), "w"),
        ("action_out.b", (ACTION_DIM,), "b"),
    ]
    return m


def weight_count(n_layers):
    return int(sum(int(np.prod(s)) for _, s, _ in manifest(n_layers)))


def f32_to_bf16_bits(a):
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    Inputs are finite random draws, so NaN handling is not needed here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def lm_manifest(n_layers):
    """Ordered (name, shape, kind) list of the prefix language model's tensors.

    Every layer is a pre-norm GQA block (q, k, v, o, then a SwiGLU MLP); no
    biases.  Only the layers whose keys/values the expert reads are listed.
    """
    m = []
    for l in range(n_layers):
        p = f"lm.{l}."
        m += [
            (p + "norm1.g", (LM_D_MODEL,), "g"),
            (p + "q.w", (N_Q * HEAD_DIM, LM_D_MODEL), "w"),
            (p + "k.w", (N_KV * HEAD_DIM, LM_D_MODEL), "w"),
            (p + "v.w", (N_KV * HEAD_DIM, LM_D_MODEL), "w"),
            (p + "o.w", (LM_D_MODEL, N_Q * HEAD_DIM), "w"),
            (p + "norm2.g", (LM_D_MODEL,), "g"),
            (p + "gate.w", (LM_FFN, LM_D_MODEL), "w"),
            (p + "up.w", (LM_FFN, LM_D_MODEL), "w"),
            (p + "down.w", (LM_D_MODEL, LM_FFN), "w"),
        ]
    return m


def lm_weight_count(n_layers):
    return int(sum(int(np.prod(s)) for _, s, _ in lm_manifest(n_layers)))


def draw_weights(n_layers, seed=SEED_WEIGHTS, gain_seed=None, std=0.02, which=None):
    """Named bf16 weights (uint16 bit patterns), drawn in manifest order.

    With gain_seed set, RMSNorm gains become 1 + N(0, 0.1) from that seed
    (a variant that makes a kernel ignoring the gain fail); otherwise 1.
    which: the manifest function (the expert's by default).
    """
    rng = np.random.default_rng(seed)
    grng = np.random.default_rng(gain_seed) if gain_seed is not None else None
    out = {}
    for name, shape, kind in (which or manifest)(n_layers):
        if kind == "g":
            if grng is None:
                vals = np.ones(shape, np.float32)
            else:
                vals = (1.0 + 0.1 * grng.standard_normal(shape, dtype=np.float32)).astype(np.float32)
        else:
            vals = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        out[name] = f32_to_bf16_bits(vals)
    return out


def draw_lm_weights(n_layers, seed=SEED_LM_WEIGHTS, gain_seed=None, std=0.02):
    """Named bf16 weights of the prefix language model, drawn in its manifest order."""
    return draw_weights(n_layers, seed=seed, gain_seed=gain_seed, std=std, which=lm_manifest)


def pack_weights(named, n_layers, which=None):
    """Concatenate named bf16 tensors into one flat uint16 buffer in manifest order."""
    parts = []
    for name, shape, _ in (which or manifest)(n_layers):
        a = named[name]
        if tuple(a.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {a.shape} != manifest {shape}")
        parts.append(a.reshape(-1))
    return np.concatenate(parts)


def pack_lm_weights(named, n_layers):
    return pack_weights(named, n_layers, which=lm_manifest)


def draw_prefix_embeddings(batch, prefix_len, seed=SEED_EMB):
    """Prefix token embeddings, bf16 N(0, 1), [B][P][960]; pad positions are drawn too."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((batch, prefix_len, LM_D_MODEL), dtype=np.float32))


def draw_prefix_kv(n_layers, batch, prefix_len, seed=SEED_KV):
    """Per-layer prefix K/V cache, bf16 N(0, 1), layout [L][2 (K, V)][B][5][P][64]."""
    rng = np.random.default_rng(seed)
    out = np.empty((n_layers, 2, batch, N_KV, prefix_len, HEAD_DIM), np.uint16)
    for l in range(n_layers):          # drawn slice by slice to bound host memory
        for kv in range(2):
            out[l, kv] = f32_to_bf16_bits(
                rng.standard_normal((batch, N_KV, prefix_len, HEAD_DIM), dtype=np.float32))
    return out


def draw_lengths(batch, lo, hi, seed=SEED_LENGTHS):
    """Valid prefix length per query, uniform on the integers lo..hi inclusive."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=batch).astype(np.int64)


def make_mask(batch, prefix_len, lengths=None):
    """uint8 [B, P] pad mask, 1 = valid; right-padded to P."""
    m = np.zeros((batch, prefix_len), np.uint8)
    if lengths is None:
        m[:] = 1
    else:
        for b, n in enumerate(lengths):
            m[b, :int(n)] = 1
    return m


def draw_noise(batch, seed=SEED_NOISE):
    """Gaussian noise N(0, 1), fp32 [B, 50, 32]: the flow's state at t = 1."""
    return np.random.default_rng(seed).standard_normal((batch, CHUNK, ACTION_DIM), dtype=np.float32)


def draw_prev_actions(batch, rows, seed=SEED_PREV):
    """Tail of the previous chunk for prefix overwrite, N(0, 0.5) fp32 [B, d, 32]."""
    rng = np.random.default_rng(seed)
    return (np.float32(0.5) * rng.standard_normal((batch, rows, ACTION_DIM), dtype=np.float32)).astype(np.float32)


def draw_actions(batch, seed=SEED_ACTIONS):
    """Training action chunks a, N(0, 1) float32 [B, 50, 32]."""
    return np.random.default_rng(seed).standard_normal((batch, CHUNK, ACTION_DIM), dtype=np.float32)


def draw_flow_times(batch, seed=SEED_TIMES):
    """Training flow times, one per query, uniform on [0, 1) float32 [B]."""
    return np.random.default_rng(seed).random(batch, dtype=np.float32)


def make_workload(name, batch=None, with_weights=True, gain_seed=None):
    """Every input of one named workload as a dict of numpy arrays.

    batch overrides the workload's batch (draws for the first queries are
    unchanged only for noise/prev-actions/lengths, whose streams are drawn
    row by row; K/V slices depend on the batch size).
    """
    w = dict(WORKLOADS[name])
    if batch is not None:
        w["batch"] = batch
    L, B, P, d = w["n_layers"], w["batch"], w["prefix_len"], w["overwrite_rows"]
    lengths = None
    if w["lengths"] is not None:
        lengths = draw_lengths(B, *w["lengths"])
    out = dict(name=name, n_layers=L, batch=B, prefix_len=P, overwrite_rows=d)
    if with_weights:
        out["weights"] = draw_weights(L, gain_seed=gain_seed)
    out["prefix_kv"] = draw_prefix_kv(L, B, P)
    out["lengths"] = lengths if lengths is not None else np.full(B, P, np.int64)
    out["mask"] = make_mask(B, P, lengths)
    out["noise"] = draw_noise(B)
    out["prev_actions"] = draw_prev_actions(B, d) if d > 0 else None
    return out

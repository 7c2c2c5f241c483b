"""Pins for the CPU oracle: each function is fixed by something other than itself.

Closed forms, brute force on tiny shapes, textbook/library special cases and
invariants that the method's definition implies.  CPU only.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import ExpertConfig
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "architecture.txt")


def _golden():
    out = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0] if line.lstrip().startswith("#") else line
            if "=" not in line:
                continue
            key, rest = line.split("=", 1)
            out[key.strip()] = rest.split("|", 1)[0].strip()
    return out


# ---------------------------------------------------------------- golden facts

def test_golden_architecture_matches_oracle_and_manifest():
    g = _golden()
    cfg = ExpertConfig()
    assert cfg.n_layers == int(g["expert_layers"])
    assert cfg.d_model == int(g["expert_width"])
    assert cfg.n_q == int(g["query_heads"]) and cfg.n_kv == int(g["kv_heads"])
    assert cfg.head_dim == int(g["head_dim"])
    assert cfg.chunk == int(g["chunk"]) and cfg.action_dim == int(g["action_width"])
    assert g["self_attention_layers"] == "even"
    names = [n for n, _, _ in synth.manifest(16)]
    for l in range(16):
        assert (f"layers.{l}.k.w" in names) == (l % 2 == 0)
    ts, dt = oracle.schedule(int(g["euler_steps"]))
    assert len(ts) == 10 and float(ts[0]) == float(g["t_start"])
    assert abs(float(ts[-1]) + float(dt) - float(g["t_end"])) < 1e-6
    assert synth.WORKLOADS["expert16_b128_p177_ow7"]["overwrite_rows"] == int(g["overwrite_rows"])


def test_weight_count_matches_manifest_totals():
    # Independent count from the architecture: per self layer q,k,v,o + 3 FFN + 2 gains.
    w, f, a = 720, 2048, 32
    self_l = 2 * w + 960 * w + 2 * 320 * w + w * 960 + 3 * f * w
    cross_l = self_l - 2 * 320 * w
    io = (w * a + w) + (w * 1440 + w) + (w * w + w) + w + (a * w + a)
    assert synth.weight_count(16) == io + 8 * (self_l + cross_l) == 98_210_912
    assert synth.weight_count(4) == io + 2 * (self_l + cross_l) == 25_755_872


# ---------------------------------------------------------------- elementwise ops

def test_rms_norm_closed_form_and_library():
    eps = 1e-6
    g = np.linspace(0.5, 1.5, 720)
    for c in (3.0, -0.25, 1e-3):
        h = np.full((2, 720), c)
        want = g * np.sign(c) / np.sqrt(1.0 + eps / (c * c))
        np.testing.assert_allclose(oracle.rms_norm(h, g, eps), np.broadcast_to(want, (2, 720)), rtol=1e-13)
    rng = np.random.default_rng(11)
    h = rng.standard_normal((7, 720))
    ref = F.rms_norm(torch.from_numpy(h), (720,), weight=torch.from_numpy(g), eps=eps).numpy()
    np.testing.assert_allclose(oracle.rms_norm(h, g, eps), ref, rtol=1e-12, atol=1e-14)


def test_silu_values_and_library():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([1.0])), [1.0 / (1.0 + np.exp(-1.0))], rtol=1e-15)
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)


def test_rope_closed_forms():
    theta, D = 10000.0, 64
    x = np.random.default_rng(3).standard_normal((2, 5, D))
    # position 0 is the identity
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(5), theta), x)
    # unit vector in dim d rotates into the plane (d, d + D/2) by pos * theta^(-2d/D)
    for d in (0, 5, 31):
        e = np.zeros((1, D))
        e[0, d] = 1.0
        p = 17.0
        ang = p * theta ** (-2.0 * d / D)
        r = oracle.rope(e, np.array([p]), theta)[0]
        want = np.zeros(D)
        want[d], want[d + D // 2] = np.cos(ang), np.sin(ang)
        np.testing.assert_allclose(r, want, atol=1e-15)
    # norms are preserved
    pos = np.arange(5) * 13.0 + 2
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(x, pos, theta), axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-13)
    # q.k depends only on the position difference
    q, k = x[0, 0:1], x[1, 0:1]
    for shift in (0.0, 5.0, 123.0):
        a = oracle.rope(q, np.array([40.0 + shift]), theta) @ oracle.rope(k, np.array([7.0 + shift]), theta).T
        b = oracle.rope(q, np.array([33.0]), theta) @ oracle.rope(k, np.array([0.0]), theta).T
        np.testing.assert_allclose(a, b, rtol=1e-11)


def test_time_embedding_closed_forms():
    cfg = ExpertConfig()
    e0 = oracle.time_embedding(0.0, 720, cfg.t_min_period, cfg.t_max_period)
    np.testing.assert_array_equal(e0, np.concatenate([np.zeros(360), np.ones(360)]))
    e = oracle.time_embedding(0.37, 720, cfg.t_min_period, cfg.t_max_period)
    np.testing.assert_allclose(e[:360] ** 2 + e[360:] ** 2, 1.0, rtol=1e-14)
    # at a quarter of the largest period the last sine is exactly at its peak;
    # at a quarter of the smallest period the first sine is at its peak
    e = oracle.time_embedding(cfg.t_max_period / 4, 720, cfg.t_min_period, cfg.t_max_period)
    assert abs(e[359] - 1.0) < 1e-15 and abs(e[719]) < 1e-15
    e = oracle.time_embedding(cfg.t_min_period / 4, 720, cfg.t_min_period, cfg.t_max_period)
    assert abs(e[0] - 1.0) < 1e-15


# ---------------------------------------------------------------- attention

def _brute_attention(q, k, v, allowed, scale):
    nq, D = q.shape
    out = np.zeros((nq, v.shape[1]))
    for i in range(nq):
        num = np.zeros(v.shape[1])
        den = 0.0
        mx = max([sum(q[i, d] * k[j, d] for d in range(D)) * scale
                  for j in range(k.shape[0]) if allowed[i, j]], default=None)
        if mx is None:
            continue
        for j in range(k.shape[0]):
            if not allowed[i, j]:
                continue
            s = sum(q[i, d] * k[j, d] for d in range(D)) * scale
            w = np.exp(s - mx)
            den += w
            num += w * v[j]
        out[i] = num / den
    return out


@pytest.mark.parametrize("seed", range(6))
def test_attention_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    P, C, D = int(rng.integers(1, 10)), int(rng.integers(1, 6)), 8
    pmask = rng.random(P) < 0.6
    q = rng.standard_normal((C, D)) * 2.0
    kp, vp = rng.standard_normal((P, D)), rng.standard_normal((P, D))
    kc, vc = rng.standard_normal((C, D)), rng.standard_normal((C, D))
    for is_self in (True, False):
        if is_self:
            k = np.concatenate([kp[pmask], kc])
            v = np.concatenate([vp[pmask], vc])
            allowed = np.concatenate([np.ones((C, pmask.sum()), bool), np.tril(np.ones((C, C), bool))], 1)
        else:
            k, v, allowed = kp[pmask], vp[pmask], np.ones((C, pmask.sum()), bool)
        got = oracle.attention(q, k, v, allowed, 1 / np.sqrt(D))
        want = _brute_attention(q, k, v, allowed, 1 / np.sqrt(D))
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_attention_single_key_returns_v_and_equal_keys_average():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 16)) * 30.0
    k = rng.standard_normal((6, 16))
    v = rng.standard_normal((6, 16))
    allowed = np.zeros((4, 6), bool)
    allowed[np.arange(4), [2, 0, 5, 3]] = True
    np.testing.assert_array_equal(oracle.attention(q, k, v, allowed, 0.125), v[[2, 0, 5, 3]])
    kk = np.broadcast_to(k[0], (6, 16))
    allowed = rng.random((4, 6)) < 0.5
    allowed[:, 0] = True
    got = oracle.attention(q, kk, v, allowed, 0.125)
    want = np.stack([v[allowed[i]].mean(0) for i in range(4)])
    np.testing.assert_allclose(got, want, rtol=1e-12)
    # no allowed key -> zero output
    assert not oracle.attention(q, k, v, np.zeros((4, 6), bool), 0.125).any()
    assert not oracle.attention(q, k[:0], v[:0], np.zeros((4, 0), bool), 0.125).any()


def test_attention_matches_library_sdpa_with_gqa_and_block_mask():
    rng = np.random.default_rng(9)
    H, G, C, P, D = 15, 5, 50, 23, 64
    q = rng.standard_normal((H, C, D))
    k = rng.standard_normal((G, P + C, D))
    v = rng.standard_normal((G, P + C, D))
    allowed = np.concatenate([np.ones((C, P), bool), np.tril(np.ones((C, C), bool))], 1)
    got = np.stack([oracle.attention(q[h], k[h // 3], v[h // 3], allowed, 0.125) for h in range(H)])
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(allowed), scale=0.125, enable_gqa=True)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_block_mask_joint_pass_equals_prefill_plus_chunk():
    """The prefix never sees the chunk: a joint pass over [prefix ; chunk]
    with the block mask gives the prefix rows of a prefix-only pass, and the
    chunk rows of the cached-prefix formulation (noeira docs, Architecture)."""
    rng = np.random.default_rng(21)
    P, C, D = 11, 6, 16
    qp, kp, vp = (rng.standard_normal((P, D)) for _ in range(3))
    qc, kc, vc = (rng.standard_normal((C, D)) for _ in range(3))
    q = np.concatenate([qp, qc])
    k = np.concatenate([kp, kc])
    v = np.concatenate([vp, vc])
    allowed = np.zeros((P + C, P + C), bool)
    allowed[:P, :P] = True                      # prefix block
    allowed[P:, :P] = True                      # chunk sees the prefix
    allowed[P:, P:] = np.tril(np.ones((C, C), bool))  # causal chunk
    joint = oracle.attention(q, k, v, allowed, 0.25)
    prefix_only = oracle.attention(qp, kp, vp, np.ones((P, P), bool), 0.25)
    np.testing.assert_allclose(joint[:P], prefix_only, rtol=1e-13, atol=1e-15)
    # changing the chunk leaves the prefix rows bit-identical
    k2, v2 = k.copy(), v.copy()
    k2[P:] += 5.0
    v2[P:] -= 3.0
    np.testing.assert_array_equal(oracle.attention(q, k2, v2, allowed, 0.25)[:P], joint[:P])
    cached = oracle.attention(qc, k, v, allowed[P:], 0.25)
    np.testing.assert_allclose(joint[P:], cached, rtol=1e-14)


# ---------------------------------------------------------------- expert layer vs torch library composition

def _rope_complex(x, pos, theta):
    """Rotary embedding written as multiplication by a unit complex number
    (pairs (d, d + D/2) as real and imaginary parts)."""
    D = x.shape[-1]
    z = torch.complex(x[..., : D // 2], x[..., D // 2:])
    freqs = theta ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones(len(pos), D // 2, dtype=torch.float64), pos[:, None] * freqs[None, :])
    zr = z * rot
    return torch.cat([zr.real, zr.imag], dim=-1)


def _torch_layer(W, cfg, l, h, pk, pv, pmask):
    t = {k: torch.from_numpy(v) for k, v in W.items() if k.startswith(f"layers.{l}.")}
    p = f"layers.{l}."
    h = torch.from_numpy(h)
    C = h.shape[0]
    nv = int(pmask.sum())
    pos = torch.arange(C, dtype=torch.float64) + nv
    n1 = F.rms_norm(h, (cfg.d_model,), weight=t[p + "norm1.g"], eps=cfg.rms_eps)
    q = _rope_complex(F.linear(n1, t[p + "q.w"]).view(C, 15, 64).transpose(0, 1), pos, cfg.rope_theta)
    kp = torch.from_numpy(pk[:, pmask])
    vp = torch.from_numpy(pv[:, pmask])
    if l % 2 == 0:
        kc = _rope_complex(F.linear(n1, t[p + "k.w"]).view(C, 5, 64).transpose(0, 1), pos, cfg.rope_theta)
        vc = F.linear(n1, t[p + "v.w"]).view(C, 5, 64).transpose(0, 1)
        k, v = torch.cat([kp, kc], 1), torch.cat([vp, vc], 1)
        mask = torch.cat([torch.ones(C, nv, dtype=torch.bool), torch.ones(C, C, dtype=torch.bool).tril()], 1)
    else:
        k, v = kp, vp
        mask = torch.ones(C, nv, dtype=torch.bool)
    o = F.scaled_dot_product_attention(q[None], k[None].contiguous(), v[None].contiguous(),
                                       attn_mask=mask, enable_gqa=True)[0]
    h = h + F.linear(o.transpose(0, 1).reshape(C, 960), t[p + "o.w"])
    n2 = F.rms_norm(h, (cfg.d_model,), weight=t[p + "norm2.g"], eps=cfg.rms_eps)
    h = h + F.linear(F.silu(F.linear(n2, t[p + "gate.w"])) * F.linear(n2, t[p + "up.w"]), t[p + "down.w"])
    return h.numpy()


@pytest.fixture(scope="module")
def small_model():
    L = 2
    W = oracle.decode_weights(synth.draw_weights(L, gain_seed=synth.gen.SEED_GAINS))
    cfg = ExpertConfig(n_layers=L)
    P = 31
    kv = synth.draw_prefix_kv(L, 3, P)
    mask = synth.make_mask(3, P, [31, 20, 26])
    noise = synth.draw_noise(3)
    return W, cfg, kv, mask, noise


@pytest.mark.parametrize("layer", [0, 1])
def test_expert_layer_matches_torch_library_composition(small_model, layer):
    W, cfg, kv, mask, _ = small_model
    rng = np.random.default_rng(layer)
    h = rng.standard_normal((50, 720)) * 0.3
    b = 1
    pk = oracle.bf16_bits_to_float(kv[layer, 0, b])
    pv = oracle.bf16_bits_to_float(kv[layer, 1, b])
    pm = mask[b].astype(bool)
    got = oracle.expert_layer(W, cfg, layer, h, pk, pv, pm)
    want = _torch_layer(W, cfg, layer, h, pk, pv, pm)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- whole expert invariants

def _query(kv, mask, b):
    return (oracle.bf16_bits_to_float(kv[:, 0, b]), oracle.bf16_bits_to_float(kv[:, 1, b]),
            mask[b].astype(bool))


def test_expert_chunk_causality(small_model):
    W, cfg, kv, mask, noise = small_model
    pk, pv, pm = _query(kv, mask, 1)
    x = noise[1].astype(np.float64)
    v0 = oracle.velocity(W, cfg, x, 0.7, pk, pv, pm)
    for j in (0, 17, 49):
        x2 = x.copy()
        x2[j] += 1.5
        v1 = oracle.velocity(W, cfg, x2, 0.7, pk, pv, pm)
        np.testing.assert_array_equal(v1[:j], v0[:j])
        assert np.abs(v1[j:] - v0[j:]).max() > 1e-6


def test_expert_pad_invariance_with_nan_pads(small_model):
    W, cfg, kv, mask, noise = small_model
    b = 1
    pk, pv, pm = _query(kv, mask, b)
    x = noise[b].astype(np.float64)
    v0 = oracle.velocity(W, cfg, x, 0.4, pk, pv, pm)
    pk2, pv2 = pk.copy(), pv.copy()
    pk2[:, :, ~pm] = np.nan
    pv2[:, :, ~pm] = np.nan
    np.testing.assert_array_equal(oracle.velocity(W, cfg, x, 0.4, pk2, pv2, pm), v0)
    # moving the pads elsewhere (interleaved) changes nothing: positions come
    # from the number of valid tokens, and keys are a set
    perm = np.random.default_rng(0).permutation(pm.shape[0])
    v_perm = oracle.velocity(W, cfg, x, 0.4, pk[:, :, perm], pv[:, :, perm], pm[perm])
    np.testing.assert_allclose(v_perm, v0, rtol=1e-12, atol=1e-13)


def test_oracle_float32_rounding_gap_is_far_below_the_tolerance(small_model):
    """Every activation of the velocity field rounded to float32 (as a float32 evaluation
    would hold it) moves the float64 result by orders of magnitude less than the 1e-2
    velocity tolerance: the oracle's own rounding does not use up the parity budget."""
    W, cfg, kv, mask, noise = small_model
    pk, pv, pm = _query(kv, mask, 2)
    x = noise[2].astype(np.float64)
    v64 = oracle.velocity(W, cfg, x, 0.55, pk, pv, pm)
    v32 = oracle.velocity(W, cfg, x, 0.55, pk, pv, pm, act_round=lambda a: a.astype(np.float32).astype(np.float64))
    rel = np.linalg.norm(v32 - v64) / np.linalg.norm(v64)
    assert 0.0 < rel < 1e-5, rel


def test_expert_batch_invariance(small_model):
    W, cfg, kv, mask, noise = small_model
    xb = oracle.denoise_batch(W, cfg, kv, mask, noise, n_steps=2)
    for b in range(3):
        xa = oracle.denoise_batch(W, cfg, kv, mask, noise, n_steps=2, queries=[b])
        np.testing.assert_array_equal(xa[0], xb[b])


def test_whole_loop_closed_form_with_zero_action_out(small_model):
    """W_out = 0 makes v = b_out at every step, so x_n = eps + n * dt * b_out."""
    W, cfg, kv, mask, noise = small_model
    W2 = dict(W)
    W2["action_out.w"] = np.zeros_like(W["action_out.w"])
    x, vs, xs = oracle.denoise_batch(W2, cfg, kv, mask, noise, n_steps=10, record=True, queries=[0])
    ts, dt = oracle.schedule(10)
    want = noise[0].astype(np.float64) + 10 * float(dt) * W["action_out.b"]
    np.testing.assert_allclose(x[0], want, rtol=1e-13, atol=1e-14)
    assert vs.shape == (10, 1, 50, 32) and xs.shape == (10, 1, 50, 32)
    np.testing.assert_array_equal(xs[-1], x)       # the final chunk is the last Euler state


def test_whole_loop_closed_form_with_identity_layers(small_model):
    """Zero o/down projections make every layer the identity; with time_out = 0
    the stream is b_t2 everywhere, so v is the constant RMSNorm(b_t2) W_out^T + b_out.
    With b_t2 = beta * 1 and unit gains that constant is sign(beta)/sqrt(1 + eps/beta^2) * rowsum(W_out) + b_out."""
    W, cfg, kv, mask, noise = small_model
    W2 = dict(W)
    for l in range(cfg.n_layers):
        W2[f"layers.{l}.o.w"] = np.zeros_like(W[f"layers.{l}.o.w"])
        W2[f"layers.{l}.down.w"] = np.zeros_like(W[f"layers.{l}.down.w"])
    W2["time_out.w"] = np.zeros_like(W["time_out.w"])
    beta = -0.3
    W2["time_out.b"] = np.full(720, beta)
    W2["final_norm.g"] = np.ones(720)
    c = np.sign(beta) / np.sqrt(1 + cfg.rms_eps / beta ** 2) * W["action_out.w"].sum(1) + W["action_out.b"]
    x = oracle.denoise_batch(W2, cfg, kv, mask, noise, n_steps=10, queries=[2])
    ts, dt = oracle.schedule(10)
    np.testing.assert_allclose(x[0], noise[2] + 10 * float(dt) * c, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- schedule and Euler

def test_schedule():
    for n in (1, 4, 10):
        ts, dt = oracle.schedule(n)
        assert len(ts) == n and ts[0] == np.float32(1.0) and dt == np.float32(-1.0 / n)
        assert all(isinstance(t, np.float32) for t in ts)
        np.testing.assert_allclose([float(t) for t in ts], 1.0 - np.arange(n) / n, atol=1e-6)
        assert all(a > b for a, b in zip(ts, ts[1:]))


def test_euler_constant_and_linear_fields():
    rng = np.random.default_rng(1)
    eps = rng.standard_normal((50, 32))
    c = rng.standard_normal((50, 32))
    ts, dt = oracle.schedule(10)
    x = oracle.euler_denoise(lambda x, t: c, eps, 10)
    np.testing.assert_allclose(x, eps + 10 * float(dt) * c, rtol=1e-14, atol=1e-14)
    lam = 2.5
    x = oracle.euler_denoise(lambda x, t: lam * x, eps, 10)
    np.testing.assert_allclose(x, (1 + float(dt) * lam) ** 10 * eps, rtol=1e-13)


def test_euler_straight_path_reaches_target():
    """For one target a, the flow-matching velocity along x_t = t*eps + (1-t)*a
    is eps - a = (x - a)/t; Euler stays on the path and lands on a at t = 0."""
    rng = np.random.default_rng(2)
    eps = rng.standard_normal((50, 32))
    a = rng.standard_normal((50, 32))
    x, vs, xs = oracle.euler_denoise(lambda x, t: (x - a) / float(t), eps, 10, record=True)
    ts, dt = oracle.schedule(10)
    for k in range(10):
        tk1 = float(ts[k]) + float(dt)
        np.testing.assert_allclose(xs[k], tk1 * eps + (1 - tk1) * a, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(vs[k], eps - a, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(x, a, atol=1e-6)


def test_overwrite_closed_form_and_fixed_point():
    rng = np.random.default_rng(4)
    eps = rng.standard_normal((50, 32))
    prev = rng.standard_normal((7, 32)) * 0.5
    ts, dt = oracle.schedule(10)
    x = oracle.euler_denoise(lambda x, t: np.zeros_like(x), eps, 10, prev=prev, d=7)
    t9 = float(ts[-1])
    np.testing.assert_allclose(x[:7], t9 * eps[:7] + (1 - t9) * prev, rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(x[7:], eps[7:])
    # on the straight path toward a (with a = prev on the first rows) the overwrite is a fixed point
    a = rng.standard_normal((50, 32))
    a[:7] = prev
    field = lambda x, t: (x - a) / float(t)  # noqa: E731
    x_ow = oracle.euler_denoise(field, eps, 10, prev=prev, d=7)
    x_plain = oracle.euler_denoise(field, eps, 10)
    np.testing.assert_allclose(x_ow, x_plain, atol=1e-6)
    np.testing.assert_allclose(x_ow, a, atol=1e-6)


# ---------------------------------------------------------------- action and time embedding (embed)
#
# What fixes embed (noeira docs "SmolVLA", Architecture, action-head row): action_in
# 32 -> 720, the sinusoidal time embedding
# concatenated after the action embedding, a 1440 -> 720 projection with SiLU, then
# 720 -> 720.  Degenerate weights reduce embed to closed forms that depend on each of
# those choices: which half of time_in reads the time embedding, where the SiLU sits,
# and every one of the three biases it adds before the layers.

def _silu_closed(z):
    return z / (1.0 + np.exp(-z))


def _embed_weights(rng, time_path):
    """Weights for embed's closed forms.  time_path: time_in = [0 | I] (only the time
    embedding reaches the hidden layer), time_out = c I, random b_t1 and b_t2.  Otherwise:
    action_in a per-row-scaled selector of the 32 action dims with a random bias,
    time_in = [I | 0], time_out = c I, no b_t1 / b_t2 (c = 1.75 in both: a SiLU placed
    after time_out would see c z instead of z)."""
    D, A = 720, 32
    W = {}
    if time_path:
        W["action_in.w"] = np.zeros((D, A))
        W["action_in.b"] = np.zeros(D)
        W["time_in.w"] = np.concatenate([np.zeros((D, D)), np.eye(D)], axis=1)
        W["time_in.b"] = rng.standard_normal(D) * 0.5
        W["time_out.w"] = 1.75 * np.eye(D)
        W["time_out.b"] = rng.standard_normal(D) * 0.5
    else:
        sel = np.zeros((D, A))
        scale = 0.5 + np.arange(D) / D
        sel[np.arange(D), np.arange(D) % A] = scale
        W["action_in.w"] = sel
        W["action_in.b"] = rng.standard_normal(D) * 0.5
        W["time_in.w"] = np.concatenate([np.eye(D), np.zeros((D, D))], axis=1)
        W["time_in.b"] = np.zeros(D)
        W["time_out.w"] = 1.75 * np.eye(D)
        W["time_out.b"] = np.zeros(D)
    return W


def _embed_closed_form(W, cfg, x, t, time_path):
    if time_path:
        e = oracle.time_embedding(t, cfg.d_model, cfg.t_min_period, cfg.t_max_period)
        row = 1.75 * _silu_closed(e + W["time_in.b"]) + W["time_out.b"]
        return np.broadcast_to(row, (x.shape[0], cfg.d_model))
    D = cfg.d_model
    cols = np.arange(D) % 32
    scale = 0.5 + np.arange(D) / D
    return 1.75 * _silu_closed(x[:, cols] * scale + W["action_in.b"])


def _embed_pin_failures(embed_fn):
    """Names of the closed forms that embed_fn violates (empty: all hold)."""
    cfg = ExpertConfig(n_layers=1)
    rng = np.random.default_rng(71)
    x = rng.standard_normal((50, 32))
    bad = []
    for time_path in (True, False):
        W = _embed_weights(rng, time_path)
        for t in (1.0, 0.37, 0.1):
            got = embed_fn(W, cfg, x, t)
            want = _embed_closed_form(W, cfg, x, t, time_path)
            if not np.allclose(got, want, rtol=1e-12, atol=1e-13):
                bad.append(("time" if time_path else "action", t))
    return bad


# Plausible mistakes in embed, each planted in a copy of it on the CPU.
def _embed_swapped_concat(W, cfg, x, t, act_round=None):
    y = x @ W["action_in.w"].T + W["action_in.b"]
    e = oracle.time_embedding(t, cfg.d_model, cfg.t_min_period, cfg.t_max_period)
    z = np.concatenate([np.broadcast_to(e, (x.shape[0], e.shape[0])), y], axis=1)
    return oracle.silu(z @ W["time_in.w"].T + W["time_in.b"]) @ W["time_out.w"].T + W["time_out.b"]


def _embed_silu_after_time_out(W, cfg, x, t, act_round=None):
    y = x @ W["action_in.w"].T + W["action_in.b"]
    e = oracle.time_embedding(t, cfg.d_model, cfg.t_min_period, cfg.t_max_period)
    z = np.concatenate([y, np.broadcast_to(e, (x.shape[0], e.shape[0]))], axis=1)
    return oracle.silu((z @ W["time_in.w"].T + W["time_in.b"]) @ W["time_out.w"].T + W["time_out.b"])


def _embed_no_action_bias(W, cfg, x, t, act_round=None):
    y = x @ W["action_in.w"].T
    e = oracle.time_embedding(t, cfg.d_model, cfg.t_min_period, cfg.t_max_period)
    z = np.concatenate([y, np.broadcast_to(e, (x.shape[0], e.shape[0]))], axis=1)
    return oracle.silu(z @ W["time_in.w"].T + W["time_in.b"]) @ W["time_out.w"].T + W["time_out.b"]


def _embed_no_hidden_bias(W, cfg, x, t, act_round=None):
    y = x @ W["action_in.w"].T + W["action_in.b"]
    e = oracle.time_embedding(t, cfg.d_model, cfg.t_min_period, cfg.t_max_period)
    z = np.concatenate([y, np.broadcast_to(e, (x.shape[0], e.shape[0]))], axis=1)
    return oracle.silu(z @ W["time_in.w"].T) @ W["time_out.w"].T + W["time_out.b"]


_EMBED_MUTANTS = [_embed_swapped_concat, _embed_silu_after_time_out, _embed_no_action_bias, _embed_no_hidden_bias]


def test_embed_closed_forms():
    """The time path alone gives h0 = 1.75 SiLU(e(t) + b_t1) + b_t2 on every row; the
    action path alone gives h0[:, i] = 1.75 SiLU(s_i x[:, i mod 32] + b_in[i])."""
    assert _embed_pin_failures(oracle.embed) == []


@pytest.mark.parametrize("mutant", _EMBED_MUTANTS, ids=lambda f: f.__name__)
def test_embed_closed_forms_catch_planted_mistakes(mutant):
    assert _embed_pin_failures(mutant) != []


def _velocity_through_identity_layers(W_embed, x, t):
    """v from oracle.velocity with every layer made the identity (zero o and down
    projections) and unit final-norm gains, on a 2-layer expert."""
    cfg = ExpertConfig(n_layers=2)
    W = oracle.decode_weights(synth.draw_weights(2))
    W.update(W_embed)
    for l in range(2):
        W[f"layers.{l}.o.w"] = np.zeros_like(W[f"layers.{l}.o.w"])
        W[f"layers.{l}.down.w"] = np.zeros_like(W[f"layers.{l}.down.w"])
    W["final_norm.g"] = np.ones(720)
    P = 9
    kv = synth.draw_prefix_kv(2, 1, P)
    pk, pv, pm = _query(kv, synth.make_mask(1, P, [6]), 0)
    return oracle.velocity(W, cfg, x, t, pk, pv, pm), W, cfg


def test_velocity_closed_form_through_embed_and_head(monkeypatch):
    """The action-path embedding pushed through identity layers and the head:
    v = h0 / sqrt(mean(h0^2) + eps) W_out^T + b_out with h0 in closed form.  The same
    check fails when any planted mistake replaces embed inside the velocity field."""
    rng = np.random.default_rng(72)
    x = rng.standard_normal((50, 32))
    W_embed = _embed_weights(rng, time_path=False)

    def closed(W, cfg, t):
        h0 = _embed_closed_form(W, cfg, x, t, time_path=False)
        n = h0 / np.sqrt(np.mean(h0 * h0, axis=1, keepdims=True) + cfg.rms_eps)
        return n @ W["action_out.w"].T + W["action_out.b"]

    v, W, cfg = _velocity_through_identity_layers(W_embed, x, 0.37)
    np.testing.assert_allclose(v, closed(W, cfg, 0.37), rtol=1e-11, atol=1e-13)
    for mutant in _EMBED_MUTANTS[:3]:  # the action path has no b_t1 to drop
        monkeypatch.setattr(oracle.expert, "embed", mutant)
        v, W, cfg = _velocity_through_identity_layers(W_embed, x, 0.37)
        assert not np.allclose(v, closed(W, cfg, 0.37), rtol=1e-6, atol=1e-8), mutant.__name__

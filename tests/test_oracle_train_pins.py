"""Pins for the oracle's training step (oracle/train.py): every derivative is fixed
by something other than itself -- central finite differences of the float64 loss
(the definition of the derivative), torch autograd through an independent
composition of torch library routines, and closed forms.  CPU only.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.expert import ExpertConfig
from oracle.train import (silu_grad, rms_norm_bwd, rope_bwd, attention_bwd, query_loss_and_grads,
                          train_batch)
import synth


def _fd(f, x, dx, h=1e-5):
    return (f(x + h * dx) - f(x - h * dx)) / (2 * h)


# ---------------------------------------------------------------- per-op derivatives vs finite differences

def test_silu_grad_finite_differences_and_closed_values():
    z = np.linspace(-8, 8, 41)
    fd = (oracle.silu(z + 1e-6) - oracle.silu(z - 1e-6)) / 2e-6
    np.testing.assert_allclose(silu_grad(z), fd, rtol=1e-8, atol=1e-10)
    assert silu_grad(np.array([0.0]))[0] == 0.5


def test_rms_norm_bwd_finite_differences():
    rng = np.random.default_rng(11)
    h, g, dy = rng.standard_normal((5, 24)), 1 + 0.3 * rng.standard_normal(24), rng.standard_normal((5, 24))
    dh, dg = rms_norm_bwd(dy, h, g, 1e-6)
    for _ in range(3):
        d = rng.standard_normal(h.shape)
        want = _fd(lambda x: np.sum(dy * oracle.rms_norm(x, g, 1e-6)), h, d)
        assert abs(np.sum(dh * d) - want) <= 1e-8 * abs(want) + 1e-10
        d = rng.standard_normal(g.shape)
        want = _fd(lambda x: np.sum(dy * oracle.rms_norm(h, x, 1e-6)), g, d)
        assert abs(np.sum(dg * d) - want) <= 1e-8 * abs(want) + 1e-10


def test_rope_bwd_is_the_transpose():
    rng = np.random.default_rng(12)
    x, dy = rng.standard_normal((3, 7, 64)), rng.standard_normal((3, 7, 64))
    pos = np.arange(7) + 40
    # <dy, R x> = <R^T dy, x> for every x: the backward is the transpose (and R^T R = I)
    np.testing.assert_allclose(np.sum(dy * oracle.rope(x, pos, 1e4)), np.sum(rope_bwd(dy, pos, 1e4) * x), rtol=1e-12)
    np.testing.assert_allclose(rope_bwd(oracle.rope(x, pos, 1e4), pos, 1e4), x, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_bwd_finite_differences(seed):
    rng = np.random.default_rng(100 + seed)
    nq, nk, D = 5, 9, 8
    q, k, v = (rng.standard_normal((n, D)) * 1.5 for n in (nq, nk, nk))
    allowed = rng.random((nq, nk)) < 0.6
    allowed[0] = False  # a row with no key: no output, no gradient
    allowed[1, :] = False
    allowed[1, 3] = True  # one key: output is that V row
    do = rng.standard_normal((nq, D))
    dq, dk, dv = attention_bwd(q, k, v, allowed, 0.35, do)
    f = lambda q_, k_, v_: np.sum(do * oracle.attention(q_, k_, v_, allowed, 0.35))
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        for _ in range(3):
            d = rng.standard_normal(grad.shape)
            args = [q, k, v]
            want = _fd(lambda x: f(*[x if i == which else a for i, a in enumerate(args)]), args[which], d)
            assert abs(np.sum(grad * d) - want) <= 1e-8 * abs(want) + 1e-10
    assert not dq[0].any() and not dq[1].any()  # no key, and a single key (softmax constant)


# ---------------------------------------------------------------- the whole step

@pytest.fixture(scope="module")
def model():
    L, B, P = 2, 2, 23
    W = oracle.decode_weights(synth.draw_weights(L, gain_seed=synth.gen.SEED_GAINS))
    cfg = ExpertConfig(n_layers=L)
    kv = synth.draw_prefix_kv(L, B, P)
    mask = synth.make_mask(B, P, [23, 14])
    mask[0, [2, 9]] = 0  # interleaved pads too
    a = synth.draw_actions(B).astype(np.float64)
    eps = synth.draw_noise(B).astype(np.float64)
    t = np.array([0.83, 0.27])
    return W, cfg, kv, mask, a, eps, t


def test_forward_velocity_is_the_expert_velocity(model):
    W, cfg, kv, mask, a, eps, t = model
    pk, pv = oracle.bf16_bits_to_float(kv[:, 0, 1]), oracle.bf16_bits_to_float(kv[:, 1, 1])
    pm = mask[1].astype(bool)
    _, _, v = query_loss_and_grads(W, cfg, a[1], eps[1], t[1], pk, pv, pm, 3200)
    x = t[1] * eps[1] + (1 - t[1]) * a[1]
    np.testing.assert_allclose(v, oracle.velocity(W, cfg, x, t[1], pk, pv, pm), rtol=1e-13, atol=1e-14)


def test_every_gradient_tensor_by_finite_differences(model):
    """Directional derivative of the batch loss along a random direction in each tensor."""
    W, cfg, kv, mask, a, eps, t = model
    loss, grads = train_batch(W, cfg, kv, mask, a, eps, t)
    names = [n for n, _, _ in synth.manifest(cfg.n_layers)]
    assert sorted(grads) == sorted(names)
    rng = np.random.default_rng(7)
    for n in names:
        d = rng.standard_normal(W[n].shape)
        d /= np.linalg.norm(d)

        def f(x):
            W2 = dict(W)
            W2[n] = x
            return train_batch(W2, cfg, kv, mask, a, eps, t)[0]

        want = _fd(f, W[n], d, h=1e-4)
        got = float(np.sum(grads[n] * d))
        assert abs(got - want) <= 1e-6 * np.linalg.norm(grads[n]) + 1e-12, (n, got, want)


def _torch_loss(W, cfg, kv, mask, a, eps, t):
    """The batch loss as torch library routines (float64), for autograd."""
    tw = {k: torch.tensor(v, requires_grad=True) for k, v in W.items()}
    B, C = a.shape[0], a.shape[1]
    total = 0.0
    for b in range(B):
        pm = torch.from_numpy(mask[b].astype(bool))
        nv = int(pm.sum())
        x = torch.from_numpy(t[b] * eps[b] + (1 - t[b]) * a[b])
        target = torch.from_numpy(eps[b] - a[b])
        y = F.linear(x, tw["action_in.w"], tw["action_in.b"])
        k = torch.arange(360, dtype=torch.float64)
        period = cfg.t_min_period * (cfg.t_max_period / cfg.t_min_period) ** (k / 359)
        ang = 2 * torch.pi * t[b] / period
        e = torch.cat([torch.sin(ang), torch.cos(ang)]).expand(C, 720)
        h = F.linear(F.silu(F.linear(torch.cat([y, e], 1), tw["time_in.w"], tw["time_in.b"])),
                     tw["time_out.w"], tw["time_out.b"])
        pos = torch.arange(C, dtype=torch.float64) + nv
        freqs = cfg.rope_theta ** (-torch.arange(0, 64, 2, dtype=torch.float64) / 64)
        rot = torch.polar(torch.ones(C, 32, dtype=torch.float64), pos[:, None] * freqs[None, :])

        def rope(z):
            zc = torch.complex(z[..., :32], z[..., 32:]) * rot
            return torch.cat([zc.real, zc.imag], -1)

        for l in range(cfg.n_layers):
            p = f"layers.{l}."
            n1 = F.rms_norm(h, (720,), weight=tw[p + "norm1.g"], eps=cfg.rms_eps)
            q = rope(F.linear(n1, tw[p + "q.w"]).view(C, 15, 64).transpose(0, 1))
            kp = torch.from_numpy(oracle.bf16_bits_to_float(kv[l, 0, b]))[:, pm]
            vp = torch.from_numpy(oracle.bf16_bits_to_float(kv[l, 1, b]))[:, pm]
            if l % 2 == 0:
                kc = rope(F.linear(n1, tw[p + "k.w"]).view(C, 5, 64).transpose(0, 1))
                vc = F.linear(n1, tw[p + "v.w"]).view(C, 5, 64).transpose(0, 1)
                keys, vals = torch.cat([kp, kc], 1), torch.cat([vp, vc], 1)
                am = torch.cat([torch.ones(C, nv, dtype=torch.bool), torch.ones(C, C, dtype=torch.bool).tril()], 1)
            else:
                keys, vals, am = kp, vp, torch.ones(C, nv, dtype=torch.bool)
            o = F.scaled_dot_product_attention(q[None], keys[None].contiguous(), vals[None].contiguous(),
                                               attn_mask=am, enable_gqa=True)[0]
            h = h + F.linear(o.transpose(0, 1).reshape(C, 960), tw[p + "o.w"])
            n2 = F.rms_norm(h, (720,), weight=tw[p + "norm2.g"], eps=cfg.rms_eps)
            h = h + F.linear(F.silu(F.linear(n2, tw[p + "gate.w"])) * F.linear(n2, tw[p + "up.w"]), tw[p + "down.w"])
        v = F.linear(F.rms_norm(h, (720,), weight=tw["final_norm.g"], eps=cfg.rms_eps),
                     tw["action_out.w"], tw["action_out.b"])
        total = total + F.mse_loss(v, target, reduction="sum")
    loss = total / (B * C * a.shape[2])
    loss.backward()
    return float(loss.detach()), {k: v.grad.numpy() for k, v in tw.items()}


def test_loss_and_gradients_match_torch_autograd(model):
    W, cfg, kv, mask, a, eps, t = model
    loss, grads = train_batch(W, cfg, kv, mask, a, eps, t)
    tl, tg = _torch_loss(W, cfg, kv, mask, a, eps, t)
    assert abs(loss - tl) <= 1e-12 * tl
    for n, g in grads.items():
        np.testing.assert_allclose(g, tg[n], rtol=1e-9, atol=1e-9 * np.abs(tg[n]).max(), err_msg=n)


def test_closed_form_with_zero_action_out(model):
    """W_out = 0: v = b_out on every row, so the loss is the mean of (b_out - (eps - a))^2,
    column j of d loss / d b_out is 2 / n times the sum of (b_out - target) over that column,
    and nothing upstream of action_out receives a gradient."""
    W, cfg, kv, mask, a, eps, t = model
    W2 = dict(W)
    W2["action_out.w"] = np.zeros_like(W["action_out.w"])
    loss, grads = train_batch(W2, cfg, kv, mask, a, eps, t)
    err = W["action_out.b"][None, None, :] - (eps - a)
    n = err.size
    assert abs(loss - np.sum(err ** 2) / n) <= 1e-13 * loss
    np.testing.assert_allclose(grads["action_out.b"], 2 * err.sum(axis=(0, 1)) / n, rtol=1e-12, atol=1e-15)
    for name, g in grads.items():
        if name not in ("action_out.w", "action_out.b"):
            assert not g.any(), name


def test_batch_share_and_query_subsets_add_up(model):
    W, cfg, kv, mask, a, eps, t = model
    loss, grads = train_batch(W, cfg, kv, mask, a, eps, t)
    l0, g0 = train_batch(W, cfg, kv, mask, a, eps, t, queries=[0])
    l1, g1 = train_batch(W, cfg, kv, mask, a, eps, t, queries=[1])
    assert loss == l0 + l1
    for n in grads:
        np.testing.assert_array_equal(grads[n], g0[n] + g1[n])

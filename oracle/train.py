"""Flow-matching training step of the action expert: the loss and its weight gradients, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

noeira docs "SmolVLA", Architecture (the flow-matching objective used to fine-tune):
a training sample mixes the action chunk a with Gaussian noise at flow time t,
x_t = t * eps + (1 - t) * a, and the expert's velocity at (x_t, t) is regressed
onto the straight path's velocity eps - a with a squared error.  noeira docs
"SmolVLA", Fine-tuning: only the expert trains (its layers and the action and
time projections); the vision tower and the language model are frozen, so the
prefix keys/values are inputs without gradients.

Readings where the pages are silent:
  * the loss of a batch is the mean of the squared error over its
    B x 50 x 32 elements (the pages write a squared norm; the held-out losses
    they report, 0.22-0.55, are per-element means, not sums over 1,600-element
    chunks);
  * t (one value per query) and eps are drawn by the caller and are inputs
    here, as is every random number of the method;
  * the step produces the loss and the gradient of every expert tensor in the
    weight manifest; the optimizer update is not part of it.

The backward pass is the chain rule through the forward of ``expert.py``, written
per operation; each backward function states the derivative it implements.
"""
import numpy as np

from .expert import rms_norm, silu, rope, time_embedding, attention, bf16_bits_to_float


# ---------------------------------------------------------------------------- per-op derivatives

def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu_grad(z):
    """d/dz [z sigmoid(z)] = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def linear_bwd(dy, x, w):
    """y = x w^T (+ b): dx = dy w, dw = dy^T x, db = sum over rows of dy."""
    return dy @ w, dy.T @ x, dy.sum(axis=0)


def rms_norm_bwd(dy, h, g, eps):
    """y = g * h * r with r = (mean(h^2) + eps)^(-1/2), over the last axis.

    With u = dy * g and hat = h * r:  dh = r * (u - hat * mean(u * hat)),
    dg = sum over rows of dy * hat.
    """
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    hat = h * r
    u = dy * g
    dh = r * (u - hat * np.mean(u * hat, axis=-1, keepdims=True))
    return dh, (dy * hat).sum(axis=0)


def rope_bwd(dy, pos, theta):
    """The rotation is orthogonal: its transpose is the rotation by the negated angles."""
    return rope(dy, -np.asarray(pos, np.float64), theta)


def attention_bwd(q, k, v, allowed, scale, do):
    """Gradients of one head's masked softmax attention (``expert.attention``).

    S = scale q k^T over the allowed keys, P = softmax(S) by rows, O = P v.
    dv = P^T dO;  dP = dO v^T;  dS = P * (dP - rowsum(dP * P));
    dq = scale dS k;  dk = scale dS^T q.  A row with no allowed key has O = 0
    and passes no gradient.
    """
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if k.shape[0] == 0:
        return dq, dk, dv
    s = np.where(allowed, (q @ k.T) * scale, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(allowed, np.exp(s - m), 0.0)
    den = p.sum(axis=1, keepdims=True)
    p = np.divide(p, den, out=np.zeros_like(p), where=den > 0)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
    return scale * ds @ k, scale * ds.T @ q, dv


# ---------------------------------------------------------------------------- one query

def _layer_forward(W, cfg, l, h, pk, pv, pmask):
    """``expert.expert_layer`` with its intermediates kept for the backward pass."""
    p = f"layers.{l}."
    C, H, G, D = h.shape[0], cfg.n_q, cfg.n_kv, cfg.head_dim
    n_valid = int(pmask.sum())
    pos = n_valid + np.arange(C)
    self_layer = l % 2 == 0
    t = {"h": h, "pos": pos}
    t["n1"] = rms_norm(h, W[p + "norm1.g"], cfg.rms_eps)
    t["q"] = rope((t["n1"] @ W[p + "q.w"].T).reshape(C, H, D).transpose(1, 0, 2), pos, cfg.rope_theta)
    kp, vp = pk[:, pmask, :], pv[:, pmask, :]
    if self_layer:
        t["kc"] = rope((t["n1"] @ W[p + "k.w"].T).reshape(C, G, D).transpose(1, 0, 2), pos, cfg.rope_theta)
        t["vc"] = (t["n1"] @ W[p + "v.w"].T).reshape(C, G, D).transpose(1, 0, 2)
        keys, vals = np.concatenate([kp, t["kc"]], axis=1), np.concatenate([vp, t["vc"]], axis=1)
        allowed = np.concatenate([np.ones((C, n_valid), bool), np.tril(np.ones((C, C), bool))], axis=1)
    else:
        keys, vals = kp, vp
        allowed = np.ones((C, n_valid), bool)
    t["keys"], t["vals"], t["allowed"] = keys, vals, allowed
    group = H // G
    o = np.stack([attention(t["q"][hq], keys[hq // group], vals[hq // group], allowed, 1.0 / np.sqrt(D))
                  for hq in range(H)])
    t["o"] = o.transpose(1, 0, 2).reshape(C, H * D)
    t["hm"] = h + t["o"] @ W[p + "o.w"].T
    t["n2"] = rms_norm(t["hm"], W[p + "norm2.g"], cfg.rms_eps)
    t["gate"] = t["n2"] @ W[p + "gate.w"].T
    t["up"] = t["n2"] @ W[p + "up.w"].T
    t["act"] = silu(t["gate"]) * t["up"]
    return t["hm"] + t["act"] @ W[p + "down.w"].T, t


def _layer_backward(W, cfg, l, t, dh_out, grads):
    """Chain rule through one layer; adds the layer's weight gradients to ``grads``."""
    p = f"layers.{l}."
    C, H, G, D = t["h"].shape[0], cfg.n_q, cfg.n_kv, cfg.head_dim
    group = H // G
    # MLP: h_out = hm + act W_down^T, act = silu(gate) * up
    d_act, grads[p + "down.w"], _ = linear_bwd(dh_out, t["act"], W[p + "down.w"])
    d_gate = d_act * t["up"] * silu_grad(t["gate"])
    d_up = d_act * silu(t["gate"])
    dn2_g, grads[p + "gate.w"], _ = linear_bwd(d_gate, t["n2"], W[p + "gate.w"])
    dn2_u, grads[p + "up.w"], _ = linear_bwd(d_up, t["n2"], W[p + "up.w"])
    dhm, grads[p + "norm2.g"] = rms_norm_bwd(dn2_g + dn2_u, t["hm"], W[p + "norm2.g"], cfg.rms_eps)
    dhm = dhm + dh_out
    # attention: hm = h + o W_o^T
    do, grads[p + "o.w"], _ = linear_bwd(dhm, t["o"], W[p + "o.w"])
    do = do.reshape(C, H, D).transpose(1, 0, 2)
    n_prefix = t["keys"].shape[1] - (C if l % 2 == 0 else 0)
    dq = np.zeros((H, C, D))
    dkeys = np.zeros((G,) + t["keys"].shape[1:])
    dvals = np.zeros((G,) + t["vals"].shape[1:])
    for hq in range(H):
        g = hq // group
        dq[hq], dk, dv = attention_bwd(t["q"][hq], t["keys"][g], t["vals"][g], t["allowed"], 1.0 / np.sqrt(D), do[hq])
        dkeys[g] += dk
        dvals[g] += dv
    dq = rope_bwd(dq, t["pos"], cfg.rope_theta).transpose(1, 0, 2).reshape(C, H * D)
    dn1, grads[p + "q.w"], _ = linear_bwd(dq, t["n1"], W[p + "q.w"])
    if l % 2 == 0:
        # the prefix keys/values are frozen inputs: only the chunk's own keys/values carry gradients
        dkc = rope_bwd(dkeys[:, n_prefix:], t["pos"], cfg.rope_theta).transpose(1, 0, 2).reshape(C, G * D)
        dvc = dvals[:, n_prefix:].transpose(1, 0, 2).reshape(C, G * D)
        dn1_k, grads[p + "k.w"], _ = linear_bwd(dkc, t["n1"], W[p + "k.w"])
        dn1_v, grads[p + "v.w"], _ = linear_bwd(dvc, t["n1"], W[p + "v.w"])
        dn1 = dn1 + dn1_k + dn1_v
    dh, grads[p + "norm1.g"] = rms_norm_bwd(dn1, t["h"], W[p + "norm1.g"], cfg.rms_eps)
    return dh + dhm


def query_loss_and_grads(W, cfg, a, eps, t, pk, pv, pmask, n_total):
    """One query's share of the batch loss and of every weight gradient.

    a, eps [chunk, action_dim]; t the query's flow time; pk, pv [n_layers,
    n_kv, P, head_dim]; pmask [P] bool.  The batch loss is the sum of every
    query's squared error divided by n_total = B * chunk * action_dim, so each
    query contributes its sum over n_total.  Returns (loss share, grads, v).
    """
    pmask = np.asarray(pmask, bool)
    a, eps, t = np.asarray(a, np.float64), np.asarray(eps, np.float64), float(t)
    x = t * eps + (1.0 - t) * a
    target = eps - a
    # action and time projections (expert.embed)
    y = x @ W["action_in.w"].T + W["action_in.b"]
    e = time_embedding(t, cfg.d_model, cfg.t_min_period, cfg.t_max_period)
    z = np.concatenate([y, np.broadcast_to(e, (x.shape[0], e.shape[0]))], axis=1)
    s = z @ W["time_in.w"].T + W["time_in.b"]
    h = silu(s) @ W["time_out.w"].T + W["time_out.b"]
    tapes = []
    for l in range(cfg.n_layers):
        h, tp = _layer_forward(W, cfg, l, h, pk[l], pv[l], pmask)
        tapes.append(tp)
    nf = rms_norm(h, W["final_norm.g"], cfg.rms_eps)
    v = nf @ W["action_out.w"].T + W["action_out.b"]
    err = v - target
    loss = float(np.sum(err * err)) / n_total

    grads = {}
    dv = 2.0 * err / n_total
    dnf, grads["action_out.w"], grads["action_out.b"] = linear_bwd(dv, nf, W["action_out.w"])
    dh, grads["final_norm.g"] = rms_norm_bwd(dnf, h, W["final_norm.g"], cfg.rms_eps)
    for l in reversed(range(cfg.n_layers)):
        dh = _layer_backward(W, cfg, l, tapes[l], dh, grads)
    dsil, grads["time_out.w"], grads["time_out.b"] = linear_bwd(dh, silu(s), W["time_out.w"])
    ds = dsil * silu_grad(s)
    dz, grads["time_in.w"], grads["time_in.b"] = linear_bwd(ds, z, W["time_in.w"])
    # the time embedding has no parameters; x_t is data
    _, grads["action_in.w"], grads["action_in.b"] = linear_bwd(dz[:, : cfg.d_model], x, W["action_in.w"])
    return loss, grads, v


def train_batch(W, cfg, prefix_kv_bits, mask, actions, noise, t, queries=None):
    """Loss and gradients of one training batch.

    prefix_kv_bits: bf16 bits [L, 2, B, 5, P, 64]; mask [B, P]; actions, noise
    [B, chunk, action_dim]; t [B].  queries: the batch indices whose terms are
    summed (default all; the loss is always normalised by the whole batch's
    element count, so a subset gives that subset's share).  Returns (loss,
    grads by manifest name).
    """
    B = actions.shape[0]
    n_total = B * actions.shape[1] * actions.shape[2]
    qs = range(B) if queries is None else queries
    loss, grads = 0.0, None
    for b in qs:
        pk = bf16_bits_to_float(prefix_kv_bits[:, 0, b])
        pv = bf16_bits_to_float(prefix_kv_bits[:, 1, b])
        lb, gb, _ = query_loss_and_grads(W, cfg, actions[b], noise[b], t[b], pk, pv, mask[b], n_total)
        loss += lb
        if grads is None:
            grads = gb
        else:
            for k in grads:
                grads[k] = grads[k] + gb[k]
    return loss, grads

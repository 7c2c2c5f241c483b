"""Flow-matching Euler loop and prefix overwrite, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: noeira docs "SmolVLA", Architecture (the chunk is integrated from
pure noise at flow time 1 down to flow time 0 by explicit Euler, one velocity
evaluation of the expert per step; training pairs noise eps with an action
chunk a on the straight line x_t = t * eps + (1 - t) * a, so the velocity to
learn is the constant eps - a).  "Paper vs hardware 11: SmolVLA", What I ran
(when a new chunk starts, its first d ~ 7 rows are pinned to the previous
chunk's tail without any gradient step: the prefix overwrite).
"""
import numpy as np

from .expert import velocity as expert_velocity, bf16_bits_to_float


def schedule(n_steps):
    """Flow times t_0..t_{n-1} and the step dt, as float32 values.

    dt = fl32(-1/n); t_0 = 1; t_{k+1} = fl32(t_k + dt) (repeated float32
    addition).  Exactly n_steps steps are taken.
    """
    dt = np.float32(-1.0 / n_steps)
    ts = []
    t = np.float32(1.0)
    for _ in range(n_steps):
        ts.append(t)
        t = np.float32(t + dt)
    return ts, dt


def overwrite_rows(x, t, eps, prev, d):
    """Prefix overwrite: rows i < d of x become t * eps_i + (1 - t) * a_prev_i.

    This is the point of the flow-matching path at time t between the
    query's own noise eps and the previous chunk's tail a_prev.
    """
    x = x.copy()
    if d > 0:
        t = float(t)
        x[:d] = t * eps[:d] + (1.0 - t) * prev[:d]
    return x


def euler_denoise(vel_fn, noise, n_steps, prev=None, d=0, record=False):
    """Explicit Euler from t = 1 toward t = 0: x <- x + dt * v(x, t).

    vel_fn(x, t) -> v has the shape of x.  When d > 0 the prefix overwrite
    is applied before every step (at step 0 it is a no-op because x = eps)
    and not after the last one.  Returns the final x, or with record=True
    (x, [v_0..v_{n-1}], [x after step 0 .. after step n-1]).
    """
    eps = np.asarray(noise, np.float64)
    x = eps.copy()
    ts, dt = schedule(n_steps)
    vs, xs = [], []
    for t in ts:
        if d > 0:
            x = overwrite_rows(x, t, eps, np.asarray(prev, np.float64), d)
        v = np.asarray(vel_fn(x, t), np.float64)
        x = x + float(dt) * v
        if record:
            vs.append(v)
            xs.append(x)
    return (x, vs, xs) if record else x


def denoise_query(W, cfg, noise, pk, pv, pmask, n_steps=10, prev=None, d=0, record=False,
                  act_round=None):
    """Whole denoising loop for one query with the expert as the velocity field.

    noise [50, 32]; pk, pv [L, 5, P, 64] float64; pmask [P] bool.
    """
    kw = {} if act_round is None else {"act_round": act_round}

    def vel(x, t):
        return expert_velocity(W, cfg, x, t, pk, pv, pmask, **kw)

    return euler_denoise(vel, noise, n_steps, prev=prev, d=d, record=record)


def denoise_batch(W, cfg, prefix_kv_bits, mask, noise, n_steps=10, prev=None, d=0, record=False,
                  queries=None, act_round=None):
    """Run denoise_query on each selected query of a batch (queries are independent).

    prefix_kv_bits: uint16 bf16 bits [L, 2, B, 5, P, 64]; mask uint8 [B, P];
    noise [B, 50, 32]; prev [B, d, 32] or None.  queries: iterable of batch
    indices (default: all).  Returns x [nq, 50, 32] (and per-step v, x lists
    of [nq, 50, 32] arrays with record=True).
    """
    B = noise.shape[0]
    qs = list(range(B)) if queries is None else list(queries)
    xs_out, vs_all, st_all = [], [], []
    for b in qs:
        pk = bf16_bits_to_float(prefix_kv_bits[:, 0, b])
        pv = bf16_bits_to_float(prefix_kv_bits[:, 1, b])
        pm = np.asarray(mask[b]).astype(bool)
        pr = None if prev is None else prev[b]
        r = denoise_query(W, cfg, noise[b], pk, pv, pm, n_steps, pr, d, record, act_round)
        if record:
            xs_out.append(r[0])
            vs_all.append(np.stack(r[1]))
            st_all.append(np.stack(r[2]))
        else:
            xs_out.append(r)
    x = np.stack(xs_out)
    if record:
        # [n_steps, nq, 50, 32]
        return x, np.stack(vs_all, axis=1), np.stack(st_all, axis=1)
    return x

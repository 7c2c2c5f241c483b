"""GPU parity of the flow-matching training step (smolexp_train_step), called through the
C ABI, against the CPU oracle (oracle/train.py).

Tolerance, per gradient tensor: ||gpu - oracle||_F <= 3e-2 ||oracle||_F; the loss within
1e-3 relative.  The matrix products take bf16 operands (relative rounding up to 2^-9, RMS
about 1e-3 per operand), and a weight gradient at layer l is the product of a backward
signal that has passed through (L - l) layers of such products with a forward activation
that has passed through l of them: with 3 products per sub-block on each side, the errors
of some 3L independent roundings add in quadrature, about 1e-3 x sqrt(3 x 16) ~ 7e-3 at
L = 16, which 3e-2 bounds with margin.  The loss is a mean of 1,600 B squared errors
whose bf16 perturbations average out.
"""
import numpy as np
import pytest
import torch

import flow_matching_action_step_amd as fm
import oracle
import synth

pytestmark = pytest.mark.gpu

G_RTOL = 3e-2
LOSS_RTOL = 1e-3


def _say(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


class Trainer:
    def __init__(self, n_layers, max_batch, max_prefix, gain_seed=synth.gen.SEED_GAINS):
        self.cfg = fm.smolexp_default_config(n_layers=n_layers, max_batch=max_batch, max_prefix=max_prefix)
        self.named = synth.draw_weights(n_layers, gain_seed=gain_seed)
        self.W = oracle.decode_weights(self.named)
        self.ocfg = oracle.ExpertConfig(n_layers=n_layers)
        self.h = fm.smolexp_create(self.cfg, 0)
        fm.smolexp_load_weights(self.h, synth.pack_weights(self.named, n_layers))
        self.n = fm.smolexp_weight_count(self.cfg)

    def step(self, kv, mask, a, eps, t):
        d = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in
             (("kv", kv.view(np.int16)), ("mask", mask), ("a", a), ("eps", eps), ("t", t))}
        grads = torch.full((self.n,), float("nan"), dtype=torch.float32, device="cuda")
        loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        fm.smolexp_train_step(self.h, self.cfg, d["kv"], d["mask"], d["a"], d["eps"], d["t"], grads, loss)
        torch.cuda.synchronize()
        return float(loss.cpu()[0]), grads.cpu().numpy(), d

    def close(self):
        if self.h is not None:
            fm.smolexp_destroy(self.h)
            self.h = None


def _unpack(flat, n_layers):
    out, off = {}, 0
    for name, shape, _ in synth.manifest(n_layers):
        n = int(np.prod(shape))
        out[name] = flat[off:off + n].reshape(shape)
        off += n
    assert off == flat.size
    return out


def _compare(tr, loss, flat, kv, mask, a, eps, t, label, queries=None):
    B = a.shape[0]
    if queries is None:
        ol, og = oracle.train_batch(tr.W, tr.ocfg, kv, mask, a.astype(np.float64), eps.astype(np.float64),
                                    t.astype(np.float64))
    else:
        raise NotImplementedError
    assert np.isfinite(flat).all(), f"{label}: non-finite gradients"
    got = _unpack(flat, tr.cfg.n_layers)
    rel_loss = abs(loss - ol) / abs(ol)
    worst, worst_name = 0.0, ""
    for name, ref in og.items():
        den = np.linalg.norm(ref)
        rel = np.linalg.norm(got[name] - ref) / den if den > 0 else np.linalg.norm(got[name])
        if rel > worst:
            worst, worst_name = rel, name
        assert rel <= G_RTOL, f"{label}: {name} rel. error {rel:.3e} > {G_RTOL}"
    print(f"[parity] {label} B={B}: loss {loss:.6f} vs {ol:.6f} (rel {rel_loss:.1e}); worst gradient "
          f"{worst_name} {worst:.2e}", flush=True)
    assert rel_loss <= LOSS_RTOL, f"{label}: loss rel. error {rel_loss:.3e}"
    return worst


def test_train_step_two_layers_ragged_nan_pads():
    _say("train step, 2 layers (self, cross), batch 3, P = 70, ragged prefixes, NaN pads")
    L, B, P = 2, 3, 70
    tr = Trainer(L, B, P)
    try:
        kv = synth.draw_prefix_kv(L, B, P)
        mask = synth.make_mask(B, P, [70, 33, 1])
        mask[0, [4, 5, 66]] = 0
        for b in range(B):
            kv[:, :, b, :, mask[b] == 0] = 0x7FC0  # NaN keys and values on every pad
        a, eps, t = synth.draw_actions(B), synth.draw_noise(B), np.array([0.9, 0.35, 0.02], np.float32)
        loss, flat, _ = tr.step(kv, mask, a, eps, t)
        _compare(tr, loss, flat, kv, mask, a, eps, t, "train2 p70")
    finally:
        tr.close()


def test_train_step_four_layers_tiles_and_ragged_tail():
    # batch 5: 250 rows = one full 128-row GEMM tile and a ragged one; P = 130 spans three
    # 64-key blocks of the attention
    _say("train step, 4 layers, batch 5, P = 130")
    L, B, P = 4, 5, 130
    tr = Trainer(L, B, P)
    try:
        kv = synth.draw_prefix_kv(L, B, P)
        mask = synth.make_mask(B, P, [130, 64, 65, 100, 127])
        a, eps, t = synth.draw_actions(B), synth.draw_noise(B), synth.draw_flow_times(B)
        loss, flat, _ = tr.step(kv, mask, a, eps, t)
        _compare(tr, loss, flat, kv, mask, a, eps, t, "train4 p130")
    finally:
        tr.close()


def test_train_step_sixteen_layers():
    _say("train step, 16 layers, batch 2, P = 177")
    L, B, P = 16, 2, 177
    tr = Trainer(L, B, P)
    try:
        kv = synth.draw_prefix_kv(L, B, P)
        mask = synth.make_mask(B, P, [177, 150])
        a, eps, t = synth.draw_actions(B), synth.draw_noise(B), synth.draw_flow_times(B)
        loss, flat, _ = tr.step(kv, mask, a, eps, t)
        _compare(tr, loss, flat, kv, mask, a, eps, t, "train16 p177")
    finally:
        tr.close()


def test_train_step_edges_empty_prefix_and_t_extremes():
    # a query with no valid prefix token (its cross layers see no key: output 0, no
    # gradient through them) and flow times 0 and 1 (x_t = a and x_t = eps)
    _say("train step edges: n_valid = 0, t = 0 and t = 1, P = 1")
    L, B, P = 2, 2, 1
    tr = Trainer(L, B, P)
    try:
        kv = synth.draw_prefix_kv(L, B, P)
        mask = np.array([[0], [1]], np.uint8)
        kv[:, :, 0] = 0x7FC0
        a, eps, t = synth.draw_actions(B), synth.draw_noise(B), np.array([0.0, 1.0], np.float32)
        loss, flat, _ = tr.step(kv, mask, a, eps, t)
        _compare(tr, loss, flat, kv, mask, a, eps, t, "train2 p1 edges")
    finally:
        tr.close()


def test_train_step_deterministic_inputs_untouched_and_errors():
    _say("train step: determinism, inputs untouched, errors")
    L, B, P = 2, 2, 40
    tr = Trainer(L, B, P)
    try:
        kv = synth.draw_prefix_kv(L, B, P)
        mask = synth.make_mask(B, P, [40, 21])
        a, eps, t = synth.draw_actions(B), synth.draw_noise(B), synth.draw_flow_times(B)
        l0, g0, d = tr.step(kv, mask, a, eps, t)
        before = {k: v.clone() for k, v in d.items()}
        grads = torch.empty(tr.n, dtype=torch.float32, device="cuda")
        loss = torch.empty(1, dtype=torch.float32, device="cuda")
        fm.smolexp_train_step(tr.h, tr.cfg, d["kv"], d["mask"], d["a"], d["eps"], d["t"], grads, loss)
        torch.cuda.synchronize()
        assert float(loss.cpu()[0]) == l0
        np.testing.assert_array_equal(grads.cpu().numpy(), g0)
        for k in d:
            assert torch.equal(d[k], before[k]), k
        l1, g1, _ = tr.step(kv, mask, a, eps, t)
        np.testing.assert_array_equal(g1, g0)
        import ctypes
        lib = fm.raw()
        p = ctypes.c_void_p(grads.data_ptr())
        assert lib.smolexp_train_step(tr.h, p, p, P, p, p, p, p, None, B, None) == fm.SMOLEXP_E_INVAL
        assert lib.smolexp_train_step(tr.h, p, p, P, p, p, p, p, p, B + 1, None) == fm.SMOLEXP_E_INVAL
        cfg = fm.smolexp_default_config(n_layers=L, max_batch=B, max_prefix=P)
        h2 = fm.smolexp_create(cfg, 0)
        try:
            assert lib.smolexp_train_step(h2, p, p, P, p, p, p, p, p, B, None) == fm.SMOLEXP_E_STATE
        finally:
            fm.smolexp_destroy(h2)
    finally:
        tr.close()


def test_train_step_full_size_b64_p257():
    """The benchmarked configuration (16 layers, 64 samples, prefix 257): the loss and the
    gradient of action_out.b (2 / n times the column sums of v - target) against the oracle's
    forward pass for every sample, and the batch's gradients against the mean of the
    gradients of its two halves (the loss is a per-element mean, so that identity holds
    exactly in exact arithmetic; it exercises the full-size k-split and workspace).

    The two GPU results are not bitwise related: the k-split of a product depends on its
    row count, so the halves sum in another fp32 order, and the chain of bf16 roundings turns
    any 1-ulp difference into another draw of the same rounding noise (a perturbation d
    flips about d / 2^-9 of the roundings of the next bf16 operand, an RMS change of about
    sqrt(d 2^-9); a few such stages reach the full noise level).  Each side is within the
    parity bound of the exact gradient, so they differ by at most twice that bound.
    """
    _say("train step at the bench size: 16 layers, batch 64, P = 257")
    L, B, P = 16, 64, 257
    wl = synth.make_workload("expert16_b64_p257", with_weights=False)
    tr = Trainer(L, B, P, gain_seed=None)
    try:
        kv, mask = wl["prefix_kv"], wl["mask"]
        a, eps, t = synth.draw_actions(B), wl["noise"], synth.draw_flow_times(B)
        loss, flat, _ = tr.step(kv, mask, a, eps, t)
        assert np.isfinite(flat).all()
        halves = []
        for sl in (slice(0, 32), slice(32, 64)):
            halves.append(tr.step(np.ascontiguousarray(kv[:, :, sl]), mask[sl], a[sl], eps[sl], t[sl]))
        g_half = 0.5 * (halves[0][1] + halves[1][1])
        l_half = 0.5 * (halves[0][0] + halves[1][0])
        got, want = _unpack(flat, L), _unpack(g_half, L)
        worst = max(np.linalg.norm(got[n] - want[n]) / np.linalg.norm(want[n]) for n in got)
        # the oracle's loss: each sample's velocity from the float64 forward pass
        se, err_sum = 0.0, np.zeros(32)
        for b in range(B):
            pk, pv = oracle.bf16_bits_to_float(kv[:, 0, b]), oracle.bf16_bits_to_float(kv[:, 1, b])
            x = float(t[b]) * eps[b].astype(np.float64) + (1 - float(t[b])) * a[b].astype(np.float64)
            v = oracle.velocity(tr.W, tr.ocfg, x, float(t[b]), pk, pv, mask[b].astype(bool))
            err = v - (eps[b].astype(np.float64) - a[b])
            se += float(np.sum(err ** 2))
            err_sum += err.sum(axis=0)
        n = B * 50 * 32
        ol = se / n
        # d loss / d b_out = 2 / n times the column sums of (v - target): exact from the forward
        gb = 2.0 * err_sum / n
        rel_b = np.linalg.norm(got["action_out.b"] - gb) / np.linalg.norm(gb)
        print(f"[parity] train16 b64 p257: loss {loss:.6f} vs oracle {ol:.6f} (rel {abs(loss - ol) / ol:.1e}); "
              f"action_out.b rel {rel_b:.2e}; halves: loss {l_half:.6f}, worst gradient rel {worst:.2e}", flush=True)
        assert abs(loss - ol) <= LOSS_RTOL * ol
        assert rel_b <= G_RTOL
        assert abs(loss - l_half) <= 1e-5 * ol
        assert worst <= 2 * G_RTOL
    finally:
        tr.close()


def test_train_step_graph_replays_match_eager():
    """With graphs on (the default) a training step is captured once per call signature and
    replayed; every replay, with other device work in between, must equal the eager launches
    bit for bit."""
    _say("train step: graph replays vs eager launches")
    L, B, P = 2, 3, 48
    named = synth.draw_weights(L, gain_seed=synth.gen.SEED_GAINS)
    hs = []
    try:
        for graphs in (1, 0):
            cfg = fm.smolexp_default_config(n_layers=L, max_batch=B, max_prefix=P, use_graphs=graphs)
            h = fm.smolexp_create(cfg, 0)
            hs.append((h, cfg))
            fm.smolexp_load_weights(h, synth.pack_weights(named, L))
        kv = synth.draw_prefix_kv(L, B, P)
        mask = synth.make_mask(B, P, [48, 30, 7])
        d = [torch.from_numpy(np.ascontiguousarray(x)).cuda()
             for x in (kv.view(np.int16), mask, synth.draw_actions(B), synth.draw_noise(B), synth.draw_flow_times(B))]
        n = fm.smolexp_weight_count(hs[0][1])
        ge, le = torch.empty(n, device="cuda"), torch.empty(1, device="cuda")
        fm.smolexp_train_step(hs[1][0], hs[1][1], *d, ge, le)
        torch.cuda.synchronize()
        want_g, want_l = ge.cpu().numpy(), le.cpu().numpy()
        for rep in range(3):
            gg, lg = torch.full((n,), float("nan"), device="cuda"), torch.full((1,), float("nan"), device="cuda")
            fm.smolexp_train_step(hs[0][0], hs[0][1], *d, gg, lg)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(gg.cpu().numpy(), want_g, err_msg=f"replay {rep}")
            np.testing.assert_array_equal(lg.cpu().numpy(), want_l)
            # eager work between replays (another step on the eager handle, a torch reduction)
            fm.smolexp_train_step(hs[1][0], hs[1][1], *d, ge, le)
            _ = float((ge * 2).sum())
            torch.cuda.synchronize()
            # copies of the inputs at other addresses: a second graph, the same results
            d2 = [x.clone() for x in d]
            fm.smolexp_train_step(hs[0][0], hs[0][1], *d2, gg, lg)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(gg.cpu().numpy(), want_g)
    finally:
        for h, _ in hs:
            fm.smolexp_destroy(h)

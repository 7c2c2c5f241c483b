"""Shared helpers of the GPU tests: put seeded workloads on the device, run the
library through its C ABI, run the CPU oracle on the same inputs, compare."""
import numpy as np
import torch

import flow_matching_action_step_amd as fm
import oracle
import synth

# Tolerances of the comparison with the oracle (fixed before any kernel ran):
VEL_RTOL = 1e-2   # per step k and query b: ||v_k,b(gpu) - v_k,b(oracle)||_F / ||v_k,b(oracle)||_F
ACT_ATOL = 2e-2   # final actions: elementwise max |gpu - oracle|


class Expert:
    """A library handle with loaded weights plus the oracle's float64 copy of them."""

    def __init__(self, n_layers, n_steps=10, max_batch=16, max_prefix=512, gain_seed=None, use_graphs=1,
                 with_oracle=True, weight_format=fm.SMOLEXP_WEIGHTS_FP16):
        self.cfg = fm.smolexp_default_config(n_layers=n_layers, n_steps=n_steps, max_batch=max_batch,
                                             max_prefix=max_prefix, use_graphs=use_graphs,
                                             weight_format=weight_format)
        self.named = synth.draw_weights(n_layers, gain_seed=gain_seed)
        self.h = fm.smolexp_create(self.cfg, 0)
        fm.smolexp_load_weights(self.h, synth.pack_weights(self.named, n_layers))
        self.ocfg = oracle.ExpertConfig(n_layers=n_layers)
        self.W = oracle.decode_weights(self.named) if with_oracle else None
        if self.W is not None and weight_format == fm.SMOLEXP_WEIGHTS_E4M3:
            # the 8-bit model: the streamed matrices quantized by rows, as the oracle defines it
            self.W = oracle.quant.streamed_weights(self.W, self.ocfg)

    def sibling(self, n_steps, max_batch=4, max_prefix=256):
        """Another handle on the same weights with a different number of Euler steps."""
        e = object.__new__(Expert)
        e.cfg = fm.smolexp_default_config(n_layers=self.cfg.n_layers, n_steps=n_steps, max_batch=max_batch,
                                          max_prefix=max_prefix, use_graphs=self.cfg.use_graphs)
        e.named, e.W, e.ocfg = self.named, self.W, self.ocfg
        e.h = fm.smolexp_create(e.cfg, 0)
        fm.smolexp_load_weights(e.h, synth.pack_weights(self.named, self.cfg.n_layers))
        return e

    def close(self):
        if self.h is not None:
            fm.smolexp_destroy(self.h)
            self.h = None


def to_device(wl):
    d = {}
    d["kv"] = torch.from_numpy(np.ascontiguousarray(wl["prefix_kv"]).view(np.int16)).cuda()
    d["mask"] = torch.from_numpy(np.ascontiguousarray(wl["mask"])).cuda()
    d["noise"] = torch.from_numpy(np.ascontiguousarray(wl["noise"])).cuda()
    d["prev"] = None if wl["prev_actions"] is None else torch.from_numpy(wl["prev_actions"]).cuda()
    return d


def run_gpu(ex, dev, d=0, record=True, stream=None):
    B = dev["mask"].shape[0]
    n = ex.cfg.n_steps
    out = torch.full((B, 50, 32), float("nan"), device="cuda")
    vel = torch.full((n, B, 50, 32), float("nan"), device="cuda") if record else None
    st = torch.full((n, B, 50, 32), float("nan"), device="cuda") if record else None
    fm.smolexp_denoise_ex(ex.h, ex.cfg, dev["kv"], dev["mask"], dev["noise"], out,
                          prev_actions=dev["prev"] if d > 0 else None, overwrite_rows=d,
                          out_velocities=vel, out_states=st, stream=stream)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy()}
    if record:
        res["vel"] = vel.cpu().numpy()
        res["st"] = st.cpu().numpy()
    return res


def run_oracle(ex, wl, queries, d=0, n_steps=None):
    n = ex.cfg.n_steps if n_steps is None else n_steps
    x, vs, xs = oracle.denoise_batch(ex.W, ex.ocfg, wl["prefix_kv"], wl["mask"], wl["noise"], n_steps=n,
                                     prev=wl["prev_actions"], d=d, record=True, queries=queries)
    return {"out": x, "vel": vs, "st": xs}


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def compare(gpu, orc, queries, noise, label="", d=0):
    """Assert the tolerances; return (max velocity rel. error, max action error).

    The velocity bound holds for every query and step on its own (one bad query cannot
    hide among good ones) and, when the first d rows are overwritten, on those rows of
    every query and step separately; the error over all compared queries is printed."""
    q = list(queries)
    vg = gpu["vel"][:, q]
    worst_v = worst_joint = worst_ow = 0.0
    for k in range(vg.shape[0]):
        worst_joint = max(worst_joint, _rel(vg[k], orc["vel"][k]))
        for j, b in enumerate(q):
            rel = _rel(vg[k, j], orc["vel"][k, j])
            worst_v = max(worst_v, rel)
            assert rel <= VEL_RTOL, f"{label} step {k} query {b}: velocity rel. error {rel:.3e} > {VEL_RTOL}"
            if d > 0:
                rel = _rel(vg[k, j, :d], orc["vel"][k, j, :d])
                worst_ow = max(worst_ow, rel)
                assert rel <= VEL_RTOL, f"{label} step {k} query {b} rows < {d}: velocity rel. error {rel:.3e}"
    err = np.abs(gpu["out"][q] - orc["out"])
    act = float(err.max())
    assert act <= ACT_ATOL, f"{label}: action max-abs error {act:.3e} > {ACT_ATOL}"
    # the returned chunk is the last Euler state, and every recorded state is finite
    np.testing.assert_array_equal(gpu["out"], gpu["st"][-1])
    assert np.isfinite(gpu["vel"]).all() and np.isfinite(gpu["st"]).all()
    # the expert's contribution is far above the tolerance, so the action check is not vacuous
    assert np.abs(orc["out"] - noise[q]).max() > 10 * ACT_ATOL
    jq, row = np.unravel_index(int(np.argmax(err.max(axis=2))), err.shape[:2])
    ow = f", rows < {d} {worst_ow:.3e}" if d > 0 else ""
    print(f"[parity] {label}: velocity rel worst query {worst_v:.3e} (all queries {worst_joint:.3e}{ow}), "
          f"action max-abs {act:.3e} (query {q[jq]}, row {row})", flush=True)
    return worst_v, act

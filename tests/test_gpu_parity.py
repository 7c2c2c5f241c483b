"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Tolerances (tests/gpu_util.py): per-step velocities within 1e-2 norm-relative,
final actions within 2e-2 max-abs.  Workloads are the five seeded synthetic
ones; at batch 64 and 128 the oracle computes a sample of queries (queries are
independent) while the GPU runs the whole batch in the benchmark's launch
configuration.
"""
import ctypes

import numpy as np
import pytest
import torch

import flow_matching_action_step_amd as fm
import oracle
import synth
from gpu_util import Expert, to_device, run_gpu, run_oracle, compare, VEL_RTOL, ACT_ATOL

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def ex4():
    _say("create 4-layer expert")
    e = Expert(4, max_batch=16, max_prefix=512)
    yield e
    e.close()


@pytest.fixture(scope="module")
def ex16():
    _say("create 16-layer expert (max_batch 128)")
    e = Expert(16, max_batch=128, max_prefix=512)
    yield e
    e.close()


# ------------------------------------------------------------------ C ABI on a device

def test_abi_errors_on_device():
    _say("abi errors")
    lib = fm.raw()
    cfg = fm.smolexp_default_config(n_layers=2, max_batch=4, max_prefix=64)
    h = fm.smolexp_create(cfg, 0)
    try:
        dev = torch.zeros(16, device="cuda")
        p = ctypes.c_void_p(dev.data_ptr())
        assert lib.smolexp_denoise(h, p, p, 8, p, p, 1, None) == fm.SMOLEXP_E_STATE
        w = np.zeros(synth.weight_count(2) - 1, np.uint16)
        assert lib.smolexp_load_weights(h, w.ctypes.data_as(ctypes.c_void_p), w.size) == fm.SMOLEXP_E_SIZE
        w = synth.pack_weights(synth.draw_weights(2), 2)
        assert lib.smolexp_load_weights(h, w.ctypes.data_as(ctypes.c_void_p), w.size) == 0
        assert lib.smolexp_denoise(h, p, p, 8, p, p, 0, None) == fm.SMOLEXP_E_INVAL
        assert lib.smolexp_denoise(h, p, p, 8, p, p, 5, None) == fm.SMOLEXP_E_INVAL
        assert lib.smolexp_denoise(h, p, p, 0, p, p, 1, None) == fm.SMOLEXP_E_INVAL
        assert lib.smolexp_denoise(h, p, p, 65, p, p, 1, None) == fm.SMOLEXP_E_INVAL
        assert lib.smolexp_denoise(h, None, p, 8, p, p, 1, None) == fm.SMOLEXP_E_INVAL
        assert "NULL" in fm.smolexp_last_error(h)
        o = fm.smolexp_denoise_opts()
        o.overwrite_rows = 51
        assert lib.smolexp_denoise_ex(h, p, p, 8, p, p, 1, None, ctypes.byref(o)) == fm.SMOLEXP_E_INVAL
        o.overwrite_rows = 3
        assert lib.smolexp_denoise_ex(h, p, p, 8, p, p, 1, None, ctypes.byref(o)) == fm.SMOLEXP_E_INVAL
        assert lib.smolexp_velocity(h, p, p, 8, p, float("nan"), p, 1, None) == fm.SMOLEXP_E_INVAL
        us = ctypes.c_float()
        assert lib.smolexp_time_kernel(h, 0, 1, None, ctypes.byref(us)) == fm.SMOLEXP_E_STATE
    finally:
        fm.smolexp_destroy(h)


# ------------------------------------------------------------------ teacher-forced single steps

def test_velocity_teacher_forced_4_layers(ex4):
    _say("velocity, 4 layers, teacher forced")
    wl = synth.make_workload("expert4_b1_p177", with_weights=False)
    dev = to_device(wl)
    orc = run_oracle(ex4, wl, [0])
    ts, _ = oracle.schedule(10)
    for k in (0, 5, 9):
        x_np = wl["noise"][0].astype(np.float64) if k == 0 else orc["st"][k - 1][0]
        x = torch.from_numpy(x_np.astype(np.float32)[None]).cuda()
        v = torch.empty_like(x)
        fm.smolexp_velocity(ex4.h, ex4.cfg, dev["kv"], dev["mask"], x, float(ts[k]), v)
        torch.cuda.synchronize()
        want = oracle.velocity(ex4.W, ex4.ocfg, x_np.astype(np.float32).astype(np.float64), ts[k],
                               oracle.bf16_bits_to_float(wl["prefix_kv"][:, 0, 0]),
                               oracle.bf16_bits_to_float(wl["prefix_kv"][:, 1, 0]), wl["mask"][0].astype(bool))
        got = v.cpu().numpy()[0]
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        print(f"[parity] velocity step {k}: rel {rel:.3e}", flush=True)
        assert rel <= VEL_RTOL


@pytest.mark.parametrize("n_layers", [1, 2])
def test_velocity_one_self_layer_then_a_cross_layer(n_layers):
    """One evaluation of v_theta with a single self-attention layer (embedding, RMSNorm'd
    Q/K/V + RoPE, attention over prefix + causal chunk, o, SwiGLU MLP, head), then with the
    cross-attention layer added, at batch 3 with ragged prefixes and random x and t: the layer
    types in isolation, through the C ABI."""
    _say(f"velocity, {n_layers} layer(s), batch 3, ragged prefixes")
    ex = Expert(n_layers, max_batch=3, max_prefix=130, gain_seed=synth.gen.SEED_GAINS)
    try:
        B, P = 3, 130
        kv = synth.draw_prefix_kv(n_layers, B, P)
        mask = synth.make_mask(B, P, [130, 64, 1])
        rng = np.random.default_rng(40 + n_layers)
        x_np = rng.standard_normal((B, 50, 32)).astype(np.float32)
        kv_d = torch.from_numpy(kv.view(np.int16)).cuda()
        mask_d = torch.from_numpy(mask).cuda()
        for t in (1.0, 0.37):
            x = torch.from_numpy(x_np).cuda()
            v = torch.empty_like(x)
            fm.smolexp_velocity(ex.h, ex.cfg, kv_d, mask_d, x, t, v)
            torch.cuda.synchronize()
            got = v.cpu().numpy()
            for b in range(B):
                want = oracle.velocity(ex.W, ex.ocfg, x_np[b].astype(np.float64), np.float32(t),
                                       oracle.bf16_bits_to_float(kv[:, 0, b]), oracle.bf16_bits_to_float(kv[:, 1, b]),
                                       mask[b].astype(bool))
                rel = np.linalg.norm(got[b] - want) / np.linalg.norm(want)
                print(f"[parity] velocity L={n_layers} t={t} query {b}: rel {rel:.3e}", flush=True)
                assert rel <= VEL_RTOL
    finally:
        ex.close()


# ------------------------------------------------------------------ whole loop, the five workloads

def test_denoise_4_layers_batch1(ex4):
    _say("denoise expert4_b1_p177")
    wl = synth.make_workload("expert4_b1_p177", with_weights=False)
    gpu = run_gpu(ex4, to_device(wl))
    compare(gpu, run_oracle(ex4, wl, [0]), [0], wl["noise"], "expert4_b1_p177")


def test_denoise_16_layers_batch1(ex16):
    _say("denoise expert16_b1_p177")
    wl = synth.make_workload("expert16_b1_p177", with_weights=False)
    gpu = run_gpu(ex16, to_device(wl))
    compare(gpu, run_oracle(ex16, wl, [0]), [0], wl["noise"], "expert16_b1_p177")


def test_denoise_16_layers_four_steps(ex16):
    # the step-count variant (dt = -1/4) on the 16-layer expert, as `bench.py --n-steps 4` runs it
    _say("denoise expert16_b1_p177 with 4 Euler steps")
    ex = ex16.sibling(4)
    try:
        wl = synth.make_workload("expert16_b1_p177", batch=2, with_weights=False)
        gpu = run_gpu(ex, to_device(wl))
        assert gpu["vel"].shape[0] == 4
        compare(gpu, run_oracle(ex, wl, [0, 1]), [0, 1], wl["noise"], "expert16_b1_p177 n=4")
    finally:
        ex.close()


def test_denoise_16_layers_batch16_variable_prefix(ex16):
    _say("denoise expert16_b16_pvar241")
    wl = synth.make_workload("expert16_b16_pvar241", with_weights=False)
    gpu = run_gpu(ex16, to_device(wl))
    # the shortest and the longest prefixes plus two more
    order = np.argsort(wl["lengths"])
    q = sorted({int(order[0]), int(order[-1]), 3, 10})
    compare(gpu, run_oracle(ex16, wl, q), q, wl["noise"], "expert16_b16_pvar241")


def test_denoise_16_layers_batch24_variable_prefix(ex16):
    # 1200 chunk rows: the K-split GEMM at its largest tiles for Q/K/V and o, the pipelined
    # GEMM with 64-row tiles and a 4-stage ring for down, the streamed-ring attention
    _say("denoise expert16_b16_pvar241 at batch 24")
    wl = synth.make_workload("expert16_b16_pvar241", batch=24, with_weights=False)
    gpu = run_gpu(ex16, to_device(wl))
    order = np.argsort(wl["lengths"])
    q = sorted({int(order[0]), int(order[-1]), 17})
    compare(gpu, run_oracle(ex16, wl, q), q, wl["noise"], "expert16_b24_pvar241")


def test_streamed_attention_variants_4_layers():
    # batch 28 (four-wave workgroups, four per CU) and 40 (ten waves: all 150 rows of a
    # KV head in one workgroup), the streamed-attention variants no other test batch takes
    _say("4 layers at batch 28 and 40 (streamed attention variants)")
    ex = Expert(4, max_batch=40, max_prefix=256)
    try:
        for B, q in ((28, [0, 27]), (40, [5, 39])):
            wl = synth.make_workload("expert4_b1_p177", batch=B, with_weights=False)
            gpu = run_gpu(ex, to_device(wl))
            compare(gpu, run_oracle(ex, wl, q), q, wl["noise"], f"expert4 batch {B}")
    finally:
        ex.close()


def test_denoise_16_layers_batch64(ex16):
    _say("denoise expert16_b64_p257 (sampled queries)")
    wl = synth.make_workload("expert16_b64_p257", with_weights=False)
    gpu = run_gpu(ex16, to_device(wl))
    q = [0, 37, 63]
    compare(gpu, run_oracle(ex16, wl, q), q, wl["noise"], "expert16_b64_p257")


def test_denoise_16_layers_batch128_overwrite(ex16):
    _say("denoise expert16_b128_p177_ow7 (sampled queries)")
    wl = synth.make_workload("expert16_b128_p177_ow7", with_weights=False)
    gpu = run_gpu(ex16, to_device(wl), d=7)
    q = [0, 64, 127]
    compare(gpu, run_oracle(ex16, wl, q, d=7), q, wl["noise"], "expert16_b128_p177_ow7", d=7)
    # rows below d after the last step: the overwrite set them before step 9 and one Euler step followed
    ts, dt = oracle.schedule(10)
    t9 = float(ts[-1])
    before = t9 * wl["noise"][q, :7] + (1 - t9) * wl["prev_actions"][q]
    np.testing.assert_allclose(gpu["out"][q, :7], before + float(dt) * gpu["vel"][-1][q, :7], rtol=0, atol=1e-5)


# ------------------------------------------------------------------ invariants on the GPU

def test_inputs_untouched_and_runs_deterministic(ex4):
    _say("inputs untouched, determinism")
    wl = synth.make_workload("expert4_b1_p177", batch=3, with_weights=False)
    dev = to_device(wl)
    snap = {k: v.clone() for k, v in dev.items() if v is not None}
    a = run_gpu(ex4, dev)
    b = run_gpu(ex4, dev)
    for k, v in snap.items():
        assert torch.equal(v, dev[k]), k
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_pad_invariance_with_nan_pads(ex4):
    _say("pad invariance")
    wl = synth.make_workload("expert4_b1_p177", batch=3, with_weights=False)
    wl["mask"][0, 150:] = 0
    wl["mask"][1, ::3] = 0          # interleaved pads
    dev = to_device(wl)
    a = run_gpu(ex4, dev)
    kv = wl["prefix_kv"].copy()
    for b, p in zip(*np.nonzero(wl["mask"] == 0)):
        kv[:, :, b, :, p, :] = 0x7FC0   # bf16 NaN in every masked slot
    dev["kv"] = torch.from_numpy(kv.view(np.int16)).cuda()
    b = run_gpu(ex4, dev)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    q = [0, 1]
    compare(a, run_oracle(ex4, wl, q), q, wl["noise"], "expert4 pads")


def test_chunk_causality(ex4):
    _say("chunk causality")
    wl = synth.make_workload("expert4_b1_p177", with_weights=False)
    dev = to_device(wl)
    x = dev["noise"].clone()
    v0 = torch.empty_like(x)
    fm.smolexp_velocity(ex4.h, ex4.cfg, dev["kv"], dev["mask"], x, 0.6, v0)
    x[0, 20] += 1.0
    v1 = torch.empty_like(x)
    fm.smolexp_velocity(ex4.h, ex4.cfg, dev["kv"], dev["mask"], x, 0.6, v1)
    torch.cuda.synchronize()
    assert torch.equal(v0[0, :20], v1[0, :20])
    assert (v0[0, 20:] - v1[0, 20:]).abs().max() > 1e-4


def test_batch_invariance(ex4):
    _say("batch invariance")
    wl = synth.make_workload("expert4_b1_p177", batch=5, with_weights=False)
    wl["mask"][2, 100:] = 0
    full = run_gpu(ex4, to_device(wl))
    one = {k: (v[2:3] if k != "prefix_kv" else v[:, :, 2:3]) for k, v in wl.items()
           if isinstance(v, np.ndarray)}
    one["prev_actions"] = None
    alone = run_gpu(ex4, to_device(one))
    np.testing.assert_allclose(alone["out"][0], full["out"][2], atol=ACT_ATOL / 4)
    rel = np.linalg.norm(alone["vel"][:, 0] - full["vel"][:, 2]) / np.linalg.norm(full["vel"][:, 2])
    assert rel < VEL_RTOL / 4


# ------------------------------------------------------------------ edge cases

def test_edge_single_key_empty_prefix_and_ragged(ex4):
    _say("edge cases: P=1, empty prefix, ragged P")
    for P, lens in ((1, [1, 0]), (65, [65, 0]), (130, [3, 129])):
        wl = synth.make_workload("expert4_b1_p177", batch=2, with_weights=False)
        wl["prefix_kv"] = synth.draw_prefix_kv(4, 2, P)
        wl["mask"] = synth.make_mask(2, P, lens)
        wl["prefix_len"] = P
        gpu = run_gpu(ex4, to_device(wl))
        compare(gpu, run_oracle(ex4, wl, [0, 1]), [0, 1], wl["noise"], f"P={P} lengths={lens}")


def _nan_pads(wl):
    kv = wl["prefix_kv"]
    for b, p in zip(*np.nonzero(wl["mask"] == 0)):
        kv[:, :, b, :, p, :] = 0x7FC0   # bf16 NaN in every masked slot


def test_long_prefixes_take_several_key_rounds(ex4):
    """Prefixes longer than one staged round of the small-batch attention kernels (320 keys):
    batch 2 at P = 450 (self layers stage 500 keys, cross layers 450, in two rounds each) with
    one full prefix and one of 300 valid tokens interleaved with NaN pads; P = 300, where the
    chunk's keys straddle the round boundary; and the streamed kernel at batch 16 near the
    handle's max_prefix (P = 512, 480..512 valid, NaN pads)."""
    _say("long prefixes: several key rounds, NaN pads")
    for P, B in ((450, 2), (300, 2), (512, 16)):
        wl = synth.make_workload("expert4_b1_p177", batch=B, with_weights=False)
        wl["prefix_kv"] = synth.draw_prefix_kv(4, B, P, seed=81 + P)
        wl["prefix_len"] = P
        if B == 2:
            mask = synth.make_mask(2, P, [P, P])
            mask[1] = (np.arange(P) % 3 != 1) if P == 450 else (np.arange(P) < 270)
            wl["mask"] = mask.astype(np.uint8)
        else:
            lens = [int(x) for x in synth.draw_lengths(B, 480, 512, seed=83)]
            wl["mask"] = synth.make_mask(B, P, lens)
            wl["mask"][3, ::7] = 0   # interleaved pads in one query
        wl["lengths"] = wl["mask"].sum(axis=1)
        _nan_pads(wl)
        gpu = run_gpu(ex4, to_device(wl))
        q = [0, 1] if B == 2 else [0, 3, 15]
        compare(gpu, run_oracle(ex4, wl, q), q, wl["noise"], f"P={P} batch {B} valid {[int(x) for x in wl['lengths'][q]]}")


def test_key_block_and_round_boundaries(ex4):
    """Key counts on either side of a 64-key block and of a staged round (five blocks at batch <= 8):
    self layers see P + 50 keys, cross layers P.  Batch 2: P = 14 (self 64, one whole block), 64
    (cross one whole block), 78 (self 128), 270 (self 320, one whole round), 271 (self 321: the
    second round holds only the last chunk key), 320 (cross one whole round), 321 (cross 321);
    batch 16 (the streamed kernel): P = 206 (self 256) and 257 (cross 257).  Each second query has a
    shorter valid prefix; NaN in every masked slot."""
    cases = ((14, 2, [14, 13]), (64, 2, [64, 63]), (78, 2, [78, 1]), (270, 2, [270, 269]),
             (271, 2, [271, 200]), (320, 2, [320, 319]), (321, 2, [321, 1]), (206, 16, None), (257, 16, None))
    for P, B, lens in cases:
        _say(f"key boundaries: P = {P}, batch {B}")
        wl = synth.make_workload("expert4_b1_p177", batch=B, with_weights=False)
        wl["prefix_kv"] = synth.draw_prefix_kv(4, B, P, seed=91 + P)
        wl["prefix_len"] = P
        if lens is None:
            lens = [P] + [int(x) for x in synth.draw_lengths(B - 1, P - 63, P, seed=93 + P)]
        wl["mask"] = synth.make_mask(B, P, lens)
        wl["lengths"] = wl["mask"].sum(axis=1)
        _nan_pads(wl)
        gpu = run_gpu(ex4, to_device(wl))
        q = [0, 1] if B == 2 else [0, int(np.argmin(wl["lengths"]))]
        compare(gpu, run_oracle(ex4, wl, q), q, wl["noise"], f"P={P} batch {B} valid {[int(x) for x in wl['lengths'][q]]}")


def test_edge_full_overwrite_and_four_steps():
    _say("edge cases: d = 50, 4 Euler steps")
    ex = Expert(4, n_steps=4, max_batch=4, max_prefix=256)
    try:
        wl = synth.make_workload("expert4_b1_p177", batch=2, with_weights=False)
        wl["prev_actions"] = synth.draw_prev_actions(2, 50)
        gpu = run_gpu(ex, to_device(wl), d=50)
        compare(gpu, run_oracle(ex, wl, [0, 1], d=50), [0, 1], wl["noise"], "d=50 n=4", d=50)
    finally:
        ex.close()


def test_batch1_boundary_with_time_mlp_overwrite_four_steps():
    """Batch 1: the step-boundary launch runs action_out, the Euler update, the overwrite and both
    layers of the next step's time MLP (its hidden layer kept in LDS); with 7 overwritten rows
    and 4 Euler steps, against the oracle per step."""
    _say("batch 1, step boundary with both time-MLP layers: d = 7, 4 Euler steps")
    ex = Expert(4, n_steps=4, max_batch=1, max_prefix=256)
    try:
        wl = synth.make_workload("expert4_b1_p177", batch=1, with_weights=False)
        wl["prev_actions"] = synth.draw_prev_actions(1, 7)
        gpu = run_gpu(ex, to_device(wl), d=7)
        compare(gpu, run_oracle(ex, wl, [0], d=7), [0], wl["noise"], "b1 d=7 n=4", d=7)
    finally:
        ex.close()


def test_step_counts_one_three_and_sixty_four():
    """Step counts at the ends of the accepted range and an odd one, 7 overwritten rows: one step
    (no step-boundary launch at all: the first step's time MLP, then the last step's action_out),
    three (the state moves between its two buffers twice and the last step reads the first buffer
    again) and 64, the largest; batch 1 (the boundary launch runs both time-MLP layers) and, for
    1 and 3 steps, batch 3 (the first layer only); against the oracle per step."""
    for n in (1, 3, 64):
        ex = Expert(4, n_steps=n, max_batch=4, max_prefix=256)
        try:
            for B in ((1, 3) if n < 64 else (1,)):
                _say(f"step count n = {n}, batch {B}, d = 7")
                wl = synth.make_workload("expert4_b1_p177", batch=B, with_weights=False)
                wl["prev_actions"] = synth.draw_prev_actions(B, 7)
                gpu = run_gpu(ex, to_device(wl), d=7)
                assert gpu["vel"].shape[0] == n
                q = list(range(B))
                compare(gpu, run_oracle(ex, wl, q, d=7), q, wl["noise"], f"b{B} d=7 n={n}", d=7)
        finally:
            ex.close()


def test_gain_variant_parity():
    _say("RMSNorm gains 1 + N(0, 0.1)")
    ex = Expert(4, max_batch=4, max_prefix=256, gain_seed=synth.gen.SEED_GAINS)
    try:
        wl = synth.make_workload("expert4_b1_p177", batch=2, with_weights=False)
        compare(run_gpu(ex, to_device(wl)), run_oracle(ex, wl, [0, 1]), [0, 1], wl["noise"], "gain variant")
    finally:
        ex.close()


def test_graph_replay_matches_direct_launches(ex4):
    _say("graph replay vs direct launches")
    direct = Expert(4, max_batch=16, max_prefix=512, use_graphs=0, with_oracle=False)
    try:
        wl = synth.make_workload("expert4_b1_p177", batch=2, with_weights=False)
        dev = to_device(wl)
        ref = run_gpu(direct, dev)
        for _ in range(3):
            got = run_gpu(ex4, dev)
            junk = torch.randn(1 << 20, device="cuda")
            (junk * 2).sum().item()          # eager work between replays
            for k in ref:
                np.testing.assert_array_equal(got[k], ref[k])
    finally:
        direct.close()


def test_time_kernel_hook(ex4):
    _say("time_kernel hook")
    wl = synth.make_workload("expert4_b1_p177", with_weights=False)
    run_gpu(ex4, to_device(wl))
    for k in (0, 1, 2, 3, 4, 5, 6, 7, 9, 10):
        us = fm.smolexp_time_kernel(ex4.h, k, 3)
        assert 0.0 < us < 1e6
    # batch 1: the cross layers' Q projection runs inside the attention launch
    us = ctypes.c_float()
    assert fm.raw().smolexp_time_kernel(ex4.h, fm.K_Q_CROSS, 3, None, ctypes.byref(us)) == fm.SMOLEXP_E_STATE
    assert fm.raw().smolexp_time_kernel(ex4.h, 11, 3, None, ctypes.byref(us)) == fm.SMOLEXP_E_INVAL


def test_query_groups_run_both_kernel_paths_in_one_call():
    """A batch of 20 split into concurrent groups of 16 and 4 queries (batch_groups = 2): the
    first group takes the larger-batch kernels (streamed attention, cross-layer Q projection as
    its own launch), the second the small-batch ones (Q folded into cross attention), in one
    call, with ragged prefixes and a 5-row prefix overwrite; queries from both groups against
    the oracle, a teacher-forced velocity of a second-group query, and bitwise repeatability."""
    _say("4 layers, batch 20 as query groups of 16 and 4")
    ex = Expert(4, max_batch=20, max_prefix=160)
    try:
        cfg = fm.smolexp_default_config(n_layers=4, max_batch=20, max_prefix=160, batch_groups=2)
        assert fm.smolexp_batch_groups(cfg, 20) == [16, 4]
        h = fm.smolexp_create(cfg, 0)
        try:
            fm.smolexp_load_weights(h, synth.pack_weights(ex.named, 4))
            ex2 = object.__new__(Expert)
            ex2.cfg, ex2.h, ex2.W, ex2.ocfg, ex2.named = cfg, h, ex.W, ex.ocfg, ex.named
            B, P, d = 20, 160, 5
            wl = synth.make_workload("expert4_b1_p177", batch=B, with_weights=False)
            wl["prefix_len"] = P
            wl["prefix_kv"] = synth.draw_prefix_kv(4, B, P, seed=61)
            lengths = [160, 7, 99, 160, 1, 150, 33, 80, 120, 64, 65, 128, 129, 2, 159, 100, 160, 17, 140, 88]
            wl["lengths"] = np.array(lengths)
            wl["mask"] = synth.make_mask(B, P, lengths)
            wl["prev_actions"] = synth.draw_prev_actions(B, d)
            dev = to_device(wl)
            gpu = run_gpu(ex2, dev, d=d)
            q = [0, 4, 15, 16, 17, 19]
            compare(gpu, run_oracle(ex2, wl, q, d=d), q, wl["noise"], "query groups 16 + 4", d=d)
            again = run_gpu(ex2, dev, d=d)
            np.testing.assert_array_equal(again["out"], gpu["out"])
            # one velocity evaluation at t = 0.6 of every query, checked on a second-group query
            x = torch.from_numpy(gpu["st"][3]).cuda()
            v = torch.empty_like(x)
            fm.smolexp_velocity(h, cfg, dev["kv"], dev["mask"], x, 0.6, v)
            torch.cuda.synchronize()
            b = 17
            want = oracle.velocity(ex.W, ex.ocfg, gpu["st"][3][b].astype(np.float64), np.float32(0.6),
                                   oracle.bf16_bits_to_float(wl["prefix_kv"][:, 0, b]),
                                   oracle.bf16_bits_to_float(wl["prefix_kv"][:, 1, b]), wl["mask"][b].astype(bool))
            rel = np.linalg.norm(v.cpu().numpy()[b] - want) / np.linalg.norm(want)
            print(f"[parity] query groups: velocity of query {b} at t = 0.6: rel {rel:.3e}", flush=True)
            assert rel <= VEL_RTOL
        finally:
            fm.smolexp_destroy(h)
    finally:
        ex.close()


def test_fp16_range_overflow_is_reported():
    """Activations beyond fp16's range (the matrix cores' operand type, largest finite value
    65504) are reported in the call's status word with the documented bits, not returned as
    silent infinities: a time_out bias of 1e5 (the residual stream), gate/up weights scaled by
    300 (the SwiGLU output), prefix values of 1e6 (the attention output) and noise of 1e5 (the
    Euler state).  The oracle (float64) stays finite on the first case; the weights of the
    workloads report 0."""
    _say("fp16 range reporting")
    L, P = 2, 40
    base = synth.draw_weights(L)
    kv = synth.draw_prefix_kv(L, 1, P, seed=71)
    mask = synth.make_mask(1, P, [33])
    noise = synth.draw_noise(1, seed=72)

    def bits(a):
        return synth.f32_to_bf16_bits(np.asarray(a, np.float32))

    def run(named, kv_bits, noise_np):
        cfg = fm.smolexp_default_config(n_layers=L, max_batch=1, max_prefix=P)
        h = fm.smolexp_create(cfg, 0)
        try:
            fm.smolexp_load_weights(h, synth.pack_weights(named, L))
            out = torch.empty((1, 50, 32), device="cuda")
            st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            fm.smolexp_denoise_ex(h, cfg, torch.from_numpy(kv_bits.view(np.int16)).cuda(), torch.from_numpy(mask).cuda(),
                                  torch.from_numpy(noise_np).cuda(), out, out_status=st)
            torch.cuda.synchronize()
            return int(st.cpu()[0]), out.cpu().numpy()
        finally:
            fm.smolexp_destroy(h)

    status, out = run(base, kv, noise)
    assert status == 0 and np.isfinite(out).all()

    big_b = dict(base)
    big_b["time_out.b"] = bits(np.full(720, 1e5))
    status, _ = run(big_b, kv, noise)
    print(f"[range] time_out.b = 1e5: status {status}", flush=True)
    assert status & fm.SMOLEXP_RANGE_RESIDUAL
    W = oracle.decode_weights(big_b)
    x = oracle.denoise_batch(W, oracle.ExpertConfig(n_layers=L), kv, mask, noise, n_steps=10)
    assert np.isfinite(x).all()   # representable in the method's own arithmetic

    big_ffn = dict(base)
    for name in ("layers.0.gate.w", "layers.0.up.w"):
        big_ffn[name] = bits(oracle.bf16_bits_to_float(base[name]) * 300.0)
    status, _ = run(big_ffn, kv, noise)
    print(f"[range] gate/up x 300: status {status}", flush=True)
    assert status & fm.SMOLEXP_RANGE_FFN

    kv_big = kv.copy()
    kv_big[1, 1] = bits(np.full(kv_big[1, 1].shape, 1e6))   # layer 1 (cross) values
    status, _ = run(base, kv_big, noise)
    print(f"[range] prefix values 1e6: status {status}", flush=True)
    assert status & fm.SMOLEXP_RANGE_ATTENTION

    status, _ = run(base, kv, noise * np.float32(1e5))
    print(f"[range] noise x 1e5: status {status}", flush=True)
    assert status & fm.SMOLEXP_RANGE_TIME

#!/usr/bin/env python3
"""Benchmark of the SmolVLA action-expert denoising loop on one MI355X.

One "step" is one smolexp_denoise call: the whole Euler loop (10 steps, or
--n-steps) of the 16-layer expert over one batch of synthetic inputs already
resident in HBM.
Prints one JSON line: chunks/s, ms per call, the roofline of the dominant
kernel (timed live with HIP events on the library's stream), the whole-loop
roofline, and the CPU oracle timed on the host as a baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--n-steps N]
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_F16_PEAK_TFS = 2500.0   # MI355X dense fp16/bf16 MFMA, published
RIDGE = MFMA_F16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)

DEFAULT_WORKLOAD = "expert16_b1_p177"
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 256 << 20   # calibration copy: 256 MiB read + 256 MiB written
KERNEL_SYMBOLS = {       # kernel name fragments in a rocprofv3 trace, per timed kernel
    "qkv_self": "gemm_skinny<1, 4,", "attn_self": "attn_small_kernel<true,", "attn_cross": "attn_cross_q_kernel<",
    "o": "gemm_skinny<0, 3, 4,", "gate_up": "gemm_skinny<1, 5,", "down": "gemm_skinny<0, 3, 8,",
    "action_out": "gemm_skinny<1, 6,", "time_in": "gemm_skinny<2, 1,", "time_out": "gemm_skinny<0, 2,",
}


class GpuStateSampler:
    """Shader clock (the current level of pp_dpm_sclk) and board power (hwmon power1_input)
    read from sysfs by a background thread every few milliseconds while the timed calls run;
    None where the files are not readable."""

    def __init__(self, period=0.005):
        import glob
        import threading
        self.period = period
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.sclk = cards[0] if cards else None
        dev = os.path.dirname(cards[0]) if cards else None
        pw = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input"))) if dev else []
        self.power = pw[0] if pw else None
        self.mhz, self.watts = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            if self.sclk:
                for line in open(self.sclk):
                    if line.rstrip().endswith("*"):
                        self.mhz.append(float(line.split(":")[1].strip().split("Mhz")[0]))
            if self.power:
                self.watts.append(float(open(self.power).read()) / 1e6)
        except (OSError, ValueError, IndexError):
            pass

    def _run(self):
        while not self._stop.is_set():
            self._read()
            self._stop.wait(self.period)

    def start(self):
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        self._thread.join()
        stat = lambda v: {"mean": sum(v) / len(v), "min": min(v), "max": max(v)} if v else None
        return {"sclk_mhz": stat(self.mhz), "board_power_w": stat(self.watts), "samples": len(self.mhz)}


def kernel_source_digest():
    """Digest of the HIP sources: a stored counter reading is only valid for the kernels it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in ("kernels.hip", "smolexp_internal.h"):
        with open(os.path.join(ROOT, "flow_matching_action_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel):
    """HBM bytes per launch from profiles/traffic.json, or None if absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            e = json.load(f)[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if e.get("kernel_source") != kernel_source_digest():
        return None
    return e.get("hbm_bytes_per_launch")


def summarize_pmc(fetch_csv, write_csv, workload, kernel):
    """Per-launch HBM bytes of `kernel` from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by what the same counter reads for the calibration copy of COPY_BYTES."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    out = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        vals = per_kernel(path, counter)
        # the runtime may split one copy into several dispatches: calibrate on the total of the
        # three copies (3 * COPY_BYTES read and written)
        copy = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs]
        mine = [v for k, vs in vals.items() if KERNEL_SYMBOLS[kernel] in k for v in vs]
        if not copy or not mine:
            raise SystemExit(f"{path}: no calibration copy or no {kernel} dispatch with {counter}")
        copy_kib = sum(copy)
        scale = (3 * COPY_BYTES / 1024) / copy_kib
        out[counter] = {"kib_per_launch": sum(mine) / len(mine), "launches": len(mine),
                        "copy_kib_total": copy_kib, "copy_dispatches": len(copy), "scale": scale,
                        "bytes_per_launch": sum(mine) / len(mine) * 1024 * scale}
    entry = {"kernel_source": kernel_source_digest(), "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"],
             "hbm_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]}
    try:
        with open(TRAFFIC_FILE) as f:
            allv = json.load(f)
    except (OSError, ValueError):
        allv = {}
    allv.setdefault(workload, {})[kernel] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allv, f, indent=1, sort_keys=True)
    print(json.dumps(entry, indent=1))


def kernel_costs(L, B, lengths, P):
    """Algorithmic (bytes, flops) of ONE launch of each timed kernel, and launches per call per step.

    Bytes count each operand once: fp16 weights (2 B/element, without the K
    padding), the activation the kernel reads (the normed projections read the
    fp16 copy of the residual), the activations it writes (o and down
    read-modify-write the fp32 residual and write its fp16 copy), valid prefix
    K/V tokens only.  Flops are 2 per multiply-add; attention counts unmasked
    keys only.
    """
    M = 50 * B
    sum_nb = float(sum(lengths))
    c = {}
    c["qkv_self"] = (1600 * 720 * 2 + M * 720 * 2 + M * 1600 * 2, 2.0 * M * 1600 * 720)
    kv_self = 5 * 64 * 2 * 2 * (sum_nb + 50 * B)
    keys_self = 50 * sum_nb + 1275 * B
    c["attn_self"] = (M * 960 * 2 + kv_self + M * 960 * 2, 4.0 * 64 * 15 * keys_self)
    kv_cross = 5 * 64 * 2 * 2 * sum_nb
    if B <= CROSS_Q_MAX_BATCH:  # the cross layers' Q projection runs inside the attention launch
        c["attn_cross"] = (960 * 720 * 2 + M * 720 * 2 + kv_cross + M * 960 * 2,
                           2.0 * M * 960 * 720 + 4.0 * 64 * 15 * 50 * sum_nb)
    else:
        c["attn_cross"] = (M * 960 * 2 + kv_cross + M * 960 * 2, 4.0 * 64 * 15 * 50 * sum_nb)
    c["o"] = (720 * 960 * 2 + M * 960 * 2 + M * 720 * 10, 2.0 * M * 720 * 960)
    c["gate_up"] = (4096 * 720 * 2 + M * 720 * 2 + M * 2048 * 2, 2.0 * M * 4096 * 720)
    c["down"] = (720 * 2048 * 2 + M * 2048 * 2 + M * 720 * 10, 2.0 * M * 720 * 2048)
    c["action_out"] = (32 * 720 * 2 + M * 720 * 2 + M * 32 * 8, 2.0 * M * 32 * 720)
    # the time MLP's first layer as the kernel computes it: action_in folded into its action half
    # (a [720, 32] weight), the Euler state in, the step's time vector, fp16 activations out
    c["time_in"] = (720 * 32 * 2 + M * 32 * 4 + 720 * 4 + M * 720 * 2, 2.0 * M * 720 * 32)
    c["time_out"] = (720 * 720 * 2 + M * 720 * 2 + M * 720 * 6, 2.0 * M * 720 * 720)
    per_step = {"qkv_self": L // 2 + L % 2, "attn_self": L // 2 + L % 2, "attn_cross": L // 2, "o": L,
                "gate_up": L, "down": L, "action_out": 1, "time_in": 1, "time_out": 1}
    if B > CROSS_Q_MAX_BATCH:  # the cross layers' Q projection is a launch of its own
        c["q_cross"] = (960 * 720 * 2 + M * 720 * 2 + M * 960 * 2, 2.0 * M * 960 * 720)
        per_step["q_cross"] = L // 2
    return c, per_step


CROSS_Q_MAX_BATCH = 8  # largest batch whose cross layers fold the Q projection into attention (library constant)
KERNEL_IDS = {"qkv_self": 0, "attn_self": 1, "attn_cross": 2, "o": 3, "gate_up": 4, "down": 5, "action_out": 6,
              "q_cross": 8, "time_in": 9, "time_out": 10}
LOOP_ID = 7  # smolexp_time_kernel: the whole call


def loop_algorithmic(L, B, lengths, n_steps):
    """Whole-loop algorithmic bytes and flops per call: weights once per step (bf16,
    2 B/element), valid prefix K/V once per step, 2 flops per weight MAC per chunk row,
    attention over unmasked keys."""
    import synth
    wbytes = 2 * synth.weight_count(L)
    sum_nb = float(sum(lengths))
    kvbytes = L * 2 * 5 * 64 * 2 * sum_nb
    macs_per_row = sum(int(__import__("numpy").prod(s)) for n, s, k in synth.manifest(L) if k == "w")
    n_self, n_cross = (L + 1) // 2, L // 2
    att = 4.0 * 64 * 15 * (n_self * (50 * sum_nb + 1275 * B) + n_cross * 50 * sum_nb)
    flops = 2.0 * macs_per_row * 50 * B + att
    return n_steps * (wbytes + kvbytes), n_steps * flops


def cpu_baseline(wl, n_steps, min_seconds, max_seconds):
    """The float64 numpy oracle on the host, on whole chunks of the workload's first queries."""
    import numpy as np
    import threadpoolctl
    import oracle
    W = oracle.decode_weights(wl["weights"])
    cfg = oracle.ExpertConfig(n_layers=wl["n_layers"])
    B = wl["batch"]
    done, t0 = 0, time.perf_counter()
    while True:
        b = done % B
        oracle.denoise_batch(W, cfg, wl["prefix_kv"], wl["mask"], wl["noise"], n_steps=n_steps,
                             prev=wl["prev_actions"], d=wl["overwrite_rows"], queries=[b])
        done += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el + el / done > max_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return {"value": done / el, "unit": "chunks/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} whole {n_steps}-step chunk(s) of the first {min(done, B)} quer(ies), {el:.1f} s, "
                      f"float64 numpy, {threads} BLAS thread(s), host {os.cpu_count()} logical CPUs"}


def prefill_algorithmic(L, B, lengths, P):
    """Bytes and flops of one prefill call, counted on the valid tokens: the language model's
    weights once (bf16; the last layer needs only its K and V projections), embeddings read and
    the K/V cache written (2 bytes each); projections 2 flops per multiply-add per token,
    attention over valid keys for valid queries."""
    n = [int(x) for x in lengths]
    tok = float(sum(n))
    macs_layer = 1600 * 960 + 960 * 960 + 5120 * 960 + 960 * 2560
    macs_last = 640 * 960
    wbytes = 2 * ((L - 1) * macs_layer + macs_last + L * 2 * 960)
    io = 2 * tok * 960 + L * 2 * 5 * 64 * 2 * tok
    flops = 2.0 * tok * ((L - 1) * macs_layer + macs_last) + 4.0 * 64 * 15 * (L - 1) * sum(x * x for x in n)
    return wbytes + io, flops


def run_prefill_stage(args):
    """Time smolexp_prefill on the workload's batch and prefix (one JSON line)."""
    import numpy as np
    import torch
    import synth
    import flow_matching_action_step_amd as fm

    wl = synth.make_workload(args.workload, with_weights=False)
    L, B, P = wl["n_layers"], wl["batch"], wl["prefix_len"]
    cfg = fm.smolexp_default_config(n_layers=L, max_batch=B, max_prefix=P)
    h = fm.smolexp_create(cfg, 0)
    named = synth.draw_lm_weights(L)
    fm.smolexp_load_lm_weights(h, synth.pack_lm_weights(named, L))
    emb_bits = synth.draw_prefix_embeddings(B, P)
    emb = torch.from_numpy(emb_bits.view(np.int16)).cuda()
    mask = torch.from_numpy(wl["mask"]).cuda()
    out = torch.empty((L, 2, B, 5, P, 64), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        fm.smolexp_prefill(h, cfg, emb, mask, out)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sampler = GpuStateSampler().start()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_state = sampler.stop()
    ev_ms = e0.elapsed_time(e1) / args.steps
    ms = wall / args.steps * 1e3
    byt, fl = prefill_algorithmic(L, B, wl["lengths"], P)
    intensity = fl / byt
    if intensity < RIDGE:
        roof = {"bound": "hbm", "achieved": byt / (ev_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": fl / (ev_ms * 1e-3) / 1e12, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "whole prefill call (HIP events around the calls)"
    roof["algorithmic_bytes_per_call"] = byt
    roof["algorithmic_flops_per_call"] = fl
    line = {
        "metric": "prefix prefills/sec (language model, K/V cache of every layer)",
        "value": B * args.steps / wall, "unit": "prefills/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16",
        "precision": "GEMM operands fp16 (bf16 weights re-encoded exactly; RMSNorm gains folded), attention bf16, "
                     "fp32 accumulate and residual, K/V cache bf16",
        "data": "synthetic (seeded: weights N(0,0.02) bf16, embeddings N(0,1) bf16)",
        "config": {"workload": args.workload, "stage": "prefill", "n_layers": L, "batch": B, "prefix_len": P,
                   "width": 960, "ffn": 2560},
        "roofline": roof,
        "event_ms_per_call": ev_ms,
        "gpu_state": gpu_state,
    }
    fm.smolexp_destroy(h)
    if not args.no_cpu_baseline:
        import threadpoolctl
        import oracle
        W = oracle.decode_weights(named)
        ocfg = oracle.PrefillConfig(n_layers=L)
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.prefill_batch(W, ocfg, emb_bits, wl["mask"], queries=[done % B])
            done += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el + el / done > 3 * args.cpu_seconds:
                break
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
        line["cpu_baseline"] = {"value": done / el, "unit": "prefills/s", "cores": threads, "kind": "oracle",
                                "sample": f"{done} whole prefill(s) of the first {min(done, B)} quer(ies), "
                                          f"{el:.1f} s, float64 numpy, {threads} BLAS thread(s)"}
    print(json.dumps(line), flush=True)


def train_algorithmic(L, B, lengths):
    """Matrix-core flops of one training step (forward, input gradients, weight gradients)
    and its minimum HBM bytes.

    Projections: 2 flops per multiply-add per chunk row; the backward pass computes every
    weight gradient (the forward's flops again) and every input gradient except those of the
    data (x_t) and of the time embedding (half of time_in).  Attention, per row, head and
    allowed key: forward QK^T and PV (4 x 64), backward dP, dS K, dS^T Q and P^T dO (8 x 64);
    allowed keys are the n_b valid prefix tokens plus, in self layers, chunk keys j <= i.
    Bytes: the bf16 weights read three times (forward, input and weight gradients), the fp32
    gradients written once, the valid prefix K/V read twice (forward, backward).
    """
    D, F, A, C = 720, 2048, 32, 50
    per_row = 2 * (A * D + 2 * D * D + D * D + A * D)  # action_in, time_in, time_out, action_out
    for l in range(L):
        nq = 1600 if l % 2 == 0 else 960
        per_row += 2 * (D * nq + 960 * D + D * 2 * F + F * D)
    dx_skip = 2 * (A * D + D * D)
    gemm = B * C * (3 * per_row - dx_skip)
    n_self, n_cross = (L + 1) // 2, L // 2
    attn = 0
    for nb in lengths:
        keys_self = C * nb + C * (C + 1) // 2
        keys_cross = C * nb
        attn += 15 * (n_self * keys_self + n_cross * keys_cross) * 12 * 64
    n_w = 0
    for l in range(L):
        nq = 1600 if l % 2 == 0 else 960
        n_w += 2 * D + nq * D + D * 960 + 3 * F * D
    n_w += A * D + D + 2 * D * D + D + D * D + D + D + A * D + A
    byt = 3 * 2 * n_w + 4 * n_w + 2 * L * sum(lengths) * 5 * 64 * 2 * 2
    return byt, gemm + attn


def run_train_stage(args):
    """Time smolexp_train_step on the workload's batch and prefix (one JSON line)."""
    import numpy as np
    import torch
    import synth
    import flow_matching_action_step_amd as fm

    wl = synth.make_workload(args.workload)
    L, B, P = wl["n_layers"], wl["batch"], wl["prefix_len"]
    cfg = fm.smolexp_default_config(n_layers=L, max_batch=B, max_prefix=P)
    h = fm.smolexp_create(cfg, 0)
    fm.smolexp_load_weights(h, synth.pack_weights(wl["weights"], L))
    kv = torch.from_numpy(np.ascontiguousarray(wl["prefix_kv"]).view(np.int16)).cuda()
    mask = torch.from_numpy(wl["mask"]).cuda()
    acts_np, t_np = synth.draw_actions(B), synth.draw_flow_times(B)
    acts = torch.from_numpy(acts_np).cuda()
    noise = torch.from_numpy(wl["noise"]).cuda()
    t = torch.from_numpy(t_np).cuda()
    grads = torch.empty(fm.smolexp_weight_count(cfg), dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        fm.smolexp_train_step(h, cfg, kv, mask, acts, noise, t, grads, loss)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sampler = GpuStateSampler().start()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_state = sampler.stop()
    ev_ms = e0.elapsed_time(e1) / args.steps
    ms = wall / args.steps * 1e3
    lengths = [int(x) for x in wl["mask"].sum(axis=1)]
    byt, fl = train_algorithmic(L, B, lengths)
    roof = {"bound": "mfma", "achieved": fl / (ev_ms * 1e-3) / 1e12, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "whole training step (HIP events around the calls)"
    roof["algorithmic_flops_per_call"] = fl
    roof["algorithmic_bytes_per_call"] = byt
    line = {
        "metric": "training samples/sec (flow-matching loss and every expert weight gradient)",
        "value": B * args.steps / wall, "unit": "samples/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "precision": "GEMM and attention operands bf16, fp32 accumulate; softmax, norms, loss and residual fp32",
        "data": "synthetic (seeded: weights N(0,0.02) bf16, K/V N(0,1) bf16, actions and noise N(0,1), t U(0,1))",
        "config": {"workload": args.workload, "stage": "train", "n_layers": L, "batch": B, "prefix_len": P},
        "roofline": roof,
        "event_ms_per_call": ev_ms,
        "loss": float(loss.cpu()[0]),
        "gpu_state": gpu_state,
    }
    fm.smolexp_destroy(h)
    if not args.no_cpu_baseline:
        import threadpoolctl
        import oracle
        W = oracle.decode_weights(wl["weights"])
        ocfg = oracle.ExpertConfig(n_layers=L)
        a64, e64, t64 = acts_np.astype(np.float64), wl["noise"].astype(np.float64), t_np.astype(np.float64)
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.train_batch(W, ocfg, wl["prefix_kv"], wl["mask"], a64, e64, t64, queries=[done % B])
            done += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el + el / done > 3 * args.cpu_seconds:
                break
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
        line["cpu_baseline"] = {"value": done / el, "unit": "samples/s", "cores": threads, "kind": "oracle",
                                "sample": f"{done} sample(s) (forward and backward of one query each), "
                                          f"{el:.1f} s, float64 numpy, {threads} BLAS thread(s)"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--n-steps", type=int, default=10, help="Euler steps per chunk (dt = -1/n)")
    ap.add_argument("--stage", choices=("denoise", "prefill", "train"), default="denoise",
                    help="prefill: time the prefix language model that fills the K/V cache instead; "
                         "train: the flow-matching training step (loss and weight gradients)")
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graphs", action="store_true", help="launch kernels one by one instead of graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurement, copy 256 MiB device-to-device three times (HBM counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv files")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.summarize_pmc[2])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the denoising loop runs on a single MI355X and shards by query "
              f"(data parallel, no exchange); --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    if args.stage == "prefill":
        run_prefill_stage(args)
        return
    if args.stage == "train":
        run_train_stage(args)
        return

    import numpy as np
    import torch
    import synth
    import flow_matching_action_step_amd as fm

    wl = synth.make_workload(args.workload)
    L, B, P, d = wl["n_layers"], wl["batch"], wl["prefix_len"], wl["overwrite_rows"]
    cfg = fm.smolexp_default_config(n_layers=L, n_steps=args.n_steps, max_batch=B, max_prefix=P,
                                    use_graphs=0 if args.no_graphs else 1)
    h = fm.smolexp_create(cfg, 0)
    fm.smolexp_load_weights(h, synth.pack_weights(wl["weights"], L))
    kv = torch.from_numpy(np.ascontiguousarray(wl["prefix_kv"]).view(np.int16)).cuda()
    mask = torch.from_numpy(wl["mask"]).cuda()
    noise = torch.from_numpy(wl["noise"]).cuda()
    prev = torch.from_numpy(wl["prev_actions"]).cuda() if d > 0 else None
    out = torch.empty((B, 50, 32), device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        fm.smolexp_denoise_ex(h, cfg, kv, mask, noise, out, prev_actions=prev, overwrite_rows=d)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sampler = GpuStateSampler().start()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_state = sampler.stop()
    ev_ms = e0.elapsed_time(e1)
    assert torch.isfinite(out).all().item(), "non-finite actions"

    # per-kernel average launch duration, HIP events on the library's stream
    costs, per_step = kernel_costs(L, B, wl["lengths"], P)
    kern = {}
    for name, kid in KERNEL_IDS.items():
        if name not in per_step:  # not launched at this batch (folded into another kernel)
            continue
        us = fm.smolexp_time_kernel(h, kid, args.kernel_reps)
        byt, fl = costs[name]
        kern[name] = {"avg_us": us, "launches_per_call": per_step[name] * cfg.n_steps,
                      "us_per_call": us * per_step[name] * cfg.n_steps, "bytes": byt, "flops": fl}
    loop_us = fm.smolexp_time_kernel(h, LOOP_ID, max(3, args.steps // 5))
    dom_name = max(kern, key=lambda k: kern[k]["us_per_call"])
    dom = kern[dom_name]
    intensity = dom["flops"] / dom["bytes"]
    if intensity < RIDGE:
        achieved = dom["bytes"] / (dom["avg_us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        achieved = dom["flops"] / (dom["avg_us"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(args.workload, dom_name)
    roof["kernel"] = dom_name
    roof["avg_us"] = dom["avg_us"]
    roof["algorithmic_bytes_per_launch"] = dom["bytes"]
    roof["algorithmic_flops_per_launch"] = dom["flops"]

    ms = wall / args.steps * 1e3
    lb, lf = loop_algorithmic(L, B, wl["lengths"], cfg.n_steps)
    loop = {"algorithmic_bytes_per_call": lb, "algorithmic_flops_per_call": lf,
            "hbm_frac": lb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "mfma_frac": lf / (ms * 1e-3) / (MFMA_F16_PEAK_TFS * 1e12),
            "event_ms_per_call": ev_ms / args.steps, "replay_us_per_call": loop_us}

    line = {
        "metric": f"action chunks/sec (50x32, {cfg.n_steps} Euler steps) + ms/chunk at B=1; % HBM/MFMA roofline",
        "value": B * args.steps / wall,
        "unit": "chunks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "precision": "GEMM operands fp16 (bf16 weights re-encoded exactly; RMSNorm gains folded into the "
                     "following weights, rounded once), attention bf16, fp32 accumulate, fp32 residual/norm "
                     "scale/softmax/Euler",
        "data": "synthetic (seeded: weights N(0,0.02) bf16, prefix K/V N(0,1) bf16, noise N(0,1))",
        "config": {"workload": args.workload, "n_layers": L, "batch": B, "prefix_len": P,
                   "n_steps": cfg.n_steps, "chunk": 50, "action_dim": 32, "overwrite_rows": d,
                   "graphs": not args.no_graphs},
        "roofline": roof,
        "loop_roofline": loop,
        "kernels": kern,
        "gpu_state": gpu_state,
    }
    fm.smolexp_destroy(h)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, cfg.n_steps, args.cpu_seconds, 3 * args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

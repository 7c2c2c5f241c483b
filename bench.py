#!/usr/bin/env python3
"""Benchmark of the SmolVLA action-expert denoising loop on one MI355X.

One "step" is one smolexp_denoise call: the whole Euler loop (10 steps, or
--n-steps) of the 16-layer expert over one batch of synthetic inputs already
resident in HBM.
Prints one JSON line: chunks/s and ms per call at batch 1 (the 16-layer expert,
prefix 177), the roofline of the dominant kernel (its time per launch taken live
with HIP events on the library's stream, its bytes counted algorithmically:
parameters once, valid prefix K/V tokens), the whole-loop roofline, the
prefix-overwrite difference, the large-batch workloads (batch 64 at prefix 257;
batch 128 at prefix 177 with 7 overwritten rows: ms per call, chunks/s, MFMA
fraction of the loop and of its dominant kernel), and the CPU oracle timed on the
host as a baseline (all threads, and one).

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
LARGE_BATCH_WORKLOADS = ("expert16_b64_p257", "expert16_b128_p177_ow7", "expert16_b16_pvar241")
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 256 << 20   # calibration copy: 256 MiB read + 256 MiB written
KERNEL_SYMBOLS = {       # kernel name fragments in a rocprofv3 trace, per timed kernel
    "qkv_self": "gemm_skinny<1, 4,", "attn_self": "attn_small_kernel<true,", "attn_cross": "attn_cross_q_kernel<",
    "o": "gemm_skinny<0, 3, 4,", "gate_up": "gemm_skinny<1, 5,", "down": "gemm_skinny<0, 3, 8,",
    "action_out": "step_boundary_kernel<", "time_in": "gemm_skinny<2, 1,", "time_out": "gemm_skinny<0, 2,",
    # the pipelined 128 x 128 gate/up of the large batches (traffic counters only)
    "gate_up_big": "gemm_big<5, true, 128,",
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


def summarize_trace(trace_csv):
    """Per kernel, from the rocprofv3 --kernel-trace of one bench command: the dispatches of the
    whole calls (warm-up, timed calls and the hook's whole-call replays: everything up to the
    end of the last call, which starts with its prologue_kernel) and those of the per-kernel
    timing graphs that follow them (bench.py's avg_us times those with HIP events).  Prints a
    markdown table of calls and average durations."""
    import csv
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    mine = [r for r in rows if "smolexp::" in r[2]]
    pro = [i for i, r in enumerate(mine) if "prologue_kernel" in r[2]]
    per_call = pro[-1] - pro[-2]                 # dispatches of one call
    end_loop = pro[-1] + per_call                 # first dispatch after the last call
    stats = {}
    for i, (t0, t1, name) in enumerate(mine):
        e = stats.setdefault(name, [0, 0.0, 0, 0.0])
        k = 0 if i < end_loop else 2
        e[k] += 1
        e[k + 1] += (t1 - t0) / 1e3
    loop_total = sum(e[1] for e in stats.values())
    short = lambda n: n.replace("void ", "").replace("smolexp::", "").split("(")[0]  # noqa: E731
    fmt = lambda t, c: f"{t / c:.2f}" if c else "-"  # noqa: E731
    print(f"{per_call} dispatches per call; {end_loop} dispatches of whole calls, {len(mine) - end_loop} of timing graphs")
    print()
    print("| kernel | calls in whole calls | avg us | % of their GPU time | calls in timing graphs | avg us |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, e in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        print(f"| `{short(name)}` | {e[0]} | {fmt(e[1], e[0])} | {100 * e[1] / loop_total:.1f} | {e[2]} | {fmt(e[3], e[2])} |")


def summarize_mfma(counter_csv):
    """Per kernel, from one rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE,
    SQ_INSTS_VALU_MFMA_MOPS_F16 and SQ_INSTS_VALU_MFMA_MOPS_BF16: matrix-core utilisation (busy
    cycles summed over the 1024 SIMDs, over GUI_ACTIVE summed over the 8 XCDs / 8 x 1024) and the
    matrix flops issued per dispatch (MOPS x 512).  Prints a markdown table."""
    import csv
    per = {}
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            d = per.setdefault(key, {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    stats = {}
    for (_, name), d in per.items():
        e = stats.setdefault(name, [0, 0.0, 0.0, 0.0, 0.0])
        e[0] += 1
        e[1] += d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        e[2] += d.get("GRBM_GUI_ACTIVE", 0.0) / 8 * 1024
        e[3] += (d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)) * 512
        e[4] += d["dur"]
    total = sum(e[4] for n, e in stats.items() if "smolexp::" in n)
    short = lambda n: n.replace("void ", "").replace("smolexp::", "").split("(")[0]  # noqa: E731
    print("| kernel | dispatches | MFMA utilisation | MFMA TFLOP per dispatch | % of GPU time |")
    print("|---|---:|---:|---:|---:|")
    for name, e in sorted(stats.items(), key=lambda kv: -kv[1][4]):
        if "smolexp::" not in name:
            continue
        util = e[1] / e[2] if e[2] else 0.0
        print(f"| `{short(name)}` | {e[0]} | {100 * util:.1f}% | {e[3] / e[0] / 1e12:.4f} | {100 * e[4] / total:.1f} |")


def summarize_stalls(pass1_csv, pass2_csv):
    """Per kernel, from two rocprofv3 --pmc runs of the same command: (1) SQ_WAVE_CYCLES,
    SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_ANY; (2) SQ_VALU_MFMA_BUSY_CYCLES,
    GRBM_GUI_ACTIVE, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE.  Fractions of the wave cycles spent
    waiting (waitcnt, barrier), waiting to issue and issuing; matrix-core busy (as in
    summarize_mfma); LDS bank-conflict cycles per LDS-active cycle.  Prints a markdown table."""
    import csv
    tot = {}
    for path in (pass1_csv, pass2_csv):
        with open(path) as f:
            for r in csv.DictReader(f):
                if "smolexp::" not in r["Kernel_Name"]:
                    continue
                e = tot.setdefault(r["Kernel_Name"], {})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    short = lambda n: n.replace("void ", "").replace("smolexp::", "").split("(")[0]  # noqa: E731
    print("| kernel | waiting (waitcnt, barrier) | waiting to issue | issuing | matrix cores busy | LDS bank conflicts |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, e in sorted(tot.items(), key=lambda kv: -kv[1].get("SQ_WAVE_CYCLES", 0.0)):
        wc = e.get("SQ_WAVE_CYCLES", 0.0)
        simd = e.get("GRBM_GUI_ACTIVE", 0.0) / 8 * 1024
        if not wc or not simd:
            continue
        lds = e.get("SQ_LDS_IDX_ACTIVE", 0.0)
        print(f"| `{short(name)}` | {e.get('SQ_WAIT_ANY', 0.0) / wc:.2f} | {e.get('SQ_WAIT_INST_ANY', 0.0) / wc:.2f} | "
              f"{e.get('SQ_ACTIVE_INST_ANY', 0.0) / wc:.2f} | {100 * e.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / simd:.1f}% | "
              f"{e.get('SQ_LDS_BANK_CONFLICT', 0.0) / lds if lds else 0.0:.2f} |")


def kernel_costs(L, B, lengths, P, w8=False):
    """Per launch of each timed kernel: (algorithmic bytes, activation bytes, flops), and its
    launches per Euler step.

    Up to BOUNDARY_MAX_ROWS chunk rows per query group (the library's register-resident K split of
    action_out) the end of one step and the start of the next are one launch:
    "action_out" then stands for that step-boundary launch (action_out + Euler + the next step's
    overwrite and time-MLP first layer; for one query, BOUNDARY_TIME_OUT_MAX_ROWS, the time MLP's
    second layer too) and "time_in" (and "time_out") have no launch per step: only the call's first
    step runs them alone (kernel_table adds those launches once per call).  The last step's action_out
    also runs alone; counting it as a boundary launch keeps the per-step work, and so the loop's
    totals, exact.

    Algorithmic bytes follow the counting of the loop's roofline: the parameters the launch
    reads, once, at 2 bytes per element (the bf16 manifest; RMSNorm gains are folded into the
    matrices that follow them, action_in into a [720, 32] matrix with the action half of
    time_in, and the time-embedding half of time_in into one time vector per step, all when
    the weights are loaded), plus the valid prefix K/V tokens the launch attends to.  With
    8-bit weights (w8) a matrix costs 1 byte per element plus a 4-byte scale per row.
    Activation bytes (the fp16/bf16/fp32 rows each launch reads and writes) are counted apart.
    Flops are 2 per multiply-add; attention counts unmasked keys only.
    """
    def mat(n, k):  # bytes of one streamed [n, k] matrix
        return n * k + 4 * n if w8 else 2 * n * k

    M = 50 * B
    sum_nb = float(sum(lengths))
    kv = 5 * 64 * 2 * 2 * sum_nb            # one layer's valid prefix K and V
    keys_self = 50 * sum_nb + 1275 * B
    c = {}
    c["qkv_self"] = (mat(1600, 720), M * 720 * 2 + M * 1600 * 2, 2.0 * M * 1600 * 720)
    c["attn_self"] = (kv, M * 960 * 2 + M * 640 * 2 + M * 960 * 2, 4.0 * 64 * 15 * keys_self)
    if B <= CROSS_Q_MAX_BATCH:  # the cross layers' Q projection runs inside the attention launch
        c["attn_cross"] = (mat(960, 720) + kv, M * 720 * 2 + M * 960 * 2,
                           2.0 * M * 960 * 720 + 4.0 * 64 * 15 * 50 * sum_nb)
    else:
        c["attn_cross"] = (kv, M * 960 * 2 + M * 960 * 2, 4.0 * 64 * 15 * 50 * sum_nb)
    # o and down read-modify-write the fp32 residual and write its fp16 copy (10 B per element)
    c["o"] = (mat(720, 960), M * 960 * 2 + M * 720 * 10, 2.0 * M * 720 * 960)
    c["gate_up"] = (mat(4096, 720), M * 720 * 2 + M * 2048 * 2, 2.0 * M * 4096 * 720)
    c["down"] = (mat(720, 2048), M * 2048 * 2 + M * 720 * 10, 2.0 * M * 720 * 2048)
    c["action_out"] = (mat(32, 720) + 32 * 2, M * 720 * 2 + M * 32 * 8, 2.0 * M * 32 * 720)
    # the time MLP's first layer: the folded [720, 32] matrix and the step's time vector
    c["time_in"] = (mat(720, 32) + 720 * 2, M * 32 * 4 + M * 720 * 2, 2.0 * M * 720 * 32)
    c["time_out"] = (mat(720, 720) + 720 * 2, M * 720 * 2 + M * 720 * 6, 2.0 * M * 720 * 720)
    per_step = {"qkv_self": L // 2 + L % 2, "attn_self": L // 2 + L % 2, "attn_cross": L // 2, "o": L,
                "gate_up": L, "down": L, "action_out": 1, "time_in": 1, "time_out": 1}
    if M <= BOUNDARY_MAX_ROWS:  # the step boundary: action_out and the next time_in in one launch
        c["action_out"] = tuple(x + y for x, y in zip(c["action_out"], c["time_in"]))
        del per_step["time_in"]  # c["time_in"] stays: the first step's time_in runs alone
        if M <= BOUNDARY_TIME_OUT_MAX_ROWS:  # ... and the next time_out (one query)
            c["action_out"] = tuple(x + y for x, y in zip(c["action_out"], c["time_out"]))
            del per_step["time_out"]
    if B > CROSS_Q_MAX_BATCH:  # the cross layers' Q projection is a launch of its own
        c["q_cross"] = (mat(960, 720), M * 720 * 2 + M * 960 * 2, 2.0 * M * 960 * 720)
        per_step["q_cross"] = L // 2
    return c, per_step


CROSS_Q_MAX_BATCH = 8  # largest batch whose cross layers fold the Q projection into attention (library constant)
BOUNDARY_MAX_ROWS = 4800  # largest query group (chunk rows) whose step boundary is one launch (library plan)
BOUNDARY_TIME_OUT_MAX_ROWS = 64  # largest group whose boundary launch also runs the time MLP's second layer
KERNEL_IDS = {"qkv_self": 0, "attn_self": 1, "attn_cross": 2, "o": 3, "gate_up": 4, "down": 5, "action_out": 6,
              "q_cross": 8, "time_in": 9, "time_out": 10}
LOOP_ID = 7  # smolexp_time_kernel: the whole call


def loop_algorithmic(L, B, lengths, n_steps, w8=False):
    """Whole-call algorithmic bytes and flops: per step, every launch's algorithmic bytes
    (parameters once, valid prefix K/V once) and flops, from kernel_costs."""
    c, per_step = kernel_costs(L, B, lengths, 0, w8)
    byt = sum(c[k][0] * n for k, n in per_step.items())
    fl = sum(c[k][2] * n for k, n in per_step.items())
    return n_steps * byt, n_steps * fl


def roofline_of(bytes_, flops, seconds):
    """Bound by arithmetic intensity against the ridge of the published peaks."""
    if flops / bytes_ < RIDGE:
        r = {"bound": "hbm", "achieved": bytes_ / seconds / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": flops / seconds / 1e12, "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    return r


def kernel_table(fm, h, cfg, L, B, lengths, P, reps, w8=False):
    """Per timed kernel: the hook's HIP-event time per launch (one graph of `reps` launches,
    each repeating that kernel's launch of the next layer, and of the next query group, in the
    first step of the last call), launches per call, and the launch's algorithmic bytes,
    activation bytes and flops (averaged over the call's query groups, which the library runs
    as concurrent chains of launches)."""
    groups = fm.smolexp_batch_groups(cfg, B)
    tot, launches = {}, {}
    # groups whose step boundary runs the time MLP's layers: the first step's launches of them
    first = {"time_in": [0.0, 0.0, 0.0, 0], "time_out": [0.0, 0.0, 0.0, 0]}
    b0 = 0
    for bg in groups:
        costs, per_step = kernel_costs(L, bg, lengths[b0:b0 + bg], P, w8)
        b0 += bg
        for name, n in per_step.items():
            t = tot.setdefault(name, [0.0, 0.0, 0.0])
            for i in range(3):
                t[i] += costs[name][i] * n
            launches[name] = launches.get(name, 0) + n
        for name, f in first.items():
            if name not in per_step:
                for i in range(3):
                    f[i] += costs[name][i]
                f[3] += 1
    kern = {}
    for name, kid in KERNEL_IDS.items():
        if name in launches:
            n, n_call, sums = launches[name], launches[name] * cfg.n_steps, tot[name]
        elif name in first and first[name][3]:  # once per call and group
            n, n_call, sums = first[name][3], first[name][3], first[name][:3]
        else:  # not launched at this batch (folded into another kernel)
            continue
        us = fm.smolexp_time_kernel(h, kid, reps)
        byt, act, fl = (v / n for v in sums)
        kern[name] = {"avg_us": us, "launches_per_call": n_call, "us_per_call": us * n_call,
                      "bytes": byt, "activation_bytes": act, "flops": fl}
    return kern


def timed_calls(call, n, warmup, stream):
    """Per-call milliseconds of n calls, each bracketed by HIP events on the stream."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def median(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def device_inputs(wl):
    import numpy as np
    import torch
    d = {"kv": torch.from_numpy(np.ascontiguousarray(wl["prefix_kv"]).view(np.int16)).cuda(),
         "mask": torch.from_numpy(wl["mask"]).cuda(), "noise": torch.from_numpy(wl["noise"]).cuda()}
    d["prev"] = torch.from_numpy(wl["prev_actions"]).cuda() if wl["prev_actions"] is not None else None
    return d


def overwrite_delta(fm, h, cfg, dev, prev, d, calls, warmup, stream):
    """Per-call time with the first d rows overwritten before every step against the same call
    without the overwrite, on one handle: `calls` calls of each, alternating in rounds of 5."""
    import torch
    B = dev["mask"].shape[0]
    out = torch.empty((B, 50, 32), device="cuda")
    with_ow = lambda: fm.smolexp_denoise_ex(h, cfg, dev["kv"], dev["mask"], dev["noise"], out,  # noqa: E731
                                            prev_actions=prev, overwrite_rows=d)
    without = lambda: fm.smolexp_denoise_ex(h, cfg, dev["kv"], dev["mask"], dev["noise"], out)  # noqa: E731
    a, b = [], []
    for r in range((calls + 4) // 5):
        a += timed_calls(with_ow, 5, warmup if r == 0 else 1, stream)
        b += timed_calls(without, 5, warmup if r == 0 else 1, stream)
    ma, mb = median(a), median(b)
    return {"overwrite_rows": d, "ms_per_call_with": ma, "ms_per_call_without": mb, "calls_each": len(a),
            "delta_ms_per_call": ma - mb, "delta_ms_per_chunk": (ma - mb) / B,
            "note": "median of per-call HIP-event times; the call's latency is each chunk's latency, "
                    "delta_ms_per_chunk spreads the call's difference over its batch"}


def large_batch_entry(fm, h, cfg, wl, calls, warmup, reps, stream):
    """One large-batch workload on the handle: per-call median, chunks/s, the loop's MFMA
    fraction and the dominant kernel's (hook time), and the prefix-overwrite difference when
    the workload overwrites rows."""
    import torch
    L, B, P, d = wl["n_layers"], wl["batch"], wl["prefix_len"], wl["overwrite_rows"]
    dev = device_inputs(wl)
    out = torch.empty((B, 50, 32), device="cuda")
    call = lambda: fm.smolexp_denoise_ex(h, cfg, dev["kv"], dev["mask"], dev["noise"], out,  # noqa: E731
                                         prev_actions=dev["prev"], overwrite_rows=d)
    ms = timed_calls(call, calls, warmup, stream)
    assert torch.isfinite(out).all().item(), "non-finite actions"
    lb, lf = loop_algorithmic(L, B, wl["lengths"], cfg.n_steps)
    med = median(ms)
    kern = kernel_table(fm, h, cfg, L, B, wl["lengths"], P, reps)
    dom_name = max(kern, key=lambda k: kern[k]["us_per_call"])
    dom = kern[dom_name]
    e = {"batch": B, "prefix_len": P, "overwrite_rows": d, "query_groups": fm.smolexp_batch_groups(cfg, B),
         "calls": calls, "ms_per_call": med,
         "ms_per_call_min": min(ms), "ms_per_call_max": max(ms), "chunks_per_s": B / (med * 1e-3),
         "loop_algorithmic_flops_per_call": lf, "loop_algorithmic_bytes_per_call": lb,
         "loop_tflops": lf / (med * 1e-3) / 1e12, "loop_mfma_frac": lf / (med * 1e-3) / (MFMA_F16_PEAK_TFS * 1e12),
         "dominant_kernel": {"kernel": dom_name, "avg_us": dom["avg_us"], "us_per_call": dom["us_per_call"],
                             "tflops": dom["flops"] / (dom["avg_us"] * 1e-6) / 1e12,
                             "mfma_frac": dom["flops"] / (dom["avg_us"] * 1e-6) / (MFMA_F16_PEAK_TFS * 1e12),
                             # fabric bytes per launch from the calibrated FETCH/WRITE counters, where
                             # profiles/ holds them for this workload and the current kernel sources
                             "traffic": stored_traffic(wl["name"], "gate_up_big") if dom_name == "gate_up" else None},
         "kernels": {k: {"avg_us": v["avg_us"], "us_per_call": v["us_per_call"],
                         "mfma_frac": v["flops"] / (v["avg_us"] * 1e-6) / (MFMA_F16_PEAK_TFS * 1e12)}
                     for k, v in kern.items()}}
    if d > 0:
        e["overwrite"] = overwrite_delta(fm, h, cfg, dev, dev["prev"], d, calls, 2, stream)
    return e


def e4m3_entry(fm, wl, packed, n_steps, calls, warmup, reps, stream):
    """The same workload on a handle with 8-bit weights (E4M3 codes, a scale per row):
    median per-call time of `calls` HIP-event-timed calls, the per-kernel hook times and the
    dominant kernel's roofline at the 8-bit byte count."""
    import torch
    L, B, P, d = wl["n_layers"], wl["batch"], wl["prefix_len"], wl["overwrite_rows"]
    cfg = fm.smolexp_default_config(n_layers=L, n_steps=n_steps, max_batch=B, max_prefix=P,
                                    weight_format=fm.SMOLEXP_WEIGHTS_E4M3)
    h = fm.smolexp_create(cfg, 0)
    try:
        fm.smolexp_load_weights(h, packed)
        dev = device_inputs(wl)
        out = torch.empty((B, 50, 32), device="cuda")

        def call():
            fm.smolexp_denoise_ex(h, cfg, dev["kv"], dev["mask"], dev["noise"], out, prev_actions=dev["prev"],
                                  overwrite_rows=d)

        ms = median(timed_calls(call, calls, warmup, stream))
        assert torch.isfinite(out).all().item(), "non-finite actions (8-bit weights)"
        kern = kernel_table(fm, h, cfg, L, B, wl["lengths"], P, reps, w8=True)
    finally:
        fm.smolexp_destroy(h)
    dom_name = max(kern, key=lambda k: kern[k]["us_per_call"])
    dom = kern[dom_name]
    roof = roofline_of(dom["bytes"], dom["flops"], dom["avg_us"] * 1e-6)
    roof.update(kernel=dom_name, avg_us=dom["avg_us"], algorithmic_bytes_per_launch=dom["bytes"])
    lb, _ = loop_algorithmic(L, B, wl["lengths"], n_steps, w8=True)
    return {"weight_format": "OCP FP8 E4M3 codes, one power-of-two scale per output row (opt-in)",
            "ms_per_call": ms, "chunks_per_s": B / (ms * 1e-3), "calls": calls,
            "loop_algorithmic_bytes_per_call": lb, "loop_hbm_frac": lb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "roofline": roof, "kernels": {k: {"avg_us": v["avg_us"], "us_per_call": v["us_per_call"]}
                                          for k, v in kern.items()}}


def cpu_baseline(wl, n_steps, min_seconds, max_seconds, threads=None):
    """The float64 numpy oracle on the host, on whole chunks of the workload's first queries
    (BLAS threads: all, or `threads`)."""
    import contextlib
    import threadpoolctl
    import oracle
    W = oracle.decode_weights(wl["weights"])
    cfg = oracle.ExpertConfig(n_layers=wl["n_layers"])
    B = wl["batch"]
    limit = threadpoolctl.threadpool_limits(threads) if threads else contextlib.nullcontext()
    with limit:
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
    ap.add_argument("--kernel-reps", type=int, default=200,
                    help="launches per kernel in the timing hook; 0: only the timed calls (loop-only profiling run)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graphs", action="store_true", help="launch kernels one by one instead of graph replay")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the workload's own line: no large-batch block and no overwrite difference")
    ap.add_argument("--large-calls", type=int, default=20, help="timed calls per large-batch workload")
    ap.add_argument("--large-kernel-reps", type=int, default=20)
    ap.add_argument("--batch", type=int, default=None,
                    help="override the workload's batch (the first queries of its seeded draws)")
    ap.add_argument("--weights", choices=("fp16", "e4m3"), default="fp16",
                    help="weight storage of the timed handle (e4m3: 8-bit, batches up to 8)")
    ap.add_argument("--batch-groups", type=int, default=0,
                    help="concurrent query groups per call (0: the library's automatic choice)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurement, copy 256 MiB device-to-device three times (HBM counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter_collection.csv files")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="per-kernel averages of the whole calls and of the timing graphs, from a rocprofv3 "
                         "--kernel-trace of a bench command")
    ap.add_argument("--summarize-stalls", nargs=2, metavar=("PASS1_CSV", "PASS2_CSV"),
                    help="print per-kernel wait / issue / MFMA-busy fractions from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-mfma", metavar="COUNTER_CSV",
                    help="per-kernel matrix-core utilisation from a rocprofv3 --pmc run of the MFMA counters")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_stalls:
        summarize_stalls(*args.summarize_stalls)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
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

    wl = synth.make_workload(args.workload, batch=args.batch)
    L, B, P, d = wl["n_layers"], wl["batch"], wl["prefix_len"], wl["overwrite_rows"]
    w8 = args.weights == "e4m3"
    cfg = fm.smolexp_default_config(n_layers=L, n_steps=args.n_steps, max_batch=B, max_prefix=P,
                                    use_graphs=0 if args.no_graphs else 1, batch_groups=args.batch_groups,
                                    weight_format=fm.SMOLEXP_WEIGHTS_E4M3 if w8 else fm.SMOLEXP_WEIGHTS_FP16)
    h = fm.smolexp_create(cfg, 0)
    packed = synth.pack_weights(wl["weights"], L)
    fm.smolexp_load_weights(h, packed)
    dev = device_inputs(wl)
    out = torch.empty((B, 50, 32), device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        fm.smolexp_denoise_ex(h, cfg, dev["kv"], dev["mask"], dev["noise"], out, prev_actions=dev["prev"],
                              overwrite_rows=d)

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

    # the whole call replayed by the timing hook (HIP events around the replays)
    loop_us = fm.smolexp_time_kernel(h, LOOP_ID, max(3, args.steps // 5))
    if args.kernel_reps == 0:
        # loop-only run (the reference for --summarize-trace): everything but the per-kernel timing
        print(json.dumps({"metric": "loop-only run for a kernel trace (no per-kernel timing)",
                          "ms_per_step": wall / args.steps * 1e3, "steps": args.steps, "warmup": args.warmup,
                          "config": {"workload": args.workload, "batch": B, "prefix_len": P}}), flush=True)
        fm.smolexp_destroy(h)
        return
    # per-kernel time per launch: HIP events on the library's stream around one graph of launches
    kern = kernel_table(fm, h, cfg, L, B, wl["lengths"], P, args.kernel_reps, w8=w8)
    dom_name = max(kern, key=lambda k: kern[k]["us_per_call"])
    dom = kern[dom_name]
    roof = roofline_of(dom["bytes"], dom["flops"], dom["avg_us"] * 1e-6)
    roof["traffic"] = None if w8 else stored_traffic(args.workload, dom_name)
    roof["kernel"] = dom_name
    roof["avg_us"] = dom["avg_us"]
    roof["algorithmic_bytes_per_launch"] = dom["bytes"]
    roof["algorithmic_flops_per_launch"] = dom["flops"]
    roof["activation_bytes_per_launch"] = dom["activation_bytes"]
    roof["timing"] = ("hook: HIP events around one graph of launches of this kernel, each repeating its "
                      "launch of the next layer (the loop's weights in turn)")

    ms = wall / args.steps * 1e3
    lb, lf = loop_algorithmic(L, B, wl["lengths"], cfg.n_steps, w8=w8)
    loop = {"algorithmic_bytes_per_call": lb, "algorithmic_flops_per_call": lf,
            "hbm_frac": lb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "mfma_frac": lf / (ms * 1e-3) / (MFMA_F16_PEAK_TFS * 1e12),
            "event_ms_per_call": ev_ms / args.steps, "replay_us_per_call": loop_us,
            "launches_per_call": 1 + sum(v["launches_per_call"] for v in kern.values())}

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
        "precision": ("GEMM weights OCP E4M3 with a power-of-two scale per output row (8-bit opt-in), widened "
                      "exactly to fp16; " if w8 else
                      "GEMM operands fp16 (the bf16 weights re-encoded exactly; RMSNorm gains folded into the "
                      "following weights, rounded once; ") +
                     "activations rounded to fp16), attention operands bf16 "
                     "(the bf16 K/V cache as given, chunk Q/K/V and probabilities rounded to bf16), fp32 "
                     "accumulate, fp32 residual/norm scale/softmax/Euler state",
        "data": "synthetic (seeded: weights N(0,0.02) bf16, prefix K/V N(0,1) bf16, noise N(0,1))",
        "config": {"workload": args.workload, "n_layers": L, "batch": B, "prefix_len": P,
                   "n_steps": cfg.n_steps, "chunk": 50, "action_dim": 32, "overwrite_rows": d,
                   "weights": args.weights,
                   "graphs": not args.no_graphs, "query_groups": fm.smolexp_batch_groups(cfg, B)},
        "roofline": roof,
        "loop_roofline": loop,
        "kernels": kern,
        "gpu_state": gpu_state,
    }
    if B == 1 and d == 0 and not args.no_extra:
        # the prefix overwrite at batch 1 (the pages' per-chunk figure is a batch-1 latency)
        prev1 = torch.from_numpy(synth.draw_prev_actions(1, 7)).cuda()
        line["overwrite_b1"] = overwrite_delta(fm, h, cfg, dev, prev1, 7, 20, 3, stream)
    fm.smolexp_destroy(h)
    if B <= CROSS_Q_MAX_BATCH and not w8 and not args.no_extra:
        # the same workload with 8-bit weights (half the weight bytes, rounded weights)
        line["weights_e4m3"] = e4m3_entry(fm, wl, packed, cfg.n_steps, 20, 5, min(args.kernel_reps, 50), stream)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if args.workload == DEFAULT_WORKLOAD and args.batch is None and not args.no_extra:
        # the large-batch workloads on one handle with the same weights
        big = [synth.make_workload(n, with_weights=False) for n in LARGE_BATCH_WORKLOADS]
        cfg2 = fm.smolexp_default_config(n_layers=L, n_steps=args.n_steps,
                                         max_batch=max(w["batch"] for w in big),
                                         max_prefix=max(w["prefix_len"] for w in big),
                                         batch_groups=args.batch_groups)
        h2 = fm.smolexp_create(cfg2, 0)
        fm.smolexp_load_weights(h2, packed)
        line["large_batch"] = {}
        for w in big:
            line["large_batch"][w["name"]] = large_batch_entry(fm, h2, cfg2, w, args.large_calls, 3,
                                                               args.large_kernel_reps, stream)
            del w["prefix_kv"]
        fm.smolexp_destroy(h2)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, cfg.n_steps, args.cpu_seconds, 3 * args.cpu_seconds)
        if B == 1:
            line["cpu_baseline"]["single_thread"] = cpu_baseline(wl, cfg.n_steps, args.cpu_seconds / 2,
                                                                 3 * args.cpu_seconds, threads=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

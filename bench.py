#!/usr/bin/env python3
"""Benchmark of exact attention backward-over-backward (fa_bob) on one MI355X.

A step is one fa_bob call on inputs already resident in HBM: for bf16 inputs
the row-major pass (which also computes D = rowsum(dO * O)) and the
column-major pass; for fp32 inputs a row-scalar kernel runs first.  fa_fwd
(which supplies O and L) runs once before the timed region and is reported
separately, as is fa_bwd.

Throughput: 38 B H N^2 d flops per step (19 N x N x d contractions per head:
11 in the row pass, 8 in the column pass; half for causal attention) divided
by the step time, in TFLOP/s.  The default workload is "mid" (B=2, H=8,
N=4096, d=64, bf16); the other workloads (N = 16K, 64K, 262K, the causal
isolated-layer shapes and the multi-query range) are timed as a sweep in the
same JSON line.

Per-kernel times come from HIP events recorded on the launch stream between
the kernels of each timed step (fa_bob_phase in order is exactly fa_bob).
The dominant kernel is the row pass (22 of the 38 flops).  Progress lines go
to stderr; the JSON line is the only line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_FP32_MFMA_TFLOPS = 157.3
# The FlashBoB paper's own BoB wall-clock times and peak memory for these shapes
# (Table 1: batch 4, 12 heads, causal, bf16 inputs with fp32 reductions), on
# other GPUs: context printed beside ours (time, device_bytes), never a target.
PAGES_MS = {
    "gpt2c_4k": {"ms": 25.80, "peak_mib": 1243, "gpu": "A100 80GB", "source": "FlashBoB Table 1, d=64"},
    "gpt2c_16k": {"ms": 365.73, "peak_mib": 3372, "gpu": "A100 80GB", "source": "FlashBoB Table 1, d=64"},
    "c128_16k": {"ms": 263.6, "peak_mib": 4422, "gpu": "B300", "source": "FlashBoB Table 1, d=128"},
}
# The pages' schedule ablation (three-pass vs two-pass; GPT-2 Small shape,
# batch 4, on A100), context only.
PAGES_ABLATION = {
    "gpt2c_4k": {"three_pass_ms": 27.30, "two_pass_ms": 25.80, "ratio": 1.06, "gpu": "A100 80GB",
                 "source": "FlashBoB Table 8"},
    "gpt2c_16k": {"three_pass_ms": 389.14, "two_pass_ms": 365.73, "ratio": 1.06, "gpu": "A100 80GB",
                  "source": "FlashBoB Table 8"},
    "gpt2c_64k": {"three_pass_ms": 6227.59, "two_pass_ms": 5843.14, "ratio": 1.07, "gpu": "A100 80GB",
                  "source": "FlashBoB Table 8"},
    "gpt2c_256k": {"three_pass_ms": 100696.16, "two_pass_ms": 94853.72, "ratio": 1.06, "gpu": "A100 80GB",
                   "source": "FlashBoB Table 8"},
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bob_pass1_traffic.json")
KERNEL_SOURCES = ("exact_second_order_fa_amd/csrc/fa_bob.hip", "exact_second_order_fa_amd/csrc/fa_bob_ws.hip",
                  "exact_second_order_fa_amd/csrc/fa_fwd_bwd.hip",
                  "exact_second_order_fa_amd/csrc/fa_lds.h",
                  "exact_second_order_fa_amd/csrc/fa_kernels.hip", "exact_second_order_fa_amd/csrc/fa_tile.h")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def host_info():
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process
    may use, CPU model and RAM."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ram = None
    try:
        ram = os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES")
    except (ValueError, OSError):
        pass
    return {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
            "ram_gib": round(ram / 2 ** 30, 1) if ram else None}


# Workloads whose inputs are drawn on the device (torch's generator, same
# distribution: N(0,1) rounded to bf16) because the host generator would
# take minutes for them; they are timed, never compared with the oracle.
DEVICE_DRAWN = ("gpt2c_64k", "gpt2c_256k")


def device_inputs(w):
    import torch

    from fa_inputs import NAMES, workload_inputs

    if w.name in DEVICE_DRAWN:
        g = torch.Generator(device="cuda").manual_seed(w.seed)
        out = {}
        for n in NAMES:
            heads = w.Hkv if n in ("k", "v", "uk", "uv") else w.H
            out[n] = torch.randn((w.B, heads, w.N, w.d), device="cuda", generator=g).to(torch.bfloat16)
        return out
    raw, _ = workload_inputs(w, with_f64=False)
    out = {}
    for k, v in raw.items():
        if w.dtype == "bf16":
            out[k] = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            out[k] = torch.from_numpy(v).cuda()
    return out


class Runner:
    """Inputs, saved forward state and preallocated outputs of one workload."""

    def __init__(self, w, dropout=0.0, seed=0):
        import torch

        import exact_second_order_fa_amd as fa

        self.fa, self.w = fa, w
        self.drop = dict(dropout=dropout, seed=seed)
        self.t = device_inputs(w)
        shape = (w.B, w.H, w.N, w.d)
        kshape = (w.B, w.Hkv, w.N, w.d)  # key-side outputs: one per key/value head
        self.o, self.lse = fa.fa_fwd(self.t["q"], self.t["k"], self.t["v"], causal=w.causal, **self.drop)
        self.outs = [torch.empty(s, dtype=torch.float32, device="cuda") for s in (shape, kshape, kshape, shape)]
        code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP32
        self.ws = torch.empty(fa.bob_workspace_bytes(*shape, code, w.causal, w.Hkv) // 4, dtype=torch.float32,
                              device="cuda")
        torch.cuda.synchronize()

    def bob(self, phase=None, schedule=None):
        t, g = self.t, self.outs
        self.fa.fa_bob(t["q"], t["k"], t["v"], self.o, self.lse, t["do"], t["uq"], t["uk"], t["uv"],
                       gq=g[0], gk=g[1], gv=g[2], gdo=g[3], ws=self.ws, phase=phase, causal=self.w.causal,
                       schedule=schedule, **self.drop)

    def fwd(self):
        self.fa.fa_fwd(self.t["q"], self.t["k"], self.t["v"], o=self.o, lse=self.lse, causal=self.w.causal,
                       **self.drop)

    def bwd(self):
        t, g = self.t, self.outs
        if not hasattr(self, "bws"):
            self.bws = None
        _, _, _, self.bws = self.fa.fa_bwd(t["q"], t["k"], t["v"], self.o, self.lse, t["do"], dq=g[0], dk=g[1],
                                           dv=g[2], ws=self.bws, causal=self.w.causal, **self.drop)


def time_steps(r, steps, warmup):
    """Warmup, then `steps` timed steps of the plain fa_bob call (wall clock,
    synchronized on both sides: the headline), then `steps` more with the
    three kernels launched one by one and HIP events recorded on the launch
    stream around each (the per-kernel breakdown; the events between kernels
    cost the step about 2 %).  Returns (wall ms/step, per-step ms of the
    event loop, per-kernel average ms)."""
    import torch

    for _ in range(warmup):
        r.bob()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.bob()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    stream = torch.cuda.current_stream()
    # bf16: phase 0 (the row-scalar kernel) launches nothing, D comes out of
    # the row pass, so only phases 1 and 2 are timed.
    phases = (1, 2) if r.w.dtype == "bf16" else (0, 1, 2)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(stream)
        for i, ph in enumerate(phases):
            r.bob(phase=ph)
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    per = {ph: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
           for i, ph in enumerate(phases)}
    step_ev = float(np.mean([ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]))
    return wall, step_ev, per


# From a cold start the step time of the mid workload falls by about 20 % over
# the first tens of milliseconds of continuous load while the GPU clock ramps,
# then stays flat for seconds.  Legs that follow host-side work (input
# generation) first run their step back to back for SETTLE_MS, and time at
# least TIMED_MS.
SETTLE_MS = 200.0
TIMED_MS = 100.0


def settle(fn, ms=SETTLE_MS):
    """Run fn back to back for about `ms` milliseconds of GPU time; returns the
    duration of one call in ms."""
    import torch

    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    t1 = a.elapsed_time(b)
    for _ in range(int(ms / max(t1, 1e-3))):
        fn()
    torch.cuda.synchronize()
    return t1


def reps_for(t1, lo=3, hi=2000):
    return max(lo, min(hi, int(math.ceil(TIMED_MS / max(t1, 1e-3)))))


def time_plain(fn, reps):
    import torch

    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def hvp_leg(r):
    """One Hessian-vector product through attention ([FlashBoB] section 4.1):
    the linear loss <O, W> through sdpa_bob, its gradient with create_graph,
    then the gradient of <(dQ, dK, dV), z>: fa_fwd, fa_bwd and fa_bob through
    the autograd wrapper, with its elementwise torch ops and Python overhead."""
    import torch

    from exact_second_order_fa_amd.autograd import sdpa_bob

    w = r.w
    q, k, v = (r.t[n].detach().clone().requires_grad_(True) for n in ("q", "k", "v"))
    W = r.t["do"].float()
    z = [r.t[n].float() for n in ("uq", "uk", "uv")]

    def step():
        o = sdpa_bob(q, k, v, causal=w.causal)
        g = torch.autograd.grad((o * W).sum(), (q, k, v), create_graph=True)
        s_ = sum((gi.float() * zi).sum() for gi, zi in zip(g, z))
        torch.autograd.grad(s_, (q, k, v))

    ms = time_plain(step, reps_for(settle(step)))
    return {"workload": w.name, "ms": round(ms, 4), "loss": "linear <O, W>",
            "calls": "sdpa_bob autograd: fa_fwd, fa_bwd, fa_bob and the loss's elementwise torch ops"}


def traffic_for(workload):
    """Per-launch HBM bytes of the row pass from the committed rocprofv3
    counter summary, or None when missing or taken on other kernel code."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_source_sha() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, heads):
    """The float64 oracle on a bounded sample (the first `heads` heads of the
    workload, full row and column passes), scaled to TFLOP/s in the same
    38 N^2 d accounting, on every CPU this process may use."""
    from fa_inputs import workload_inputs
    from oracle import col_pass, row_pass

    _, f64 = workload_inputs(w)
    threads = len(os.sched_getaffinity(0))
    done = 0
    t0 = time.perf_counter()
    for bh in range(heads):
        b, h = divmod(bh, w.H)
        a = [f64[n][b, h] for n in ("q", "k", "v", "do", "uq", "uk", "uv")]
        r = row_pass(*a, w.scale, outputs="all", threads=threads)
        col_pass(*a, w.scale, r, threads=threads)
        done += 1
    dt = time.perf_counter() - t0
    flops = 38.0 * done * w.N * w.N * w.d
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} heads of workload {w.name} (N={w.N}, d={w.d}), full row and "
                      f"column passes in float64 on a pool of {threads} threads, {dt:.1f} s",
            "host": host_info()}


def peak_of(w):
    return PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS


def streamed_bytes(w, schedule):
    """Algorithmic bytes the sweeps stream from the other side (bf16 tiles and
    fp32 chain inits), with the row and column blocks of 128: the two-pass row
    pass streams K, V, U_K, U_V (8 d bytes per key per row block), the column
    pass Q, dO, U_Q and four row scalars (6 d + 16 bytes per row per key
    block), the three-pass alpha sweep K and U_K (4 d bytes per key per row
    block).  Causal attention streams half.  Counted per query head (with
    grouped heads, a key block streams the rows of the group's G heads)."""
    blocks = (w.N + 127) // 128
    row = blocks * w.N * 8 * w.d
    col = blocks * w.N * (6 * w.d + 16)
    alpha = blocks * w.N * 4 * w.d if schedule == 2 else 0
    f = w.B * w.H * (0.5 if w.causal else 1.0)
    return {"row_pass": row * f, "column_pass": col * f, "alpha_sweep": alpha * f, "total": (row + col + alpha) * f}


def model_bytes(w):
    """Algorithmic HBM bytes of one two-pass fa_bob call ([FlashBoB]
    Theorem 4.3 with element sizes): the streamed tiles above plus the
    stationary traffic, each resident block read once and each output written
    once: Q, U_Q, dO (bf16) and O (fp32) and L by the row pass; K, V, U_K, U_V
    (bf16) by the column pass; gQ, gdO, gK, gV written in fp32; D, alpha, E
    and the four per-row chain inits (28 bytes per row) written by the row
    pass."""
    e = 2 if w.dtype == "bf16" else 4
    qrows, krows = w.B * w.H * w.N, w.B * w.Hkv * w.N
    stationary = qrows * (3 * e * w.d + 4 * w.d + 4) + krows * 4 * e * w.d
    writes = qrows * (8 * w.d + 28) + krows * 8 * w.d
    return {"stationary": stationary + writes, "streamed": streamed_bytes(w, 0)["total"],
            "total": stationary + writes + streamed_bytes(w, 0)["total"]}


def device_bytes(r):
    """Device memory of one fa_bob call: what the workload holds resident
    (inputs, O, L, outputs, workspace) and what the call itself adds (torch's
    peak counter and the driver's free-memory delta; both 0: the library
    allocates nothing and no N x N buffer exists)."""
    import torch

    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    r.bob()
    torch.cuda.synchronize()
    return {"resident": int(base), "call_peak_extra": int(torch.cuda.max_memory_allocated() - base),
            "call_free_delta": int(free0 - torch.cuda.mem_get_info()[0])}


def bob_flops_pass1(w):
    """Row-pass flops: 11 of the 19 contractions, halved for causal attention."""
    return 22.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)


def ablation(names, reps=5):
    """Three-pass vs two-pass ([FlashBoB] appendix G.1) on the same kernel
    machinery: the two-pass row pass with one wave per SIMD (the kernel the
    three-pass row sweep is built from) against the three-pass schedule, and
    the production two-pass (warp-specialised row pass) beside them.  Calls
    of a second or more are timed twice after one untimed call, with HIP
    events between the phases of the same calls."""
    import torch

    from fa_inputs import WORKLOADS

    out = {}
    for name in names:
        w = WORKLOADS[name]
        progress(f"ablation {name}")
        r = Runner(w)
        res = {}
        for label, sched, nph in (("two_pass", 0, 3), ("two_pass_1wave", 1, 3), ("three_pass", 2, 4)):
            t1 = settle(lambda: r.bob(schedule=sched))
            if t1 < 500.0:
                n = reps_for(t1, lo=reps)
                ms = time_plain(lambda: r.bob(schedule=sched), n)
                phases = [time_plain(lambda ph=ph: r.bob(phase=ph, schedule=sched), n) for ph in range(nph)]
            else:
                stream = torch.cuda.current_stream()
                ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(2)]
                for k in range(2):
                    ev[k][0].record(stream)
                    for ph in range(nph):
                        r.bob(phase=ph, schedule=sched)
                        ev[k][ph + 1].record(stream)
                torch.cuda.synchronize()
                phases = [float(np.mean([ev[k][ph].elapsed_time(ev[k][ph + 1]) for k in range(2)]))
                          for ph in range(nph)]
                ms = float(np.mean([ev[k][0].elapsed_time(ev[k][-1]) for k in range(2)]))
            res[label] = {"ms": round(ms, 3), "phase_ms": [round(x, 3) for x in phases]}
        sb2, sb3 = streamed_bytes(w, 0), streamed_bytes(w, 2)
        res["ratio_three_over_two_1wave"] = round(res["three_pass"]["ms"] / res["two_pass_1wave"]["ms"], 3)
        res["ratio_three_over_two"] = round(res["three_pass"]["ms"] / res["two_pass"]["ms"], 3)
        res["streamed_bytes"] = {"two_pass": sb2["total"], "three_pass": sb3["total"],
                                 "saving_of_two_pass": round(1 - sb2["total"] / sb3["total"], 4)}
        res["shape"] = {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                        "inputs": "drawn on the device" if name in DEVICE_DRAWN else "host generator"}
        if name in PAGES_ABLATION:
            res["pages_context"] = PAGES_ABLATION[name]
        out[name] = res
        del r
        torch.cuda.empty_cache()
    return out


# Sweep workloads whose line also times the prerequisites (fa_fwd, fa_bwd).
PREREQ_SWEEP = ("long", "hd128", "gpt2c_16k")


def prerequisites(r, w):
    """fa_fwd and fa_bwd on the runner's workload: back to back for SETTLE_MS,
    then timed over at least TIMED_MS, so that both are reported at a settled
    clock.  Flops ([FlashBoB] section 3): 2 N^2 d per contraction; forward 2
    contractions, first backward 5 (S, dP, dV, dQ, dK); causal half."""
    fwd_ms = time_plain(r.fwd, reps_for(settle(r.fwd)))
    bwd_ms = time_plain(r.bwd, reps_for(settle(r.bwd)))
    cf = (0.5 if w.causal else 1.0) * 2.0 * w.B * w.H * w.N * w.N * w.d
    out = {}
    for op, ms, n in (("fa_fwd", fwd_ms, 2), ("fa_bwd", bwd_ms, 5)):
        tf = n * cf / (ms * 1e9)
        out[op] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_peak": round(tf / peak_of(w), 4)}
    return out


def sweep_leg(name):
    import torch

    from fa_inputs import WORKLOADS

    sw = WORKLOADS[name]
    progress(f"sweep {name}")
    r = Runner(sw)
    reps = reps_for(settle(r.bob))
    _, s_ev, s_per = time_steps(r, reps, 0)
    tf = sw.bob_flops / (s_ev * 1e9)
    mb = model_bytes(sw)
    res = {"B": sw.B, "H": sw.H, "H_kv": sw.Hkv, "N": sw.N, "d": sw.d, "causal": sw.causal,
           "ms": round(s_ev, 3), "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
           "pass1_ms": round(s_per[1], 3), "pass2_ms": round(s_per[2], 3),
           "model_GBps": round(mb["total"] / (s_ev * 1e6), 1),
           "device_bytes": device_bytes(r)}
    if 0 in s_per:
        res["rowscalar_ms"] = round(s_per[0], 4)
    if name in PREREQ_SWEEP:
        res["prerequisites"] = prerequisites(r, sw)
    if name in PAGES_MS:
        res["pages_ms_context"] = PAGES_MS[name]
    del r
    torch.cuda.empty_cache()
    return res


def main():
    from fa_inputs import MQA_SWEEP

    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: 200 warm-up steps (about 130 ms on the mid workload) take the
    # GPU past its clock ramp; 400 timed steps.
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="mid")
    ap.add_argument("--sweep", default="hd128,long,max,gpt2c_4k,gpt2c_16k,c128_16k," + ",".join(MQA_SWEEP),
                    help="comma list of extra workloads ('' for none)")
    ap.add_argument("--ablation", default="gpt2c_4k,gpt2c_16k,gpt2c_64k,gpt2c_256k",
                    help="workloads of the three-pass vs two-pass schedule ablation ('' for none)")
    ap.add_argument("--only-ablation", action="store_true", help="run only the schedule ablation (profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--dropout", type=float, default=0.1,
                    help="rate of the dropout-variant timing leg on the main workload (0: skip)")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU oracle sample (0: all)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (three times), the reference kernel "
                         "for scaling the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; the kernel runs on one GPU's share of the "
              "heads and --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}), flush=True)
        return

    from fa_inputs import WORKLOADS

    abl_names = [s_ for s_ in args.ablation.split(",") if s_]
    if args.only_ablation:
        print(json.dumps({"ablation": ablation(abl_names)}), flush=True)
        return

    w = WORKLOADS[args.workload]
    progress(f"workload {w.name}: inputs")
    r = Runner(w)
    # Legs on the same resident inputs first (one Hessian-vector product
    # through sdpa_bob; fa_fwd and fa_bwd), then the headline: W warm-up and K
    # timed fa_bob steps, which so start at the clock those legs leave.
    progress("hvp step")
    hvp = hvp_leg(r)
    progress("prerequisites")
    prereq = prerequisites(r, w)
    progress(f"headline: {args.warmup} warm-up and {args.steps} timed steps")
    wall, step_ev, per = time_steps(r, args.steps, args.warmup)
    bob_ms = time_plain(r.bob, args.steps)
    dev_bytes = device_bytes(r)
    flops = w.bob_flops
    peak = peak_of(w)
    value = flops / (wall * 1e9)
    pass1_flops = bob_flops_pass1(w)
    ach = pass1_flops / (per[1] * 1e9)
    traffic = traffic_for(w.name)
    mb = model_bytes(w)

    sweep = {}
    for name in [s_ for s_ in args.sweep.split(",") if s_]:
        del r
        torch.cuda.empty_cache()
        r = None
        sweep[name] = sweep_leg(name)

    # The dropout variant ([FlashBoB] appendix G) on the same workload, with
    # the Philox mask, reported beside the headline.
    dropout_leg = None
    if args.dropout > 0:
        del r
        torch.cuda.empty_cache()
        progress("dropout variant")
        r = Runner(w, dropout=args.dropout, seed=1234)
        d_ms = time_plain(r.bob, reps_for(settle(r.bob)))
        dropout_leg = {"p": args.dropout, "seed": 1234, "workload": w.name, "fa_bob_ms": round(d_ms, 4),
                       "tflops": round(w.bob_flops / (d_ms * 1e9), 1),
                       "ratio_to_dropout_free": round(d_ms / bob_ms, 3),
                       "kernels": ("LDS-DMA row pass and split-schedule column pass" if w.dtype == "bf16"
                                   else "portable") + ", mask from Philox4x64-10"}

    kernels_ms = {"bob_pass1": round(per[1], 4), "bob_pass2": round(per[2], 4), "step_events": round(step_ev, 4),
                  "fa_bob_single_call": round(bob_ms, 4), "fa_fwd": prereq["fa_fwd"]["ms"]}
    if 0 in per:
        kernels_ms["rowscalar"] = round(per[0], 4)
    else:
        kernels_ms["row_scalars"] = "D = rowsum(dO * O) is computed inside bob_pass1 (no separate kernel)"
    line = {
        "metric": "fa_bob TFLOP/s (38 B H N^2 d flops per call) and fraction of bf16 dense MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, see fa_inputs)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "in_dtype": w.dtype, "scale": "1/sqrt(d)"},
        "frac_peak": round(value / peak, 4),
        "roofline": {"bound": "mfma", "kernel": "bob_pass1 (row pass)", "achieved": round(ach, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                     "traffic": traffic, "flops_per_launch": pass1_flops,
                     "kernel_src_sha": kernel_source_sha()},
        "hbm": {"model_bytes_per_call": mb, "model_GBps": round(mb["total"] / (wall * 1e6), 1),
                "pass1_counter_GBps": (round(traffic / (per[1] * 1e6), 1) if traffic else None),
                "peak_GBps": 8000.0},
        "device_bytes": dev_bytes,
        "kernels_ms": kernels_ms,
        "prerequisites": prereq,
        "sweep": sweep,
        "dropout_variant": dropout_leg,
        "hvp_step": hvp,
    }
    if abl_names:
        del r
        torch.cuda.empty_cache()
        r = None
        line["schedule_ablation"] = ablation(abl_names)
    if not args.no_cpu:
        progress("CPU baseline")
        nh = w.B * w.H if args.cpu_heads <= 0 else min(args.cpu_heads, w.B * w.H)
        line["cpu_baseline"] = cpu_baseline(w, nh)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the gated delta rule forward + backward on one MI355X.

Default workload: the Qwen3.5-9B GatedDeltaNet layer shape (B=1, T=2048,
Hk=16, Hv=64, Dk=192, Dv=128), bf16 q/k/v/a/b/dO, fp32 state, zero initial
state, synthetic seeded inputs (the workload of the mlx-lm VJP PR's
performance table).  One step = gdn_fwd (with checkpoints) + gdn_bwd on the
same resident inputs.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
                  [--config 9b_t2048|9b_t256|decode|decode_conv|vg_t2048|vg_t256|long_t32k]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/sec at Hk16/Hv64/Dk192/Dv128 bf16, T=2048; % HBM roofline"
HBM_PEAK = 8.0e12            # B/s, MI355X HBM3E
FP32_VEC_PEAK = 157.3e12     # FLOP/s, MI355X fp32 vector (packed FMA)
# Metal VJP fwd+bwd on an M4 Max (mlx-lm PR, "Performance" table), for context
PAGES_FWD_BWD_MS = {256: 13.4, 2048: 149.8}
PAGES_FWD_BWD_MS_ALL = {256: 13.4, 512: 28.2, 1024: 62.2, 2048: 149.8}

# Kernels launched per step, in order, by kernel family.
KERNELS = {
    "scan": ["prep_fwd", "scan_fwd", "prep_bwd", "scan_bwd", "chunk_grad", "param_reduce"],
    # the forward's chunk_prep also saves the backward's chunk matrices in the
    # checkpoint buffer (gdn_dims.save, as in training), so the backward has
    # no chunk_prep of its own
    "chunk": ["chunk_prep", "chunk_fwd", "chunk_bwd_state", "chunk_bwd_grad", "param_reduce"],
}
# Algorithmic fp32 flops per state element-step (one (b, t, h, i, j)):
#   scan_fwd   decay 1 mul, read u 1 fma, update 1 fma, read o 1 fma       = 7
#   scan_bwd   recompute 5 (as above without o) + reverse step: read ein
#              1 fma, carry update 1 mul + 2 fma                           = 12
#   chunk_grad the method's per-step gradient contractions: dq = S dO
#              1 fma, dk = D delta + S' du 2 fma, dg = <dS', S> 1 fma      = 8
FLOPS_PER_ELEM = {"scan_fwd": 7, "scan_bwd": 12, "chunk_grad": 8}
# Per-key-channel gate (gdn_fwd_vg / gdn_bwd_vg): the same forward (the gate
# is applied per row, not per element), and the reverse sweep as one kernel:
#   scan_bwd_vg  recompute 5 (decay 1 mul, read u 1 fma, update 1 fma) +
#                reverse: D += qn dO^T 1 fma, dqn = S dO 1 fma, eps = D^T kn
#                1 fma, dS' = D + kn du^T 1 fma, dkn = D delta + S' du 2 fma,
#                dlg = <dS', S> along the row 1 fma, carry D = g dS' 1 mul    = 20
KERNELS["vg"] = ["prep_fwd", "scan_fwd", "prep_bwd", "scan_bwd_vg", "vg_reduce"]
# ... and its chunk form (bf16), with the saved record (gdn_dims.save, as in
# training): the forward's vg_chunk_prep (which also writes the backward's
# rows and matrices) and chunk_fwd (VG mode, which also writes X); the
# backward's step scalars (prep), chunk_bwd_state (VG mode), the gradient
# pass (the L x L gradients and db from the saved X; the per-channel
# expansions and dlg; the L2-norm backward of q, k)
KERNELS["vg_chunk"] = ["vg_prep_fwd", "chunk_fwd_vg", "prep_bwd", "chunk_bwd_state_vg",
                       "vg_chunk_x", "vg_chunk_grad", "vg_norm_bwd"]
FLOPS_PER_ELEM.update({"scan_bwd_vg": 20})
VG_METRIC = "fwd+bwd tokens/sec with a per-key-channel gate at Hk16/Hv64/Dk192/Dv128 bf16, T=2048"


def kernel_bytes(B, T, Hk, Hv, Dk, Dv, io, state0=False, dS_final=False):
    """Algorithmic HBM bytes of each chunk-form kernel: the tensors of the
    method-bytes formula (method_bytes) that the kernel reads or writes, each
    counted once, with the formula's fp32 checkpoints (written by the forward,
    read by the backward) standing for what the saved path hands from
    chunk_fwd to chunk_bwd_grad in their place (bf16 chunk-start states and X,
    which are smaller).  Intermediates in the workspace or the checkpoint
    buffer (chunk matrices, eps, per-chunk state gradients) are not counted."""
    Q1 = B * T * Hk * Dk * io            # one of q, k (or dq, dk)
    V1 = B * T * Hv * Dv * io            # one of v, o, dO, dv
    A1 = B * T * Hv * io                 # one of a, b, da, db
    Par = 2 * Hv * 4
    Sig = B * Hv * Dk * Dv * 4
    CK = max(math.ceil(T / 64) - 1, 0) * Sig
    s0 = Sig if state0 else 0
    return {
        "chunk_prep": 2 * Q1 + 2 * A1 + Par,
        "chunk_fwd": 2 * Q1 + 2 * V1 + s0 + Sig + CK,
        "chunk_bwd_state": Q1 + 2 * V1 + (Sig if dS_final else 0) + Sig,
        "chunk_bwd_grad": 2 * Q1 + V1 + A1 + CK + 2 * Q1 + 2 * A1,
        "param_reduce": Par,
    }


TRACE_FILE = os.path.join(ROOT, "profiles", "chunk_path_9b_t2048_fwd_bwd.txt")


def recorded_trace_median(kernel):
    """Median duration (ms) of `kernel` in the committed rocprofv3 kernel trace
    of the default workload, or None when there is none or the library source
    has changed since it was taken."""
    from linear_attention_recurrence_fwd_amd.srcsha import source_sha
    try:
        lines = open(TRACE_FILE).read().splitlines()
    except OSError:
        return None
    sha = next((l.split()[1] for l in lines if l.startswith("source_sha ")), None)
    if sha != source_sha():
        return None
    for l in lines:
        if "::%s_kernel<" % kernel in l:
            f = l.split()
            return float(f[-5]) / 1e3  # the median column (us)
    return None


def method_bytes(B, T, Hk, Hv, Dk, Dv, io, mask=False, dS_final=False):
    """Algorithmic HBM bytes of fwd + bwd: every I/O tensor once, plus the fp32
    checkpoints (written by fwd, read by bwd)."""
    Q = B * T * Hk * Dk * io
    V = B * T * Hv * Dv * io
    AB = 2 * B * T * Hv * io
    Par = 2 * Hv * 4
    Sig = B * Hv * Dk * Dv * 4
    Mk = B * T if mask else 0
    CK = max(math.ceil(T / 64) - 1, 0) * Sig
    fwd = 2 * Q + V + AB + Par + Mk + Sig + V + Sig + CK
    bwd = (2 * Q + V + AB + Par + Mk + Sig + CK + V + (Sig if dS_final else 0)) \
        + (2 * Q + V + AB + Par + Sig)
    return fwd, bwd


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_9b_t2048.txt")


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` at the default workload, from the
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by the copy probe), or
    None when there is none or the library source has changed since."""
    from linear_attention_recurrence_fwd_amd.srcsha import source_sha
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    sha = next((l.split()[1] for l in lines if l.startswith("source_sha ")), None)
    if sha != source_sha():
        return None
    for l in lines:
        f = l.split()
        if f and f[0] == kernel and len(f) == 6:
            return int(float(f[5]))
    return None


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            if self.hip.hipEventCreate(ctypes.byref(self.ev, i * ctypes.sizeof(ctypes.c_void_p))):
                raise RuntimeError("hipEventCreate failed")
        self.n = n

    def ptr(self, off):
        return ctypes.cast(ctypes.byref(self.ev, off * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[i]),
                                        ctypes.c_void_p(self.ev[j])):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(ctypes.c_void_p(self.ev[i]))


class Flush:
    """A 1 GiB scratch buffer written before every timed repetition, so that
    no operand of a repetition is served from the previous one's cache lines:
    the MI355X's memory-side cache (MALL, 256 MB) and the L2s hold the
    scratch afterwards, not the workload's tensors."""

    def __init__(self, torch, mib=1024):
        self.buf = torch.empty((mib << 20,), dtype=torch.uint8, device="cuda:0")
        self.n = 0

    def __call__(self):
        self.n = (self.n + 1) & 0xff
        self.buf.fill_(self.n)


def _stats(xs):
    xs = sorted(xs)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"median": round(med, 5), "min": round(xs[0], 5), "max": round(xs[-1], 5),
            "mean": round(sum(xs) / n, 5)}


def measure(torch, lib, stream, run, kernels, steps, warmup, flush):
    """Times `run` (one step: the library calls that make up the hot path).

    1. `steps` repetitions, each after a cache flush, each between two HIP
       events on the calls' stream (the flush is outside them): the per-step
       times (median, min, max).  The loop is bracketed by device
       synchronisations; its wall time includes the flushes.
    2. The same with every kernel between its own pair of events
       (gdn_set_kernel_events): per-kernel times (median over the steps).
    3. `steps` repetitions back to back without flushes, two events around
       all of them: the mean (the rate of a steady stream of calls, whose
       operands may partly come from cache)."""
    sp = ctypes.c_void_p(stream.cuda_stream)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = HipEvents(2 * steps)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(steps):
        flush()
        ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[2 * i]), sp)
        run()
        ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[2 * i + 1]), sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)]
    ev.close()
    nk = len(kernels)
    per_kernel = {k: [] for k in kernels}
    if nk:
        ev = HipEvents(2 * nk * steps)
        torch.cuda.synchronize()
        for i in range(steps):
            flush()
            lib.gdn_set_kernel_events(ev.ptr(2 * nk * i), 2 * nk)
            run()
        torch.cuda.synchronize()
        lib.gdn_set_kernel_events(None, 0)
        for i in range(steps):
            for j, k in enumerate(kernels):
                per_kernel[k].append(ev.elapsed_ms(2 * nk * i + 2 * j, 2 * nk * i + 2 * j + 1))
        ev.close()
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[0]), sp)
    for _ in range(steps):
        run()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[1]), sp)
    torch.cuda.synchronize()
    unflushed = ev.elapsed_ms(0, 1) / steps
    ev.close()
    return {"step": _stats(step_ms), "kernels": {k: _stats(v) for k, v in per_kernel.items() if v},
            "unflushed_ms": round(unflushed, 5), "wall_s": round(wall, 3)}


def time_calls(torch, fn, argl, steps, warmup, flush):
    """Decode-style timing: a step is the calls of `argl` in order (each a
    single-token call updating the state in place).  Flushed: every call after
    a cache flush, between its own two HIP events (median, min, max per call);
    unflushed: `steps` steps back to back, two events around all of them."""
    def call(a):
        rc = fn(*a)
        if rc:
            raise RuntimeError("library call failed with status %d" % rc)
    sp = argl[0][-1]
    for _ in range(warmup):
        for a in argl:
            call(a)
    torch.cuda.synchronize()
    n = steps * len(argl)
    ev = HipEvents(2 * n)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    i = 0
    for _ in range(steps):
        for a in argl:
            flush()
            ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[2 * i]), sp)
            call(a)
            ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[2 * i + 1]), sp)
            i += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    flushed = [ev.elapsed_ms(2 * j, 2 * j + 1) for j in range(n)]
    ev.close()
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[0]), sp)
    for _ in range(steps):
        for a in argl:
            call(a)
    ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[1]), sp)
    torch.cuda.synchronize()
    unflushed = ev.elapsed_ms(0, 1) / n
    ev.close()
    return {"flushed_call_ms": _stats(flushed), "unflushed_call_ms": round(unflushed, 5),
            "wall_s": round(wall, 3)}


def copy_bandwidth(torch, mib=1024, reps=5):
    """Measured device-to-device copy rate (bytes read + written per second)
    of a `mib` MiB buffer: the attainable counterpart of the nominal 8 TB/s."""
    n = mib << 20
    src = torch.empty((n,), dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    ms = _stats(ts)["median"]
    return {"bytes_per_copy": 2 * n, "median_ms": ms, "GBps": round(2 * n / (ms / 1e3) / 1e9, 1)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(T):
    """The fp64 oracle (as it stands: plain sequential C, parallel only over
    independent (batch, value head) pairs) timed on the host on bounded
    samples of the 9B workload at the same T, fwd + bwd:
      - all 16 key heads (64 value heads) on min(16, cpu_count) threads;
      - 2 key heads (8 value heads) on 1 thread, tokens/s scaled to the 64
        heads (the work is linear in the heads).
    `value` is the multi-threaded rate."""
    import oracle
    from linear_attention_recurrence_fwd_amd import inputs
    threads = max(1, min(16, os.cpu_count() or 1))

    def run(Hk, nth):
        c = inputs.make_case("9b_sample", 1, T, Hk, 4 * Hk, 192, 128, "bf16", 3, state_std=None,
                             dS_final=False)
        oracle.fwd(*c.oracle_args(), nthreads=nth)  # loads / warms the library
        t0 = time.perf_counter()
        oracle.fwd(*c.oracle_args(), nthreads=nth)
        oracle.bwd(*c.oracle_args(), c.vals["dO"], None, nthreads=nth)
        return time.perf_counter() - t0

    dt_n = run(16, threads)
    dt_1 = run(2, 1)
    return {"value": round(T / dt_n, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_thread_value": round(T / (dt_1 * 8), 3),
            "cpu_model": cpu_model(), "cpu_count": os.cpu_count(),
            "sample": "fp64 oracle fwd+bwd (64-step checkpointed recompute), B=1 T=%d Dk=192 "
                      "Dv=128: Hk=16 Hv=64 (the whole workload) in %.2f s wall on %d threads; "
                      "Hk=2 Hv=8 (1/8 of the heads) in %.2f s on 1 thread, tokens/s scaled by 1/8"
                      % (T, dt_n, threads, dt_1)}


def upload_case(torch, case, names):
    import numpy as np
    dev = torch.device("cuda:0")
    out = {}
    for n in names:
        x = case.store(n)
        if x is None:
            out[n] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(x))
        out[n] = (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)
    return out


TRAIN_NAMES = ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state0", "dO", "dS_final")


def train_plan(torch, binding, inputs, T, algo):
    case = inputs.qwen35_9b(T)
    t = upload_case(torch, case, TRAIN_NAMES)
    t["mask"] = None
    plan = binding.Plan(t, algo=algo)

    def run():
        plan.fwd()
        plan.bwd()
    return case, t, plan, run


def bench_train(args, torch, binding, inputs):
    T = {"9b_t2048": 2048, "9b_t256": 256}[args.config]
    algo = {"auto": binding.ALGO_AUTO, "scan": binding.ALGO_SCAN,
            "chunk": binding.ALGO_CHUNK}[args.algo]
    # the kernel family AUTO picks for this workload (bf16 with a supported
    # head size runs the chunked form)
    family = "scan" if args.algo == "scan" else "chunk"
    kernels = KERNELS[family]
    lib = binding.lib()
    flush = Flush(torch)
    case, t, plan, run = train_plan(torch, binding, inputs, T, algo)
    m = measure(torch, lib, plan.stream, run, kernels, args.steps, args.warmup, flush)
    del plan
    ms = m["step"]["median"]
    per_kernel = {k: v["median"] for k, v in m["kernels"].items()}

    B, Hk, Hv, Dk, Dv = case.B, case.Hk, case.Hv, case.Dk, case.Dv
    tokens = B * T
    value = tokens / (ms / 1e3)
    fb, bb = method_bytes(B, T, Hk, Hv, Dk, Dv, 2)
    E = B * T * Hv * Dk * Dv
    dom = max(per_kernel, key=lambda k: per_kernel[k])
    if family == "chunk":
        # HBM roofline of the slowest kernel, over its algorithmic bytes
        kb = kernel_bytes(B, T, Hk, Hv, Dk, Dv, 2, state0=t["state0"] is not None,
                          dS_final=t["dS_final"] is not None)
        achieved = kb[dom] / (per_kernel[dom] / 1e3) / 1e9
        traffic = recorded_traffic(dom) if T == 2048 else None
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                    "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": traffic,
                    "bytes_per_launch": kb[dom], "avg_launch_ms": round(per_kernel[dom], 4),
                    "launch_ms_timing": "median over the flushed steps, HIP events around the kernel"}
        tm = recorded_trace_median(dom) if T == 2048 else None
        if tm:
            roofline["trace_median_ms"] = round(tm, 4)
            roofline["trace_frac"] = round(kb[dom] / (tm / 1e3) / HBM_PEAK, 4)
    else:
        # fp32 vector roofline of the slowest kernel, over its algorithmic flops
        flops = FLOPS_PER_ELEM[dom] * E
        achieved = flops / (per_kernel[dom] / 1e3) / 1e12
        roofline = {"bound": "alu", "kernel": dom, "achieved": round(achieved, 3),
                    "peak": FP32_VEC_PEAK / 1e12, "unit": "TFLOP/s",
                    "frac": round(achieved * 1e12 / FP32_VEC_PEAK, 4), "traffic": None,
                    "flops_per_launch": flops, "avg_launch_ms": round(per_kernel[dom], 4)}
    copy = copy_bandwidth(torch)
    pages_ms = PAGES_FWD_BWD_MS.get(T)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        # the pages' Metal fwd+bwd at this shape and T (another machine: context)
        "vs_baseline": round(value / (tokens / (pages_ms / 1e3)), 2) if pages_ms else None,
        # chunk form: bf16 matrix-core products with fp32 accumulation and an
        # fp32 state; scan form: fp32 throughout
        "dtype": "bf16" if family == "chunk" else "f32",
        "data": "synthetic",
        "config": {"workload": "gated delta rule fwd+bwd, Qwen3.5-9B GDN layer shape",
                   "B": B, "T": T, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
                   "io_dtype": "bf16", "state_dtype": "f32", "algo": family},
        "timing": {"protocol": "per step: 1 GiB scratch write (cache flush), then HIP events around "
                               "gdn_fwd + gdn_bwd; value and ms_per_step from the median",
                   "step_ms": m["step"], "unflushed_mean_ms": m["unflushed_ms"]},
        "roofline": roofline,
        "hbm_roofline_step": {"method_bytes": fb + bb, "achieved_GBps": round(
            (fb + bb) / (ms / 1e3) / 1e9, 1), "peak_GBps": HBM_PEAK / 1e9,
            "frac": round((fb + bb) / (ms / 1e3) / HBM_PEAK, 5),
            "compulsory_bytes": compulsory_bytes(B, T, Hk, Hv, Dk, Dv, 2),
            "compulsory_frac": round(compulsory_bytes(B, T, Hk, Hv, Dk, Dv, 2) / (ms / 1e3) / HBM_PEAK, 5),
            "copy_GBps": copy["GBps"],
            "frac_of_copy": round((fb + bb) / (ms / 1e3) / 1e9 / copy["GBps"], 5)},
        "kernels_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "kernels_ms_range": {k: [v["min"], v["max"]] for k, v in m["kernels"].items()},
        "pages_context": {"metal_fwd_bwd_ms": pages_ms, "hardware": "Apple M4 Max, MLX 0.31.1"}
        if pages_ms else None,
        "wall_s_timed": m["wall_s"],
    }
    if args.config == "9b_t2048" and family == "chunk" and not args.no_sweep:
        # the pages' performance table runs T = 256 ... 2048 at this shape
        sweep = {}
        for Ts in (256, 512, 1024):
            _, _, p2, r2 = train_plan(torch, binding, inputs, Ts, algo)
            m2 = measure(torch, lib, p2.stream, r2, [], 20, 5, flush)
            del p2
            sweep[str(Ts)] = {"ms": m2["step"]["median"],
                              "tokens_per_s": round(Ts / (m2["step"]["median"] / 1e3), 1),
                              "metal_ms": PAGES_FWD_BWD_MS_ALL.get(Ts)}
        sweep["2048"] = {"ms": round(ms, 5), "tokens_per_s": round(value, 1),
                         "metal_ms": PAGES_FWD_BWD_MS_ALL.get(2048)}
        out["t_sweep"] = sweep
    return out


def compulsory_bytes(B, T, Hk, Hv, Dk, Dv, io):
    """method_bytes without the checkpoints: the I/O tensors of fwd and bwd."""
    fb, bb = method_bytes(B, T, Hk, Hv, Dk, Dv, io)
    CK = max(math.ceil(T / 64) - 1, 0) * B * Hv * Dk * Dv * 4
    return fb + bb - 2 * CK


def vg_method_bytes(B, T, Hk, Hv, Dk, Dv, io):
    """method_bytes with the per-channel log-gates (fp32 [B,T,Hv,Dk]) in place
    of a and the parameters, and their gradient in place of da."""
    Q = B * T * Hk * Dk * io
    V = B * T * Hv * Dv * io
    Bt = B * T * Hv * io
    LG = B * T * Hv * Dk * 4
    Sig = B * Hv * Dk * Dv * 4
    CK = max(math.ceil(T / 64) - 1, 0) * Sig
    fwd = 2 * Q + V + LG + Bt + V + Sig + CK
    bwd = (2 * Q + V + LG + Bt + CK + V) + (2 * Q + V + LG + Bt + Sig)
    return fwd, bwd


def vg_kernel_bytes(B, T, Hk, Hv, Dk, Dv, io):
    """Algorithmic HBM bytes of each kernel of the per-channel gate's chunk
    form: the tensors of vg_method_bytes that the kernel reads or writes, each
    counted once per kernel (the pre-scaled rows, chunk matrices, X, eps, dH'
    and the per-head partials are intermediates and not counted; the saved
    record's fp32 states are the method's checkpoints, read by vg_chunk_grad)."""
    Q1 = B * T * Hk * Dk * io
    V1 = B * T * Hv * Dv * io
    Bt = B * T * Hv * io
    LG = B * T * Hv * Dk * 4
    Sig = B * Hv * Dk * Dv * 4
    CK = max(math.ceil(T / 64) - 1, 0) * Sig
    return {
        "vg_prep_fwd": 2 * Q1 + LG + Bt,
        "chunk_fwd_vg": 2 * V1 + Sig + CK,
        "prep_bwd": 2 * Q1 + Bt,
        "chunk_bwd_state_vg": 2 * V1 + Sig,
        "vg_chunk_x": 2 * V1 + Bt,  # dO, dv, b (X from the saved record)
        "vg_chunk_grad": 2 * Q1 + 2 * V1 + 2 * LG + CK,
        "vg_norm_bwd": 4 * Q1,
    }


def cpu_baseline_vg(T):
    """The fp64 oracle of the per-channel-gate form on the same bounded sample
    as cpu_baseline (half of the heads of the 9B shape)."""
    import oracle
    from linear_attention_recurrence_fwd_amd import inputs
    threads = max(1, min(16, os.cpu_count() or 1))
    c = inputs.make_vg_case("vg_9b_sample", 1, T, 8, 32, 192, 128, "bf16", 8000 + T,
                            state_std=None, dS_final=False)
    oracle.fwd_vg(*c.vg_args(), nthreads=threads)
    t0 = time.perf_counter()
    oracle.fwd_vg(*c.vg_args(), nthreads=threads)
    oracle.bwd_vg(*c.vg_args(), c.vals["dO"], None, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(c.B * T / (dt * 2), 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "fp64 oracle fwd+bwd with per-channel gates, B=1 T=%d, Hk=8 Hv=32 Dk=192 "
                      "Dv=128 (1/2 of the heads), %.2f s wall on %d threads; tokens/s scaled by 2"
                      % (T, dt, threads)}


def bench_vg(args, torch, binding, inputs):
    """The 9B layer shape with a per-key-channel gate, fwd + bwd per step
    (timing protocol as bench_train)."""
    T = {"vg_t2048": 2048, "vg_t256": 256}[args.config]
    case = inputs.vg_qwen35_9b(T)
    t = upload_case(torch, case, ("q", "k", "v", "lg", "b", "state0", "dO", "dS_final"))
    t["mask"] = None
    algo = {"auto": binding.ALGO_AUTO, "scan": binding.ALGO_SCAN,
            "chunk": binding.ALGO_CHUNK}[args.algo]
    plan = binding.PlanVg(t, algo=algo, save=True)
    family = plan.family
    kernels = KERNELS["vg" if family == "scan" else "vg_chunk"]
    lib = binding.lib()

    def run():
        plan.fwd()
        plan.bwd()
    m = measure(torch, lib, plan.stream, run, kernels, args.steps, args.warmup, Flush(torch))
    ms = m["step"]["median"]
    per_kernel = {k: v["median"] for k, v in m["kernels"].items()}
    B, Hk, Hv, Dk, Dv = case.B, case.Hk, case.Hv, case.Dk, case.Dv
    tokens = B * T
    value = tokens / (ms / 1e3)
    E = B * T * Hv * Dk * Dv
    dom = max(per_kernel, key=lambda k: per_kernel[k])
    fb, bb = vg_method_bytes(B, T, Hk, Hv, Dk, Dv, 2)
    if family == "scan":
        flops = FLOPS_PER_ELEM.get(dom, 0) * E
        achieved = flops / (per_kernel[dom] / 1e3) / 1e12
        roofline = {"bound": "alu", "kernel": dom, "achieved": round(achieved, 3),
                    "peak": FP32_VEC_PEAK / 1e12, "unit": "TFLOP/s",
                    "frac": round(achieved * 1e12 / FP32_VEC_PEAK, 4), "traffic": None,
                    "flops_per_launch": flops, "avg_launch_ms": round(per_kernel[dom], 4)}
    else:
        kb = vg_kernel_bytes(B, T, Hk, Hv, Dk, Dv, 2)
        achieved = kb[dom] / (per_kernel[dom] / 1e3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                    "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": None,
                    "bytes_per_launch": kb[dom], "avg_launch_ms": round(per_kernel[dom], 4)}
    return {
        "metric": VG_METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if family == "scan" else "bf16",
        "data": "synthetic",
        "config": {"workload": "gated delta rule fwd+bwd with a per-key-channel gate, "
                               "Qwen3.5-9B GDN layer shape",
                   "B": B, "T": T, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
                   "io_dtype": "bf16", "state_dtype": "f32", "algo": family},
        "timing": {"protocol": "per step: 1 GiB scratch write (cache flush), then HIP events around "
                               "gdn_fwd_vg + gdn_bwd_vg; value and ms_per_step from the median",
                   "step_ms": m["step"], "unflushed_mean_ms": m["unflushed_ms"]},
        "roofline": roofline,
        "hbm_roofline_step": {"method_bytes": fb + bb, "achieved_GBps": round(
            (fb + bb) / (ms / 1e3) / 1e9, 1), "peak_GBps": HBM_PEAK / 1e9,
            "frac": round((fb + bb) / (ms / 1e3) / HBM_PEAK, 5)},
        "kernels_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "wall_s_timed": m["wall_s"],
    }


LONG = dict(B=1, T=32768, Hk=2, Hv=4, Dk=128, Dv=128)


def bench_long(args, torch, binding, inputs):
    """A long single sequence with few heads (inference prefill, forward only,
    no checkpoints): the T-parallel chunk forward (segment maps, their chain,
    every segment's outputs) against the single-pass chunk forward.  Slow
    decays (A_log in (-7, -4)) so that the state carries across chunks."""
    L = LONG
    case = inputs.make_case("long_t32k", L["B"], L["T"], L["Hk"], L["Hv"], L["Dk"], L["Dv"], "bf16",
                            11, state_std=None, dS_final=False, A_log_range=(-7.0, -4.0))
    dev = torch.device("cuda:0")

    def up(n):
        import numpy as np
        x = case.store(n)
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)

    t = {n: up(n) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "dO")}
    lib = binding.lib()
    st = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(st.cuda_stream)
    P = binding._p
    out = {}
    for name, algo in (("tpar", binding.ALGO_CHUNK_TPAR), ("single", binding.ALGO_CHUNK)):
        d = binding.make_dims(L["B"], L["T"], L["Hk"], L["Hv"], L["Dk"], L["Dv"], binding.GDN_BF16, algo)
        o = torch.empty((L["B"], L["T"], L["Hv"], L["Dv"]), dtype=torch.bfloat16, device=dev)
        so = torch.empty((L["B"], L["Hv"], L["Dk"], L["Dv"]), dtype=torch.float32, device=dev)
        wsb = binding.fwd_workspace_bytes(d)
        ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)
        fargs = (ctypes.byref(d), P(t["q"]), P(t["k"]), P(t["v"]), P(t["a"]), P(t["b"]), P(t["A_log"]),
                 P(t["dt_bias"]), None, None, P(o), P(so), None, P(ws), wsb, sp)

        def run():
            rc = lib.gdn_fwd(*fargs)
            if rc:
                raise binding.GdnError("gdn_fwd", rc)
        for _ in range(args.warmup):
            run()
        ev = HipEvents(2)
        torch.cuda.synchronize()
        ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[0]), sp)
        for _ in range(args.steps):
            run()
        ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[1]), sp)
        torch.cuda.synchronize()
        ms = ev.elapsed_ms(0, 1) / args.steps
        ev.close()
        kms = None
        if name == "tpar":
            ks = ["chunk_prep", "fill_zero", "chunk_fwd_maps", "seg_chain", "chunk_fwd"]
            ev = HipEvents(2 * len(ks))
            lib.gdn_set_kernel_events(ev.ptr(0), 2 * len(ks))
            run()
            torch.cuda.synchronize()
            lib.gdn_set_kernel_events(None, 0)
            kms = {k: round(ev.elapsed_ms(2 * i, 2 * i + 1), 4) for i, k in enumerate(ks)}
            ev.close()
        # a training step on the same sequence: fwd (saving for the backward) + bwd
        tp = dict(t, state0=None, mask=None, dS_final=None)
        plan = binding.Plan(tp, algo=algo, save=True)
        for _ in range(args.warmup):
            plan.fwd()
            plan.bwd()
        ev = HipEvents(2)
        torch.cuda.synchronize()
        ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[0]), sp)
        for _ in range(args.steps):
            plan.fwd()
            plan.bwd()
        ev.hip.hipEventRecord(ctypes.c_void_p(ev.ev[1]), sp)
        torch.cuda.synchronize()
        train_ms = ev.elapsed_ms(0, 1) / args.steps
        ev.close()
        del plan
        out[name] = (ms, kms, wsb, train_ms)
    B, T, Hk, Hv, Dk, Dv = (L[k] for k in ("B", "T", "Hk", "Hv", "Dk", "Dv"))
    ms, kms, wsb, tr = out["tpar"]
    ms1, tr1 = out["single"][0], out["single"][3]
    # algorithmic HBM bytes of the prefill: q, k, v, a, b, o once, the final state
    byts = (2 * B * T * Hk * Dk + 2 * B * T * Hv * Dv + 2 * B * T * Hv) * 2 + B * Hv * Dk * Dv * 4
    dom = max(kms, key=lambda k: kms[k])
    # per kernel: what it reads and writes of the inputs, outputs and the
    # segment maps / start states (chunk matrices and scalars not counted)
    # segments, from the extra workspace: maps n (Dk + Dv) + starts (n - 1) Dv floats per state row
    x = (wsb - out["single"][2] - 256) / (4 * B * Hv * Dk)
    nseg = max(int(round((x + Dv) / (Dk + 2 * Dv))), 1)
    maps = nseg * B * Hv * Dk * (Dk + Dv) * 4
    starts = (nseg - 1) * B * Hv * Dk * Dv * 4
    kb = {"chunk_prep": (2 * B * T * Hk * Dk + 2 * B * T * Hv) * 2,
          "fill_zero": 256,
          "chunk_fwd_maps": (B * T * Hk * Dk + B * T * Hv * Dv) * 2 + maps,
          "seg_chain": maps + starts,
          "chunk_fwd": (2 * B * T * Hk * Dk + 2 * B * T * Hv * Dv) * 2 + starts + B * Hv * Dk * Dv * 4}
    return {
        "metric": "prefill (forward) tokens/sec of one long sequence, B=1 T=32768 Hk2/Hv4/Dk128/Dv128 bf16",
        "value": round(B * T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gated delta rule forward, one long sequence with few heads, T-parallel "
                               "chunk form", "B": B, "T": T, "Hk": Hk, "Hv": Hv, "Dk": Dk, "Dv": Dv,
                   "io_dtype": "bf16", "algo": "chunk_tpar"},
        "single_pass_ms": round(ms1, 4),
        "speedup_vs_single_pass": round(ms1 / ms, 3),
        "train_step_ms": {"tpar": round(tr, 4), "single_pass": round(tr1, 4),
                          "speedup": round(tr1 / tr, 3)},
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": round(kb[dom] / (kms[dom] / 1e3) / 1e9, 1), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(kb[dom] / (kms[dom] / 1e3) / HBM_PEAK, 4),
                     "traffic": None, "bytes_per_launch": kb[dom], "avg_launch_ms": kms[dom]},
        "hbm_roofline_prefill": {"bytes": byts, "achieved_GBps": round(byts / (ms / 1e3) / 1e9, 1),
                                 "frac": round(byts / (ms / 1e3) / HBM_PEAK, 4)},
        "segments": nseg,
        "kernels_ms": kms,
    }


def bench_decode(args, torch, binding, inputs):
    """Decode workload: B=64, Hk=16, Hv=32, Dk=Dv=128, one token per call, the
    state updated in place; a step is 64 consecutive calls."""
    import numpy as np
    case = inputs.decode(64)
    dev = torch.device("cuda:0")

    def up(n):
        x = case.store(n)
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)

    t = {n: up(n) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state0")}
    calls = [{n: t[n][:, i:i + 1].contiguous() for n in ("q", "k", "v", "a", "b")}
             for i in range(case.T)]
    state = t["state0"].clone()
    d = binding.make_dims(case.B, 1, case.Hk, case.Hv, case.Dk, case.Dv, torch.bfloat16)
    wsb = binding.fwd_workspace_bytes(d)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)
    outs = [torch.empty((case.B, 1, case.Hv, case.Dv), dtype=torch.bfloat16, device=dev)
            for _ in range(case.T)]
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = binding._p
    argl = [(ctypes.byref(d), P(c["q"]), P(c["k"]), P(c["v"]), P(c["a"]), P(c["b"]),
             P(t["A_log"]), P(t["dt_bias"]), P(state), None, P(o), P(state), None, P(ws), wsb, sp)
            for c, o in zip(calls, outs)]
    lib = binding.lib()
    calls_t = time_calls(torch, lib.gdn_fwd, argl, args.steps, args.warmup, Flush(torch))
    per_call = calls_t["flushed_call_ms"]["median"]
    ms = per_call * case.T
    Sig = case.B * case.Hv * case.Dk * case.Dv * 4
    io = case.B * (2 * case.Hk * case.Dk + 2 * case.Hv * case.Dv + 2 * case.Hv) * 2 + 2 * case.Hv * 4
    call_bytes = 2 * Sig + io
    frac = call_bytes / (per_call / 1e3) / HBM_PEAK
    return {
        "metric": "decode tokens/sec, B=64 Hk16/Hv32/Dk128/Dv128, 1 token per call",
        "value": round(case.B / (per_call / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "timing": dict(calls_t, protocol="per call: 1 GiB scratch write (cache flush), then HIP "
                                         "events around the call; value from the median; unflushed: "
                                         "the steps' calls back to back (the 134 MB state may stay "
                                         "in the 256 MB memory-side cache)"),
        "unflushed_frac": round(call_bytes / (calls_t["unflushed_call_ms"] / 1e3) / HBM_PEAK, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gated delta rule decode, 64 single-token calls per step",
                   "B": case.B, "Hk": case.Hk, "Hv": case.Hv, "Dk": case.Dk, "Dv": case.Dv,
                   "io_dtype": "bf16"},
        "roofline": {"bound": "hbm", "kernel": "decode (one call)",
                     "achieved": round(call_bytes / (per_call / 1e3) / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(frac, 4),
                     "traffic": None, "bytes_per_launch": call_bytes,
                     "median_call_ms": round(per_call, 5)},
    }


def bench_decode_conv(args, torch, binding, inputs):
    """Decode workload with the conv update (gdn_decode_conv): B=64, Hk=16,
    Hv=32, Dk=Dv=128, 4 taps, one token per call, the conv state and the state
    updated in place; a step is 64 consecutive calls."""
    import numpy as np
    case = inputs.decode_conv(64)
    dev = torch.device("cuda:0")

    def up(n):
        x = case.store(n)
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)

    t = {n: up(n) for n in ("x", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state0")}
    calls = [{n: t[n][:, i].contiguous() for n in ("x", "a", "b")} for i in range(case.steps)]
    state, cstate = t["state0"].clone(), t["conv_state"].clone()
    d = binding.make_dims(case.B, 1, case.Hk, case.Hv, case.Dk, case.Dv, torch.bfloat16)
    outs = [torch.empty((case.B, case.Hv, case.Dv), dtype=torch.bfloat16, device=dev) for _ in range(case.steps)]
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = binding._p
    argl = [(ctypes.byref(d), P(c["x"]), P(t["conv_w"]), P(cstate), P(cstate), case.K, P(c["a"]), P(c["b"]),
             P(t["A_log"]), P(t["dt_bias"]), P(state), None, P(o), P(state), sp)
            for c, o in zip(calls, outs)]
    lib = binding.lib()
    calls_t = time_calls(torch, lib.gdn_decode_conv, argl, args.steps, args.warmup, Flush(torch))
    per_call = calls_t["flushed_call_ms"]["median"]
    ms = per_call * case.steps
    Sig = case.B * case.Hv * case.Dk * case.Dv * 4
    # state read + written; conv state read + written, x, taps, a, b, o (bf16); A_log, dt_bias
    io = (2 * case.B * case.C * case.K + case.B * case.C + case.C * case.K + 2 * case.B * case.Hv
          + case.B * case.Hv * case.Dv) * 2 + 2 * case.Hv * 4
    call_bytes = 2 * Sig + io
    frac = call_bytes / (per_call / 1e3) / HBM_PEAK
    return {
        "metric": "decode tokens/sec with the conv update, B=64 Hk16/Hv32/Dk128/Dv128, 4 taps, 1 token per call",
        "value": round(case.B / (per_call / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "timing": dict(calls_t, protocol="per call: 1 GiB scratch write (cache flush), then HIP "
                                         "events around the call; value from the median; unflushed: "
                                         "the steps' calls back to back"),
        "unflushed_frac": round(call_bytes / (calls_t["unflushed_call_ms"] / 1e3) / HBM_PEAK, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gated delta rule decode with conv1d + SiLU update, 64 single-token calls per step",
                   "B": case.B, "Hk": case.Hk, "Hv": case.Hv, "Dk": case.Dk, "Dv": case.Dv, "conv_taps": case.K,
                   "io_dtype": "bf16"},
        "roofline": {"bound": "hbm", "kernel": "decode_conv (one call)",
                     "achieved": round(call_bytes / (per_call / 1e3) / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(frac, 4),
                     "traffic": None, "bytes_per_launch": call_bytes,
                     "median_call_ms": round(per_call, 5)},
    }


def copy_probe(torch, mib):
    """A plain device-to-device copy of `mib` MiB, three times: under
    `rocprofv3 --pmc FETCH_SIZE` (or WRITE_SIZE) its per-dispatch reading is
    the counter's value for a known number of bytes read (or written)."""
    n = mib << 20
    src = torch.empty((n,), dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copy probe: %d bytes per copy, 3 copies" % n, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="9b_t2048",
                    choices=["9b_t2048", "9b_t256", "decode", "decode_conv", "vg_t2048", "vg_t256",
                             "long_t32k"])
    ap.add_argument("--algo", default="auto", choices=["auto", "scan", "chunk"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the T = 256, 512, 1024 sweep of the default workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB device to device 3 times "
                         "(the known-size reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the operation shards by (batch, key-head group) with no exchange); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from linear_attention_recurrence_fwd_amd import binding, inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.lib()
    if args.config == "decode":
        out = bench_decode(args, torch, binding, inputs)
    elif args.config == "decode_conv":
        out = bench_decode_conv(args, torch, binding, inputs)
    elif args.config == "long_t32k":
        out = bench_long(args, torch, binding, inputs)
    elif args.config.startswith("vg_"):
        out = bench_vg(args, torch, binding, inputs)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_vg(out["config"]["T"])
    else:
        out = bench_train(args, torch, binding, inputs)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(out["config"]["T"])
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Shared helpers for the GPU parity tests: upload a seeded case, run the
library through its C ABI binding, run the oracle, compare."""
import sys

import numpy as np
import torch

import oracle
from linear_attention_recurrence_fwd_amd import binding

TOL = {"f32": 1e-4, "bf16": 2e-2}
GRADS = ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias", "dstate")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(case, name, device="cuda"):
    x = case.store(name)
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def upload(case, device="cuda"):
    t = {n: dev_tensor(case, n, device) for n in
         ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state0", "dO", "dS_final")}
    t["mask"] = None if case.mask is None else torch.from_numpy(case.mask).to(device)
    return t


def to64(x):
    return x.detach().to(torch.float64).cpu().numpy()


def relerr(x, ref):
    """max |x - ref| / max |ref|  (max |x| when ref is all zero)."""
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(num / den)


def elemerr(x, ref, floor=0.1):
    """Elementwise companion of relerr: the 99.9th percentile and the maximum
    of |x - ref| / (|ref| + floor * rms(ref)) (an absolute floor at a tenth of
    the tensor's typical magnitude keeps entries near zero, whose relative
    error says nothing, from dominating)."""
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0, 0.0
    scale = float(np.sqrt(np.mean(ref * ref)))
    if scale == 0.0:
        m = float(np.max(np.abs(x)))
        return m, m
    r = np.abs(x - ref) / (np.abs(ref) + floor * scale)
    return float(np.quantile(r, 0.999)), float(np.max(r))


def report(tag, pairs):
    """Print normwise and elementwise errors of (name, x, ref) triples and
    return the normwise ones."""
    errs, lines = {}, []
    for n, x, ref in pairs:
        errs[n] = relerr(x, ref)
        p999, mx = elemerr(x, ref)
        lines.append("%s=%.2e (elem p99.9 %.2e max %.2e)" % (n, errs[n], p999, mx))
    say("[%s] normwise (elementwise) errors: %s" % (tag, " ".join(lines)))
    return errs


def gpu_fwd(t, algo=binding.ALGO_AUTO, need_ckpt=True, save=False):
    return binding.fwd(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                       t["state0"], t["mask"], need_ckpt=need_ckpt, algo=algo, save=save)


def gpu_bwd(t, ckpt, algo=binding.ALGO_AUTO, save=False):
    return binding.bwd(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                       t["state0"], t["mask"], ckpt, t["dO"], t["dS_final"], algo=algo, save=save)


def oracle_all(case, nthreads=8):
    v = case.vals
    o, st, ck = oracle.fwd(*case.oracle_args(), nthreads=nthreads)
    g = oracle.bwd(*case.oracle_args(), v["dO"], v.get("dS_final"), nthreads=nthreads)
    return o, st, ck, g

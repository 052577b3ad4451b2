"""fp64 CPU oracle for the gated delta rule forward scan and its VJP.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The GPU library never
imports, links or executes anything here, and nothing here calls the GPU
library.

The arithmetic lives in ``gdn_oracle.c`` (plain sequential C, fp64, no fast
math, no FMA contraction); this module only builds it with gcc and marshals
numpy float64 arrays through ctypes.  See the C file's header for the
definition it follows (mlx-lm PR "Add gated_delta_update VJP", sections "What
this PR adds" / "Design notes"; torch-to-nnef GDN page, "Op contract").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.environ.get("GDN_ORACLE_LIB") or os.path.join(_HERE, "liboracle_gdn.so")
CKPT = 64
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``liboracle_gdn.so`` (in place)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "T", "Hk", "Hv", "Dk", "Dv")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.oracle_gdn_fwd.argtypes = [ctypes.POINTER(_Dims)] + [P] * 12 + [ctypes.c_int]
        lib.oracle_gdn_fwd.restype = ctypes.c_int
        lib.oracle_gdn_bwd.argtypes = ([ctypes.POINTER(_Dims)] + [P] * 19
                                       + [ctypes.c_int64, ctypes.c_int])
        lib.oracle_gdn_bwd.restype = ctypes.c_int
        D = ctypes.c_double
        PD = ctypes.POINTER(ctypes.c_double)
        lib.oracle_gates.argtypes = [D, D, D, D, PD, PD, PD]
        lib.oracle_gates.restype = None
        lib.oracle_gdn_fwd_vg.argtypes = [ctypes.POINTER(_Dims)] + [P] * 10 + [ctypes.c_int]
        lib.oracle_gdn_fwd_vg.restype = ctypes.c_int
        lib.oracle_gdn_bwd_vg.argtypes = ([ctypes.POINTER(_Dims)] + [P] * 15
                                          + [ctypes.c_int64, ctypes.c_int])
        lib.oracle_gdn_bwd_vg.restype = ctypes.c_int
        I64 = ctypes.c_int64
        lib.oracle_conv_update.argtypes = [I64, I64, I64, I64] + [P] * 5
        lib.oracle_conv_update.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _dims(q, v):
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    return _Dims(B, T, Hk, Hv, Dk, Dv)


def _mask_u8(mask, B, T):
    if mask is None:
        return None
    m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    assert m.shape == (B, T)
    return m


def gates(a: float, b: float, A_log: float, dt_bias: float):
    """(g, log g, beta) of one step, as the oracle computes them."""
    lib = _load()
    g, ell, beta = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    lib.oracle_gates(a, b, A_log, dt_bias, ctypes.byref(g), ctypes.byref(ell),
                     ctypes.byref(beta))
    return g.value, ell.value, beta.value


def fwd(q, k, v, a, b, A_log, dt_bias, state0=None, mask=None, nthreads=1):
    """Forward scan.  Returns (o, state_out, ckpt) as float64 arrays.

    q, k: [B,T,Hk,Dk]; v: [B,T,Hv,Dv]; a, b: [B,T,Hv]; A_log, dt_bias: [Hv];
    state0: [B,Hv,Dk,Dv] or None (zeros); mask: [B,T] (nonzero = valid) or
    None.  ckpt: [ceil(T/64)-1, B, Hv, Dk, Dv], the states at t = 64, 128, ...
    """
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    A_log, dt_bias, state0 = map(_f64, (A_log, dt_bias, state0))
    d = _dims(q, v)
    m = _mask_u8(mask, d.B, d.T)
    nck = max((d.T + CKPT - 1) // CKPT - 1, 0)
    o = np.empty((d.B, d.T, d.Hv, d.Dv))
    st = np.empty((d.B, d.Hv, d.Dk, d.Dv))
    ck = np.empty((nck, d.B, d.Hv, d.Dk, d.Dv))
    rc = _load().oracle_gdn_fwd(ctypes.byref(d), *map(_ptr, (q, k, v, a, b, A_log, dt_bias, state0)),
                                _ptr(m), _ptr(o), _ptr(st), _ptr(ck) if nck else None,
                                int(nthreads))
    if rc:
        raise RuntimeError("oracle_gdn_fwd failed with code %d" % rc)
    return o, st, ck


def bwd(q, k, v, a, b, A_log, dt_bias, state0, mask, dO, dS_final=None,
        chunk=CKPT, nthreads=1):
    """Reverse sweep.  Returns a dict with dq, dk, dv, da, db, dA_log,
    ddt_bias, dstate (float64).  chunk=0 keeps every state; chunk>0 keeps one
    every `chunk` steps and recomputes inside (same result bit for bit)."""
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    A_log, dt_bias, state0, dO, dS_final = map(_f64, (A_log, dt_bias, state0, dO, dS_final))
    d = _dims(q, v)
    m = _mask_u8(mask, d.B, d.T)
    out = dict(dq=np.empty_like(q), dk=np.empty_like(k), dv=np.empty_like(v),
               da=np.empty_like(a), db=np.empty_like(b),
               dA_log=np.empty((d.Hv,)), ddt_bias=np.empty((d.Hv,)),
               dstate=np.empty((d.B, d.Hv, d.Dk, d.Dv)))
    rc = _load().oracle_gdn_bwd(
        ctypes.byref(d), *map(_ptr, (q, k, v, a, b, A_log, dt_bias, state0)), _ptr(m),
        _ptr(dO), _ptr(dS_final),
        *[_ptr(out[n]) for n in ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias", "dstate")],
        int(chunk), int(nthreads))
    if rc:
        raise RuntimeError("oracle_gdn_bwd failed with code %d" % rc)
    return out


def fwd_vg(q, k, v, lg, b, state0=None, mask=None, nthreads=1):
    """Forward scan with a per-key-channel gate (see oracle_gdn_fwd_vg).

    lg: [B,T,Hv,Dk] log-gates (g = exp(lg) scales the state's rows); b:
    [B,T,Hv] (beta = sigmoid(b)); the rest as ``fwd``.  Returns (o,
    state_out, ckpt)."""
    q, k, v, lg, b, state0 = map(_f64, (q, k, v, lg, b, state0))
    d = _dims(q, v)
    assert lg.shape == (d.B, d.T, d.Hv, d.Dk)
    m = _mask_u8(mask, d.B, d.T)
    nck = max((d.T + CKPT - 1) // CKPT - 1, 0)
    o = np.empty((d.B, d.T, d.Hv, d.Dv))
    st = np.empty((d.B, d.Hv, d.Dk, d.Dv))
    ck = np.empty((nck, d.B, d.Hv, d.Dk, d.Dv))
    rc = _load().oracle_gdn_fwd_vg(ctypes.byref(d), *map(_ptr, (q, k, v, lg, b, state0)), _ptr(m),
                                   _ptr(o), _ptr(st), _ptr(ck) if nck else None, int(nthreads))
    if rc:
        raise RuntimeError("oracle_gdn_fwd_vg failed with code %d" % rc)
    return o, st, ck


def bwd_vg(q, k, v, lg, b, state0, mask, dO, dS_final=None, chunk=CKPT, nthreads=1):
    """Reverse sweep of ``fwd_vg``.  Returns a dict with dq, dk, dv, dlg,
    db, dstate (float64); chunk as in ``bwd``."""
    q, k, v, lg, b, state0, dO, dS_final = map(_f64, (q, k, v, lg, b, state0, dO, dS_final))
    d = _dims(q, v)
    m = _mask_u8(mask, d.B, d.T)
    out = dict(dq=np.empty_like(q), dk=np.empty_like(k), dv=np.empty_like(v),
               dlg=np.empty_like(lg), db=np.empty_like(b),
               dstate=np.empty((d.B, d.Hv, d.Dk, d.Dv)))
    rc = _load().oracle_gdn_bwd_vg(
        ctypes.byref(d), *map(_ptr, (q, k, v, lg, b, state0)), _ptr(m), _ptr(dO), _ptr(dS_final),
        *[_ptr(out[n]) for n in ("dq", "dk", "dv", "dlg", "db", "dstate")],
        int(chunk), int(nthreads))
    if rc:
        raise RuntimeError("oracle_gdn_bwd_vg failed with code %d" % rc)
    return out


def conv_update(x, state, w):
    """Depthwise causal conv1d + SiLU update (see oracle_conv_update).

    x: [B, C, S] new samples; state: [B, C, K] carried samples (oldest first);
    w: [C, K] taps.  Returns (out [B, C, S], final_state [B, C, K]) as float64.
    """
    x, state, w = map(_f64, (x, state, w))
    B, C, S = x.shape
    K = w.shape[1]
    assert state.shape == (B, C, K) and w.shape == (C, K)
    out = np.empty((B, C, S))
    fin = np.empty((B, C, K))
    rc = _load().oracle_conv_update(B, C, K, S, *map(_ptr, (x, state, w, out, fin)))
    if rc:
        raise RuntimeError("oracle_conv_update failed with code %d" % rc)
    return out, fin


def decode_conv(x, conv_state, conv_w, a, b, A_log, dt_bias, Hk, Dk, Hv, Dv, state0=None, mask=None):
    """One decode step with the preceding conv update: the conv update of the
    token's mixed projection x [B, C] (C = 2 Hk Dk + Hv Dv channels, in the
    order q, k, v, each head-major), then the recurrence step (fwd with T = 1)
    on the q, k, v it yields.  A masked batch row (mask[b] == 0) keeps its conv
    state as well as its recurrent state.  a, b: [B, Hv]; mask: [B] or None.
    Returns (o [B, Hv, Dv], state_out [B, Hv, Dk, Dv], conv_state_out [B, C, K]).
    """
    x = _f64(x)
    B, C = x.shape
    assert C == 2 * Hk * Dk + Hv * Dv
    out, fin = conv_update(x[:, :, None], conv_state, conv_w)
    out = out[:, :, 0]
    if mask is not None:
        keep = np.asarray(mask).reshape(B) == 0
        fin[keep] = _f64(conv_state)[keep]
    q = out[:, :Hk * Dk].reshape(B, 1, Hk, Dk)
    k = out[:, Hk * Dk:2 * Hk * Dk].reshape(B, 1, Hk, Dk)
    v = out[:, 2 * Hk * Dk:].reshape(B, 1, Hv, Dv)
    m = None if mask is None else np.asarray(mask).reshape(B, 1)
    o, st, _ = fwd(q, k, v, _f64(a).reshape(B, 1, Hv), _f64(b).reshape(B, 1, Hv), A_log, dt_bias,
                   state0=state0, mask=m)
    return o[:, 0], st, fin

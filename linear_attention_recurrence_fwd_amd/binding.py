"""ctypes binding of libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: this module checks dtypes/shapes, allocates the
outputs and the workspace with torch (device memory), and passes raw pointers
plus the current HIP stream to the library.  Every step of the computation runs
in the library's kernels.  There is no fallback: if libgdn.so is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
CHUNK = 64

GDN_F32, GDN_BF16 = 0, 1
ALGO_AUTO, ALGO_SCAN, ALGO_CHUNK, ALGO_CHUNK_TPAR = 0, 1, 2, 3
STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED",
          3: "GDN_ERR_WORKSPACE", 4: "GDN_ERR_HIP"}

# every entry point declared in include/gdn.h
EXPORTS = ("gdn_ckpt_elems", "gdn_ckpt_bytes", "gdn_workspace_bytes", "gdn_fwd_workspace_bytes", "gdn_bwd_workspace_bytes",
           "gdn_fwd", "gdn_fwd_noalloc", "gdn_bwd", "gdn_decode_conv", "gdn_vg_ckpt_elems", "gdn_vg_ckpt_bytes",
           "gdn_fwd_vg_workspace_bytes",
           "gdn_bwd_vg_workspace_bytes", "gdn_fwd_vg", "gdn_bwd_vg", "gdn_set_kernel_events",
           "gdn_status_string", "gdn_version")


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("Hk", ctypes.c_int64),
                ("Hv", ctypes.c_int64), ("Dk", ctypes.c_int64), ("Dv", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("algo", ctypes.c_int32), ("save", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(code, code),
                                                 lib().gdn_status_string(code).decode()))


_lib = None


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn.so not built (run __graft_entry__.build()): %s" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        PD = ctypes.POINTER(Dims)
        for n in ("gdn_ckpt_elems", "gdn_fwd_workspace_bytes", "gdn_bwd_workspace_bytes", "gdn_vg_ckpt_elems",
                  "gdn_vg_ckpt_bytes", "gdn_fwd_vg_workspace_bytes", "gdn_bwd_vg_workspace_bytes"):
            getattr(L, n).argtypes = [PD, ctypes.POINTER(S)]
            getattr(L, n).restype = ctypes.c_int
        L.gdn_ckpt_bytes.argtypes = [PD, ctypes.POINTER(S)]
        L.gdn_ckpt_bytes.restype = ctypes.c_int
        L.gdn_workspace_bytes.argtypes = [PD, ctypes.c_int, ctypes.POINTER(S)]
        L.gdn_workspace_bytes.restype = ctypes.c_int
        L.gdn_fwd.argtypes = [PD] + [P] * 13 + [S, P]
        L.gdn_fwd.restype = ctypes.c_int
        L.gdn_fwd_noalloc.argtypes = [PD] + [P] * 13
        L.gdn_fwd_noalloc.restype = ctypes.c_int
        L.gdn_bwd.argtypes = [PD] + [P] * 21 + [S, P]
        L.gdn_bwd.restype = ctypes.c_int
        L.gdn_decode_conv.argtypes = [PD] + [P] * 4 + [ctypes.c_int32] + [P] * 9
        L.gdn_decode_conv.restype = ctypes.c_int
        L.gdn_fwd_vg.argtypes = [PD] + [P] * 11 + [S, P]
        L.gdn_fwd_vg.restype = ctypes.c_int
        L.gdn_bwd_vg.argtypes = [PD] + [P] * 17 + [S, P]
        L.gdn_bwd_vg.restype = ctypes.c_int
        L.gdn_set_kernel_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
        L.gdn_set_kernel_events.restype = ctypes.c_int
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_version.argtypes = []
        L.gdn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_dims(B, T, Hk, Hv, Dk, Dv, dtype, algo=ALGO_AUTO, save=False) -> Dims:
    dt = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}.get(dtype, dtype)
    return Dims(B, T, Hk, Hv, Dk, Dv, dt, algo, 1 if save else 0)


def _query(fn, d: Dims) -> int:
    out = ctypes.c_size_t(0)
    rc = getattr(lib(), fn)(ctypes.byref(d), ctypes.byref(out))
    if rc:
        raise GdnError(fn, rc)
    return out.value


def ckpt_elems(d: Dims) -> int:
    return _query("gdn_ckpt_elems", d)


def vg_ckpt_elems(d: Dims) -> int:
    return _query("gdn_vg_ckpt_elems", d)


def fwd_workspace_bytes(d: Dims) -> int:
    return _query("gdn_fwd_workspace_bytes", d)


def bwd_workspace_bytes(d: Dims) -> int:
    return _query("gdn_bwd_workspace_bytes", d)


def _p(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _check(x, name, shape, dtype, device):
    if x.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, x.dtype))
    if tuple(x.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(x.shape)))
    if x.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, x.device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dims_of(q, v, algo, save=False):
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    return make_dims(B, T, Hk, Hv, Dk, Dv, q.dtype, algo, save)


def _alloc_ckpt(d, dev, vg=False):
    """The checkpoint buffer: [ceil(T/64)-1, B, Hv, Dk, Dv] fp32, or, when the
    dims save (chunk family), a flat buffer of gdn_ckpt_elems (vg:
    gdn_vg_ckpt_elems) fp32 elements with contents private to the library."""
    nslab = max((d.T + CHUNK - 1) // CHUNK - 1, 0)
    nck = vg_ckpt_elems(d) if vg else ckpt_elems(d)
    if nck == nslab * d.B * d.Hv * d.Dk * d.Dv:
        return torch.empty((nslab, d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev)
    return torch.empty((nck,), dtype=torch.float32, device=dev)


def _check_inputs(d, q, k, v, a, b, A_log, dt_bias, state0, mask):
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("gdn runs on the GPU; got device %s" % dev)
    B, T, Hk, Hv, Dk, Dv = d.B, d.T, d.Hk, d.Hv, d.Dk, d.Dv
    _check(q, "q", (B, T, Hk, Dk), dt, dev)
    _check(k, "k", (B, T, Hk, Dk), dt, dev)
    _check(v, "v", (B, T, Hv, Dv), dt, dev)
    _check(a, "a", (B, T, Hv), dt, dev)
    _check(b, "b", (B, T, Hv), dt, dev)
    _check(A_log, "A_log", (Hv,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (Hv,), torch.float32, dev)
    if state0 is not None:
        _check(state0, "state0", (B, Hv, Dk, Dv), torch.float32, dev)
    if mask is not None:
        _check(mask, "mask", (B, T), torch.uint8, dev)


def fwd(q, k, v, a, b, A_log, dt_bias, state0=None, mask=None, *, need_ckpt=True,
        state_out=None, algo=ALGO_AUTO, save=False):
    """Forward scan.  Returns (o, state_out, ckpt); ckpt is None when not
    requested.  Pass state_out=state0 for an in-place state update.  With
    save=True the chunk form writes what the backward needs (bf16 chunk-start
    states, chunk matrices) into the checkpoint buffer instead of fp32 states
    (pass the same save to bwd)."""
    d = _dims_of(q, v, algo, save)
    if save and not need_ckpt:
        raise ValueError("save=True needs the checkpoint buffer (need_ckpt=True)")
    _check_inputs(d, q, k, v, a, b, A_log, dt_bias, state0, mask)
    dev = q.device
    o = torch.empty((d.B, d.T, d.Hv, d.Dv), dtype=q.dtype, device=dev)
    if state_out is None:
        state_out = torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev)
    else:
        _check(state_out, "state_out", (d.B, d.Hv, d.Dk, d.Dv), torch.float32, dev)
    nck = ckpt_elems(d)
    ckpt = _alloc_ckpt(d, dev) if need_ckpt else None
    wsb = fwd_workspace_bytes(d)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)
    rc = lib().gdn_fwd(ctypes.byref(d), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log), _p(dt_bias),
                       _p(state0), _p(mask), _p(o), _p(state_out),
                       _p(ckpt) if (ckpt is not None and nck) else None,
                       _p(ws), wsb, _stream(dev))
    if rc:
        raise GdnError("gdn_fwd", rc)
    return o, state_out, ckpt


NOALLOC_SCRATCH_BYTES = 64 << 20  # GDN_NOALLOC_SCRATCH_BYTES


def fwd_noalloc(q, k, v, a, b, A_log, dt_bias, state0=None, mask=None, *, o, state_out, ckpt=None,
                algo=ALGO_AUTO, save=False):
    """gdn_fwd_noalloc: the forward with the library's static workspace.  The
    caller passes every output (o, state_out and, when wanted, ckpt); nothing
    is allocated here or in the library."""
    d = _dims_of(q, v, algo, save)
    _check_inputs(d, q, k, v, a, b, A_log, dt_bias, state0, mask)
    dev = q.device
    _check(o, "o", (d.B, d.T, d.Hv, d.Dv), q.dtype, dev)
    _check(state_out, "state_out", (d.B, d.Hv, d.Dk, d.Dv), torch.float32, dev)
    nck = ckpt_elems(d)
    if ckpt is not None and ckpt.numel() != nck:
        raise ValueError("ckpt must have %d elements" % nck)
    rc = lib().gdn_fwd_noalloc(ctypes.byref(d), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log),
                               _p(dt_bias), _p(state0), _p(mask), _p(o), _p(state_out),
                               _p(ckpt) if (ckpt is not None and nck) else None, _stream(dev))
    if rc:
        raise GdnError("gdn_fwd_noalloc", rc)
    return o, state_out, ckpt


def bwd(q, k, v, a, b, A_log, dt_bias, state0, mask, ckpt, dO, dS_final=None, *,
        algo=ALGO_AUTO, save=False):
    """VJP.  Returns dict(dq, dk, dv, da, db, dA_log, ddt_bias, dstate).
    `save` must match the fwd call that wrote ckpt."""
    d = _dims_of(q, v, algo, save)
    _check_inputs(d, q, k, v, a, b, A_log, dt_bias, state0, mask)
    dev = q.device
    _check(dO, "dO", (d.B, d.T, d.Hv, d.Dv), q.dtype, dev)
    if dS_final is not None:
        _check(dS_final, "dS_final", (d.B, d.Hv, d.Dk, d.Dv), torch.float32, dev)
    nck = ckpt_elems(d)
    if nck:
        if ckpt is None or ckpt.numel() != nck:
            raise ValueError("ckpt from gdn_fwd with %d elements is required" % nck)
        if ckpt.dtype != torch.float32 or not ckpt.is_contiguous() or ckpt.device != dev:
            raise ValueError("ckpt must be a contiguous fp32 tensor on %s" % dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               da=torch.empty_like(a), db=torch.empty_like(b),
               dA_log=torch.empty((d.Hv,), dtype=torch.float32, device=dev),
               ddt_bias=torch.empty((d.Hv,), dtype=torch.float32, device=dev),
               dstate=torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev))
    wsb = bwd_workspace_bytes(d)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)
    rc = lib().gdn_bwd(ctypes.byref(d), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log), _p(dt_bias),
                       _p(state0), _p(mask), _p(ckpt) if nck else None, _p(dO), _p(dS_final),
                       *[_p(out[n]) for n in ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias",
                                              "dstate")],
                       _p(ws), wsb, _stream(dev))
    if rc:
        raise GdnError("gdn_bwd", rc)
    return out


class GatedDeltaRule(torch.autograd.Function):
    """Autograd wrapper: forward returns (o, state_out); backward calls gdn_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, a, b, A_log, dt_bias, state0, mask=None):
        o, st, ck = fwd(q, k, v, a, b, A_log, dt_bias, state0, mask, save=True)
        ctx.save_for_backward(q, k, v, a, b, A_log, dt_bias, state0, mask, ck)
        return o, st

    @staticmethod
    def backward(ctx, dO, dS):
        q, k, v, a, b, A_log, dt_bias, state0, mask, ck = ctx.saved_tensors
        g = bwd(q, k, v, a, b, A_log, dt_bias, state0, mask, ck, dO.contiguous(),
                None if dS is None else dS.contiguous(), save=True)
        return (g["dq"], g["dk"], g["dv"], g["da"], g["db"], g["dA_log"], g["ddt_bias"],
                g["dstate"] if state0 is not None else None, None)


class Plan:
    """Repeated fwd + bwd on fixed device tensors with every output and
    workspace allocated once and the ctypes argument lists built once, so a
    call costs one C-ABI call (used by the benchmark's timed loop).

    `t` maps q, k, v, a, b, A_log, dt_bias, state0, mask, dO, dS_final to
    device tensors (state0, mask, dS_final may be None).  save: the forward
    saves the bf16 states and chunk matrices for the backward (as in
    training)."""

    def __init__(self, t, algo=ALGO_AUTO, stream=None, save=True):
        q, v = t["q"], t["v"]
        self.d = d = _dims_of(q, v, algo, save)
        _check_inputs(d, q, k=t["k"], v=v, a=t["a"], b=t["b"], A_log=t["A_log"],
                      dt_bias=t["dt_bias"], state0=t["state0"], mask=t["mask"])
        dev = q.device
        self.t = t
        self.o = torch.empty((d.B, d.T, d.Hv, d.Dv), dtype=q.dtype, device=dev)
        self.state_out = torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev)
        self.ckpt = _alloc_ckpt(d, dev)
        nck = self.ckpt.numel()
        self.g = dict(dq=torch.empty_like(q), dk=torch.empty_like(t["k"]), dv=torch.empty_like(v),
                      da=torch.empty_like(t["a"]), db=torch.empty_like(t["b"]),
                      dA_log=torch.empty((d.Hv,), dtype=torch.float32, device=dev),
                      ddt_bias=torch.empty((d.Hv,), dtype=torch.float32, device=dev),
                      dstate=torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev))
        fws, bws = fwd_workspace_bytes(d), bwd_workspace_bytes(d)
        self.ws_f = torch.empty((max(fws, 1),), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty((max(bws, 1),), dtype=torch.uint8, device=dev)
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        self.stream = st
        sp = ctypes.c_void_p(st.cuda_stream)
        ck = _p(self.ckpt) if nck else None
        ins = [_p(t[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state0", "mask")]
        self._fargs = (ctypes.byref(d), *ins, _p(self.o), _p(self.state_out), ck,
                       _p(self.ws_f), fws, sp)
        self._bargs = (ctypes.byref(d), *ins, ck, _p(t["dO"]), _p(t["dS_final"]),
                       *[_p(self.g[n]) for n in ("dq", "dk", "dv", "da", "db", "dA_log",
                                                 "ddt_bias", "dstate")],
                       _p(self.ws_b), bws, sp)
        self.fwd_ws_bytes, self.bwd_ws_bytes = fws, bws

    def fwd(self):
        rc = lib().gdn_fwd(*self._fargs)
        if rc:
            raise GdnError("gdn_fwd", rc)

    def bwd(self):
        rc = lib().gdn_bwd(*self._bargs)
        if rc:
            raise GdnError("gdn_bwd", rc)


# ---- per-key-channel gate (gdn_fwd_vg / gdn_bwd_vg)

def _check_inputs_vg(d, q, k, v, lg, b, state0, mask):
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("gdn runs on the GPU; got device %s" % dev)
    B, T, Hk, Hv, Dk, Dv = d.B, d.T, d.Hk, d.Hv, d.Dk, d.Dv
    _check(q, "q", (B, T, Hk, Dk), dt, dev)
    _check(k, "k", (B, T, Hk, Dk), dt, dev)
    _check(v, "v", (B, T, Hv, Dv), dt, dev)
    _check(lg, "lg", (B, T, Hv, Dk), torch.float32, dev)
    _check(b, "b", (B, T, Hv), dt, dev)
    if state0 is not None:
        _check(state0, "state0", (B, Hv, Dk, Dv), torch.float32, dev)
    if mask is not None:
        _check(mask, "mask", (B, T), torch.uint8, dev)


def vg_uses_chunk(d) -> bool:
    """Whether gdn_fwd_vg / gdn_bwd_vg run the chunk form for these dims (the
    library's rule: bf16, Dk 64 / 128 / 192, Dv a multiple of 32 up to 128,
    under AUTO more than one step, and the chunk buffers within 4 GiB)."""
    if d.T == 0 or d.algo == ALGO_SCAN:
        return False
    ok = (d.dtype == GDN_BF16 and d.Dk in (64, 128, 192) and d.Dv % 32 == 0 and d.Dv <= 128)
    bhc = d.B * d.Hv * ((d.T + 63) // 64)
    ok = ok and max(bhc * 64 * d.Dk * 2, bhc * 64 * 64 * 2, bhc * 8 * 64 * 4) < 1 << 32
    return d.algo == ALGO_CHUNK or (d.T > 1 and ok)


def fwd_vg(q, k, v, lg, b, state0=None, mask=None, *, need_ckpt=True, state_out=None,
           algo=ALGO_AUTO, save=False):
    """Forward with a per-key-channel gate: lg [B,T,Hv,Dk] fp32 holds log g,
    and g scales the state's rows.  Returns (o, state_out, ckpt).  With
    save=True the chunk form writes the backward's rows, matrices and X into
    ckpt (pass the same save to bwd_vg)."""
    d = _dims_of(q, v, algo, save)
    if save and not need_ckpt:
        raise ValueError("save=True needs the checkpoint buffer (need_ckpt=True)")
    _check_inputs_vg(d, q, k, v, lg, b, state0, mask)
    dev = q.device
    o = torch.empty((d.B, d.T, d.Hv, d.Dv), dtype=q.dtype, device=dev)
    if state_out is None:
        state_out = torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev)
    else:
        _check(state_out, "state_out", (d.B, d.Hv, d.Dk, d.Dv), torch.float32, dev)
    nck = vg_ckpt_elems(d)
    ckpt = _alloc_ckpt(d, dev, vg=True) if need_ckpt else None
    wsb = _query("gdn_fwd_vg_workspace_bytes", d)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)
    rc = lib().gdn_fwd_vg(ctypes.byref(d), _p(q), _p(k), _p(v), _p(lg), _p(b), _p(state0),
                          _p(mask), _p(o), _p(state_out),
                          _p(ckpt) if (ckpt is not None and nck) else None,
                          _p(ws), wsb, _stream(dev))
    if rc:
        raise GdnError("gdn_fwd_vg", rc)
    return o, state_out, ckpt


def bwd_vg(q, k, v, lg, b, state0, mask, ckpt, dO, dS_final=None, *, algo=ALGO_AUTO, save=False):
    """VJP of fwd_vg.  Returns dict(dq, dk, dv, dlg, db, dstate).  `save`
    must match the fwd_vg call that wrote ckpt."""
    d = _dims_of(q, v, algo, save)
    _check_inputs_vg(d, q, k, v, lg, b, state0, mask)
    dev = q.device
    _check(dO, "dO", (d.B, d.T, d.Hv, d.Dv), q.dtype, dev)
    if dS_final is not None:
        _check(dS_final, "dS_final", (d.B, d.Hv, d.Dk, d.Dv), torch.float32, dev)
    nck = vg_ckpt_elems(d)
    if nck:
        if ckpt is None or ckpt.numel() != nck:
            raise ValueError("ckpt from gdn_fwd_vg with %d elements is required" % nck)
        if ckpt.dtype != torch.float32 or not ckpt.is_contiguous() or ckpt.device != dev:
            raise ValueError("ckpt must be a contiguous fp32 tensor on %s" % dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dlg=torch.empty_like(lg), db=torch.empty_like(b),
               dstate=torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev))
    wsb = _query("gdn_bwd_vg_workspace_bytes", d)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)
    rc = lib().gdn_bwd_vg(ctypes.byref(d), _p(q), _p(k), _p(v), _p(lg), _p(b), _p(state0),
                          _p(mask), _p(ckpt) if nck else None, _p(dO), _p(dS_final),
                          *[_p(out[n]) for n in ("dq", "dk", "dv", "dlg", "db", "dstate")],
                          _p(ws), wsb, _stream(dev))
    if rc:
        raise GdnError("gdn_bwd_vg", rc)
    return out


class PlanVg:
    """Plan (above) for the per-key-channel-gate form: `t` maps q, k, v, lg,
    b, state0, mask, dO, dS_final to device tensors."""

    def __init__(self, t, algo=ALGO_AUTO, stream=None, save=False):
        q, v = t["q"], t["v"]
        self.d = d = _dims_of(q, v, algo, save)
        self.family = "chunk" if vg_uses_chunk(d) else "scan"
        _check_inputs_vg(d, q, t["k"], v, t["lg"], t["b"], t["state0"], t["mask"])
        dev = q.device
        self.t = t
        self.o = torch.empty((d.B, d.T, d.Hv, d.Dv), dtype=q.dtype, device=dev)
        self.state_out = torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev)
        self.ckpt = _alloc_ckpt(d, dev, vg=True)
        nck = self.ckpt.numel()
        self.g = dict(dq=torch.empty_like(q), dk=torch.empty_like(t["k"]), dv=torch.empty_like(v),
                      dlg=torch.empty_like(t["lg"]), db=torch.empty_like(t["b"]),
                      dstate=torch.empty((d.B, d.Hv, d.Dk, d.Dv), dtype=torch.float32, device=dev))
        fws = _query("gdn_fwd_vg_workspace_bytes", d)
        bws = _query("gdn_bwd_vg_workspace_bytes", d)
        self.ws_f = torch.empty((max(fws, 1),), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty((max(bws, 1),), dtype=torch.uint8, device=dev)
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        self.stream = st
        sp = ctypes.c_void_p(st.cuda_stream)
        ck = _p(self.ckpt) if nck else None
        ins = [_p(t[n]) for n in ("q", "k", "v", "lg", "b", "state0", "mask")]
        self._fargs = (ctypes.byref(d), *ins, _p(self.o), _p(self.state_out), ck,
                       _p(self.ws_f), fws, sp)
        self._bargs = (ctypes.byref(d), *ins, ck, _p(t["dO"]), _p(t["dS_final"]),
                       *[_p(self.g[n]) for n in ("dq", "dk", "dv", "dlg", "db", "dstate")],
                       _p(self.ws_b), bws, sp)
        self.fwd_ws_bytes, self.bwd_ws_bytes = fws, bws

    def fwd(self):
        rc = lib().gdn_fwd_vg(*self._fargs)
        if rc:
            raise GdnError("gdn_fwd_vg", rc)

    def bwd(self):
        rc = lib().gdn_bwd_vg(*self._bargs)
        if rc:
            raise GdnError("gdn_bwd_vg", rc)


def decode_conv(x, conv_w, conv_state, a, b, A_log, dt_bias, Hk, Dk, Hv, Dv, state0=None,
                mask=None, *, conv_state_out=None, state_out=None):
    """One decode step preceded by the conv update (gdn_decode_conv).

    x: [B, C] (C = 2 Hk Dk + Hv Dv: q, k, v channels); conv_w: [C, K];
    conv_state: [B, C, K]; a, b: [B, Hv]; A_log, dt_bias: [Hv] fp32; state0:
    [B, Hv, Dk, Dv] fp32 or None; mask: [B] uint8 or None.  Pass
    conv_state_out=conv_state and / or state_out=state0 to update in place.
    Returns (o [B, Hv, Dv], state_out, conv_state_out)."""
    B, C = x.shape
    K = conv_w.shape[1]
    dt, dev = x.dtype, x.device
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError("x has %d channels, expected 2 Hk Dk + Hv Dv = %d" % (C, 2 * Hk * Dk + Hv * Dv))
    d = make_dims(B, 1, Hk, Hv, Dk, Dv, dt)
    _check(x, "x", (B, C), dt, dev)
    _check(conv_w, "conv_w", (C, K), dt, dev)
    _check(conv_state, "conv_state", (B, C, K), dt, dev)
    _check(a, "a", (B, Hv), dt, dev)
    _check(b, "b", (B, Hv), dt, dev)
    _check(A_log, "A_log", (Hv,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (Hv,), torch.float32, dev)
    if state0 is not None:
        _check(state0, "state0", (B, Hv, Dk, Dv), torch.float32, dev)
    if mask is not None:
        _check(mask, "mask", (B,), torch.uint8, dev)
    if conv_state_out is None:
        conv_state_out = torch.empty_like(conv_state)
    else:
        _check(conv_state_out, "conv_state_out", (B, C, K), dt, dev)
    if state_out is None:
        state_out = torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=dev)
    else:
        _check(state_out, "state_out", (B, Hv, Dk, Dv), torch.float32, dev)
    o = torch.empty((B, Hv, Dv), dtype=dt, device=dev)
    rc = lib().gdn_decode_conv(ctypes.byref(d), _p(x), _p(conv_w), _p(conv_state), _p(conv_state_out), K,
                               _p(a), _p(b), _p(A_log), _p(dt_bias), _p(state0), _p(mask), _p(o),
                               _p(state_out), _stream(dev))
    if rc:
        raise GdnError("gdn_decode_conv", rc)
    return o, state_out, conv_state_out

"""Seeded synthetic inputs for the gated delta rule workloads.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the recurrence's arithmetic.  Both the fp64 oracle and the GPU library
consume the values produced here: the oracle gets them exactly upcast to fp64,
the GPU gets the identical bf16 / fp32 bit patterns.

Workloads (the mlx-lm PR's "Numerical correctness" toy shape and its
"Performance" table's Qwen3.5-9B GatedDeltaNet shape; the rest are the edge,
masking and decode sweeps of the same operation):

  tiny         B=1  T=8    Hk=2  Hv=4  Dk=16  Dv=8    fp32  seed 1
  9b_t256      B=1  T=256  Hk=16 Hv=64 Dk=192 Dv=128  bf16  seed 2
  9b_t2048     B=1  T=2048 Hk=16 Hv=64 Dk=192 Dv=128  bf16  seed 3
  edge         B=4  T in {1,64,65,1024} Hk=4 Hv=8 Dk=64 Dv=32  fp32  seed 4000+T
  decode       B=64 T=64 (one step per call) Hk=16 Hv=32 Dk=Dv=128 bf16 seed 5
  decode_conv  as decode, each step preceded by the conv update (K = 4 taps), seed 6
  vg_*         the per-key-channel-gate form (log-gates lg [B,T,Hv,Dk] in place of
               a, A_log, dt_bias): vg_tiny (tiny's dims, seed 7), vg_edge (edge's
               dims, seed 7000+T), vg_9b_t* (the 9B shape, seed 8000+T)

Distributions: q, k, v, a, b ~ N(0,1); A_log ~ U(0, ln 16); dt_bias ~ N(0, 0.5);
state0 ~ N(0, 0.1) (zeros for the 9B shape); dO ~ N(0,1); dS_final ~ N(0,1)
where present.  The second argument of N is the standard deviation.  Draw
order: q, k, v, a, b, A_log, dt_bias, state0, dO, dS_final (numpy PCG64).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "bf16")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even);
    returns the uint16 bit patterns.  Inputs here are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_bits_roundtrip(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


@dataclass
class Case:
    """One workload: dims, storage dtype, and the input / cotangent values.

    ``vals`` holds float64 arrays whose values are exactly representable in the
    storage dtype; ``store(name)`` returns the array to upload (float32, or the
    uint16 bf16 bit pattern for bf16 tensors)."""
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    dtype: str
    vals: dict = field(default_factory=dict)
    mask: np.ndarray | None = None

    # tensors that use the input dtype; the rest (A_log, dt_bias, state0,
    # dS_final) are always fp32
    IO = ("q", "k", "v", "a", "b", "dO")

    @property
    def G(self) -> int:
        return self.Hv // self.Hk

    def store(self, name: str) -> np.ndarray | None:
        x = self.vals.get(name)
        if x is None:
            return None
        if name in self.IO and self.dtype == "bf16":
            return f32_to_bf16_bits(x.astype(np.float32))
        return x.astype(np.float32)

    def oracle_args(self):
        v = self.vals
        return (v["q"], v["k"], v["v"], v["a"], v["b"], v["A_log"], v["dt_bias"],
                v.get("state0"), self.mask)

    def vg_args(self):
        """Inputs of the per-key-channel-gate form (``make_vg_case``)."""
        v = self.vals
        return (v["q"], v["k"], v["v"], v["lg"], v["b"], v.get("state0"), self.mask)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f64(f32_to_bf16_bits(x32))
    return x32.astype(np.float64)


def make_case(name: str, B: int, T: int, Hk: int, Hv: int, Dk: int, Dv: int,
              dtype: str, seed: int, *, state_std: float | None = 0.1,
              dS_final: bool = True, mask: np.ndarray | None = None,
              extreme: bool = False, A_log_range: tuple | None = None) -> Case:
    """Draw one workload.  ``extreme`` sets A_log = 5 and a = 15 everywhere
    (after the draws, so the other tensors are unchanged).  ``A_log_range``
    redraws A_log ~ U(lo, hi) after all other draws (slow decays for long
    memory: A_log in (-7, -4) keeps 10 % to 98 % of the state over a 64-step
    chunk)."""
    assert dtype in DTYPES and Hv % Hk == 0
    rng = np.random.Generator(np.random.PCG64(seed))
    c = Case(name, B, T, Hk, Hv, Dk, Dv, dtype)
    v = c.vals
    v["q"] = _round(rng.standard_normal((B, T, Hk, Dk)), dtype)
    v["k"] = _round(rng.standard_normal((B, T, Hk, Dk)), dtype)
    v["v"] = _round(rng.standard_normal((B, T, Hv, Dv)), dtype)
    v["a"] = _round(rng.standard_normal((B, T, Hv)), dtype)
    v["b"] = _round(rng.standard_normal((B, T, Hv)), dtype)
    v["A_log"] = _round(rng.uniform(0.0, math.log(16.0), (Hv,)), "f32")
    v["dt_bias"] = _round(0.5 * rng.standard_normal((Hv,)), "f32")
    if state_std is not None:
        v["state0"] = _round(state_std * rng.standard_normal((B, Hv, Dk, Dv)), "f32")
    v["dO"] = _round(rng.standard_normal((B, T, Hv, Dv)), dtype)
    if dS_final:
        v["dS_final"] = _round(rng.standard_normal((B, Hv, Dk, Dv)), "f32")
    if extreme:
        v["A_log"] = np.full((Hv,), 5.0)
        v["a"] = np.full((B, T, Hv), 15.0)
    if A_log_range is not None:
        v["A_log"] = _round(rng.uniform(A_log_range[0], A_log_range[1], (Hv,)), "f32")
    if mask is not None:
        c.mask = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        assert c.mask.shape == (B, T)
    return c


def tiny() -> Case:
    return make_case("tiny", 1, 8, 2, 4, 16, 8, "f32", 1)


def qwen35_9b(T: int = 2048) -> Case:
    seed = {256: 2, 2048: 3}.get(T, 3000 + T)
    return make_case("9b_t%d" % T, 1, T, 16, 64, 192, 128, "bf16", seed,
                     state_std=None, dS_final=False)


def edge_mask(B: int, T: int) -> np.ndarray:
    """Rows 0 and 2 all valid; rows 1 and 3 valid only for t < floor(T/2)."""
    m = np.ones((B, T), dtype=np.uint8)
    for r in range(1, B, 2):
        m[r, T // 2:] = 0
    return m


def edge(T: int, *, masked: bool = True, extreme: bool = False, dtype: str = "f32") -> Case:
    B = 4
    name = "edge_T%d%s%s%s" % (T, "_mask" if masked else "", "_extreme" if extreme else "",
                               "" if dtype == "f32" else "_" + dtype)
    return make_case(name, B, T, 4, 8, 64, 32, dtype, 4000 + T,
                     mask=edge_mask(B, T) if masked else None, extreme=extreme)


def decode(steps: int = 64) -> Case:
    """The decode workload as one [B, steps] draw; call i uses column t = i."""
    return make_case("decode", 64, steps, 16, 32, 128, 128, "bf16", 5,
                     dS_final=False)


class ConvCase:
    """The decode step with the preceding conv update: per call, one token's
    mixed projection x [B, C] (C = 2 Hk Dk + Hv Dv channels: q, k, v, each
    head-major), conv taps [C, K], the carried conv samples [B, C, K], gates
    a, b [B, Hv] and the recurrent state [B, Hv, Dk, Dv].  ``vals`` holds float64
    arrays exactly representable in the storage dtype; x, conv_w, conv_state,
    a, b use the input dtype, the rest fp32."""
    IO = ("x", "conv_w", "conv_state", "a", "b")

    def __init__(self, name, B, steps, Hk, Hv, Dk, Dv, K, dtype, vals, mask):
        self.name, self.B, self.steps, self.Hk, self.Hv, self.Dk, self.Dv, self.K = name, B, steps, Hk, Hv, Dk, Dv, K
        self.dtype, self.vals, self.mask = dtype, vals, mask
        self.C = 2 * Hk * Dk + Hv * Dv

    def store(self, name: str) -> np.ndarray | None:
        x = self.vals.get(name)
        if x is None:
            return None
        if name in self.IO and self.dtype == "bf16":
            return f32_to_bf16_bits(x.astype(np.float32))
        return x.astype(np.float32)


def make_conv_case(name: str, B: int, steps: int, Hk: int, Hv: int, Dk: int, Dv: int, K: int,
                   dtype: str, seed: int, *, mask: np.ndarray | None = None) -> ConvCase:
    """Draw a conv-decode workload: x ~ N(0,1) per call ([B, steps, C]); the
    carried conv samples ~ N(0,1); taps ~ U(-1/sqrt(K), 1/sqrt(K)) (the usual
    fan-in range of a depthwise kernel of K taps); a, b ~ N(0,1) per call;
    A_log ~ U(0, ln 16); dt_bias ~ N(0, 0.5); state0 ~ N(0, 0.1).  mask: [B]
    (nonzero = valid), the same for every call, or None."""
    assert dtype in DTYPES and Hv % Hk == 0
    rng = np.random.Generator(np.random.PCG64(seed))
    C = 2 * Hk * Dk + Hv * Dv
    v = {}
    v["x"] = _round(rng.standard_normal((B, steps, C)), dtype)
    v["conv_state"] = _round(rng.standard_normal((B, C, K)), dtype)
    v["conv_w"] = _round(rng.uniform(-1.0, 1.0, (C, K)) / math.sqrt(K), dtype)
    v["a"] = _round(rng.standard_normal((B, steps, Hv)), dtype)
    v["b"] = _round(rng.standard_normal((B, steps, Hv)), dtype)
    v["A_log"] = _round(rng.uniform(0.0, math.log(16.0), (Hv,)), "f32")
    v["dt_bias"] = _round(0.5 * rng.standard_normal((Hv,)), "f32")
    v["state0"] = _round(0.1 * rng.standard_normal((B, Hv, Dk, Dv)), "f32")
    m = None if mask is None else np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    return ConvCase(name, B, steps, Hk, Hv, Dk, Dv, K, dtype, v, m)


def decode_conv(steps: int = 64) -> ConvCase:
    """The decode workload with the conv update (kernel of 4 taps)."""
    return make_conv_case("decode_conv", 64, steps, 16, 32, 128, 128, 4, "bf16", 6)


def make_vg_case(name: str, B: int, T: int, Hk: int, Hv: int, Dk: int, Dv: int,
                 dtype: str, seed: int, *, state_std: float | None = 0.1,
                 dS_final: bool = True, mask: np.ndarray | None = None,
                 lg_mu: float = -1.5, lg_sigma: float = 1.5) -> Case:
    """Draw a workload of the per-key-channel-gate form: the gate is given as
    log-gates lg [B,T,Hv,Dk] (fp32), lg = -exp(z) with z ~ N(lg_mu, lg_sigma)
    (default N(-1.5, 1.5)), so per-channel decays g = e^lg range from nearly 1
    (long memory) to nearly 0 (median e^-0.22 = 0.80; lg_mu = -6, lg_sigma = 1
    gives slow decays, median e^-0.0025).  q, k, v, b, dO ~ N(0,1); state0 ~
    N(0, 0.1); dS_final ~ N(0,1).  Draw order: q, k, v, lg, b, state0, dO,
    dS_final."""
    assert dtype in DTYPES and Hv % Hk == 0
    rng = np.random.Generator(np.random.PCG64(seed))
    c = Case(name, B, T, Hk, Hv, Dk, Dv, dtype)
    v = c.vals
    v["q"] = _round(rng.standard_normal((B, T, Hk, Dk)), dtype)
    v["k"] = _round(rng.standard_normal((B, T, Hk, Dk)), dtype)
    v["v"] = _round(rng.standard_normal((B, T, Hv, Dv)), dtype)
    v["lg"] = _round(-np.exp(lg_mu + lg_sigma * rng.standard_normal((B, T, Hv, Dk))), "f32")
    v["b"] = _round(rng.standard_normal((B, T, Hv)), dtype)
    if state_std is not None:
        v["state0"] = _round(state_std * rng.standard_normal((B, Hv, Dk, Dv)), "f32")
    v["dO"] = _round(rng.standard_normal((B, T, Hv, Dv)), dtype)
    if dS_final:
        v["dS_final"] = _round(rng.standard_normal((B, Hv, Dk, Dv)), "f32")
    if mask is not None:
        c.mask = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        assert c.mask.shape == (B, T)
    return c


def vg_tiny() -> Case:
    return make_vg_case("vg_tiny", 1, 8, 2, 4, 16, 8, "f32", 7)


def vg_edge(T: int, *, masked: bool = True, dtype: str = "f32") -> Case:
    B = 4
    name = "vg_edge_T%d%s%s" % (T, "_mask" if masked else "", "" if dtype == "f32" else "_" + dtype)
    return make_vg_case(name, B, T, 4, 8, 64, 32, dtype, 7000 + T,
                        mask=edge_mask(B, T) if masked else None)


def vg_qwen35_9b(T: int = 2048) -> Case:
    """The 9B layer shape with a per-channel gate in place of the scalar one."""
    return make_vg_case("vg_9b_t%d" % T, 1, T, 16, 64, 192, 128, "bf16", 8000 + T,
                        state_std=None, dS_final=False)


def by_name(name: str) -> Case:
    if name == "tiny":
        return tiny()
    if name.startswith("9b_t"):
        return qwen35_9b(int(name[4:]))
    if name == "decode":
        return decode()
    raise KeyError(name)

"""GPU state carry and mask invariants of the chunk family (single pass and
T-parallel), against the fp64 oracle and bit for bit where the pages' method
fixes the bits.

- State carry (mlx-lm VJP PR, "Design notes": the state is carried between
  chunks and returned; torch-to-nnef GDN page, "Op contract": the final state
  is an output): a forward over steps [0, T1) followed by a forward over
  [T1, T) from the first call's final state gives the outputs and the final
  state of one forward over [0, T); the backward chained the other way --
  the second half's backward first, then the first half's with the second
  half's dstate as its state cotangent -- gives the full gradients (the
  per-head parameter gradients are the sums of the two calls').  The split
  points fall inside chunks, so the two routes round differently: compared
  with the oracle at the bf16 bar, 2e-2 normwise.
- Masks (PR, "Covered corner cases": an all-valid mask equals no mask, and a
  row masked from step n on ends in the state of its first n steps): bitwise
  on the chunk form, whose masked steps are exact identity maps (a log-gate
  of 0 and a write strength of 0)."""
import numpy as np
import pytest
import torch

from helpers import GRADS, TOL, gpu_bwd, gpu_fwd, oracle_all, report, say, to64, upload
from linear_attention_recurrence_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu
CHUNK, TPAR = binding.ALGO_CHUNK, binding.ALGO_CHUNK_TPAR
SLOW = (-7.0, -4.0)
SEQ = ("q", "k", "v", "a", "b", "dO")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()


def part(t, lo, hi):
    return {n: (x[:, lo:hi].contiguous() if n in SEQ or n == "mask" and x is not None else x)
            for n, x in t.items()}


def bits(x):
    return x.view(torch.uint8) if x.dtype == torch.bfloat16 else x


CARRY = [
    # name, B, T, Hk, Hv, Dk, Dv, T1, seed, algo
    ("carry_chunk", 2, 384, 2, 4, 128, 64, 200, 701, CHUNK),
    ("carry_chunk_dk192", 1, 300, 1, 4, 192, 128, 131, 702, CHUNK),
    ("carry_tpar", 1, 8192, 1, 2, 128, 64, 4000, 703, TPAR),
]


@pytest.mark.parametrize("name,B,T,Hk,Hv,Dk,Dv,T1,seed,algo", CARRY)
@pytest.mark.parametrize("save", [False, True])
def test_state_carry(name, B, T, Hk, Hv, Dk, Dv, T1, seed, algo, save):
    c = inputs.make_case(name, B, T, Hk, Hv, Dk, Dv, "bf16", seed, A_log_range=SLOW)
    say("[carry] case=%s B=%d T=%d split=%d algo=%d save=%d" % (name, B, T, T1, algo, save))
    t = upload(c)
    t1, t2 = part(t, 0, T1), part(t, T1, T)
    o1, s1, k1 = gpu_fwd(t1, algo=algo, save=save)
    t2["state0"] = s1
    o2, s2, k2 = gpu_fwd(t2, algo=algo, save=save)
    g2 = gpu_bwd(t2, k2, algo=algo, save=save)
    t1["dS_final"] = g2["dstate"]
    g1 = gpu_bwd(t1, k1, algo=algo, save=save)
    torch.cuda.synchronize()
    ro, rst, _, rg = oracle_all(c, nthreads=16)
    cat = lambda n: to64(torch.cat([g1[n], g2[n]], dim=1))
    pairs = [("o", to64(torch.cat([o1, o2], dim=1)), ro), ("state", to64(s2), rst)]
    pairs += [(n, cat(n), rg[n]) for n in ("dq", "dk", "dv", "da", "db")]
    pairs += [(n, to64(g1[n]) + to64(g2[n]), rg[n]) for n in ("dA_log", "ddt_bias")]
    pairs.append(("dstate", to64(g1["dstate"]), rg["dstate"]))
    errs = report("carry %s" % name, pairs)
    bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad


@pytest.mark.parametrize("T", [200, 256])
def test_chunk_mask_invariants(T):
    """All-valid mask == no mask (outputs, states, checkpoints and all eight
    gradients, bitwise); rows masked from floor(T/2) on end in the final
    state of their unmasked prefix, bitwise (T = 200: the boundary falls
    inside a chunk; T = 256: on a chunk boundary)."""
    B = 4
    c = inputs.make_case("mask_chunk_t%d" % T, B, T, 2, 4, 128, 64, "bf16", 710 + T, A_log_range=SLOW)
    say("[mask] chunk case=%s" % c.name)
    t = upload(c)
    o0, s0, k0 = gpu_fwd(t, algo=CHUNK)
    g0 = gpu_bwd(t, k0, algo=CHUNK)
    t1 = dict(t)
    t1["mask"] = torch.ones((B, T), dtype=torch.uint8, device="cuda")
    o1, s1, k1 = gpu_fwd(t1, algo=CHUNK)
    g1 = gpu_bwd(t1, k1, algo=CHUNK)
    torch.cuda.synchronize()
    for x, y in [(o0, o1), (s0, s1), (k0, k1)] + [(g0[n], g1[n]) for n in GRADS]:
        assert torch.equal(bits(x), bits(y))
    t2 = dict(t)
    t2["mask"] = torch.from_numpy(inputs.edge_mask(B, T)).cuda()
    _, s2, _ = gpu_fwd(t2, algo=CHUNK)
    n = T // 2
    _, sp, _ = gpu_fwd(part(t, 0, n), algo=CHUNK)
    torch.cuda.synchronize()
    assert torch.equal(s2[1], sp[1]) and torch.equal(s2[3], sp[3])
    assert torch.equal(s2[0], s0[0]) and torch.equal(s2[2], s0[2])


def test_tpar_mask_invariants():
    """The T-parallel form: an all-valid mask equals no mask bitwise; a row
    masked from T/2 on ends in the state of its prefix within the bf16 bar
    (the prefix alone is split into other segments, so the rounding differs),
    and the masked run matches the oracle."""
    B, T = 2, 8192
    c = inputs.make_case("mask_tpar", B, T, 1, 2, 128, 64, "bf16", 720, A_log_range=SLOW)
    say("[mask] tpar case=%s" % c.name)
    t = upload(c)
    o0, s0, _ = gpu_fwd(t, algo=TPAR)
    t1 = dict(t)
    t1["mask"] = torch.ones((B, T), dtype=torch.uint8, device="cuda")
    o1, s1, _ = gpu_fwd(t1, algo=TPAR)
    torch.cuda.synchronize()
    assert torch.equal(bits(o0), bits(o1)) and torch.equal(s0, s1)
    m = np.ones((B, T), dtype=np.uint8)
    m[1, T // 2:] = 0
    cm = inputs.make_case("mask_tpar", B, T, 1, 2, 128, 64, "bf16", 720, A_log_range=SLOW, mask=m)
    t2 = dict(t)
    t2["mask"] = torch.from_numpy(m).cuda()
    o2, s2, _ = gpu_fwd(t2, algo=TPAR)
    _, sp, _ = gpu_fwd(part(t, 0, T // 2), algo=TPAR)
    torch.cuda.synchronize()
    ro, rst, _, _ = oracle_all(cm, nthreads=16)
    errs = report("mask tpar", [("o", to64(o2), ro), ("state", to64(s2), rst),
                                ("prefix_state", to64(s2[1]), to64(sp[1]))])
    assert torch.equal(s2[0], s0[0])
    bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad

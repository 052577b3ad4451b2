"""GPU parity of the T-parallel chunk form (GDN_ALGO_CHUNK_TPAR: segment
maps, a chain over the segments, then every segment's outputs; in the forward
and, last segment first, in the backward's reverse state pass) against the
fp64 oracle, and against the single-pass chunk form.  Long sequences with
few heads, where the library splits the chunks into segments; slow decays
(A_log in (-7, -4)), so that a segment's start state reaches far into it and
the segment maps are far from zero (with the default fast decays the state
forgets a chunk within a few steps and every route gives the same bits);
ragged tails, masks, initial states, the saved record and the backward that
follows.  bf16 bar of 2e-2 (normwise), as for every bf16
workload; repeated runs bit-identical."""
import numpy as np
import pytest
import torch

from helpers import GRADS, TOL, gpu_bwd, gpu_fwd, oracle_all, relerr, say, to64, upload
from linear_attention_recurrence_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu
TPAR, CHUNK = binding.ALGO_CHUNK_TPAR, binding.ALGO_CHUNK


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()


def segmented(c):
    """The T-parallel forward needs more workspace exactly when it splits."""
    d = binding.make_dims(c.B, c.T, c.Hk, c.Hv, c.Dk, c.Dv, binding.GDN_BF16, TPAR)
    d1 = binding.make_dims(c.B, c.T, c.Hk, c.Hv, c.Dk, c.Dv, binding.GDN_BF16, CHUNK)
    return binding.fwd_workspace_bytes(d) > binding.fwd_workspace_bytes(d1)


CASES = [
    # name, B, T, Hk, Hv, Dk, Dv, seed, masked
    ("tpar_t4096_dk128", 1, 4096, 1, 2, 128, 64, 501, False),
    ("tpar_t3000_dk64_mask", 2, 3000, 2, 4, 64, 32, 502, True),
    ("tpar_t2048_dk192", 1, 2048, 1, 1, 192, 128, 503, False),
    ("tpar_t1100_dk256", 1, 1100, 1, 1, 256, 32, 504, True),
]


@pytest.mark.parametrize("name,B,T,Hk,Hv,Dk,Dv,seed,masked", CASES)
def test_tpar_parity(name, B, T, Hk, Hv, Dk, Dv, seed, masked):
    mask = None
    if masked:
        mask = np.ones((B, T), dtype=np.uint8)
        mask[0, T // 3: T // 3 + 70] = 0
        mask[-1, T - 50:] = 0
    c = inputs.make_case(name, B, T, Hk, Hv, Dk, Dv, "bf16", seed, mask=mask, A_log_range=(-7.0, -4.0))
    assert segmented(c), "the case must run more than one segment"
    say("[tpar] case=%s B=%d T=%d Hk=%d Hv=%d Dk=%d Dv=%d" % (name, B, T, Hk, Hv, Dk, Dv))
    t = upload(c)
    o, st, ck = gpu_fwd(t, algo=TPAR)
    g = gpu_bwd(t, ck, algo=TPAR)
    o1, st1, ck1 = gpu_fwd(t, algo=CHUNK)
    g1 = gpu_bwd(t, ck1, algo=CHUNK)
    torch.cuda.synchronize()
    ro, rst, rck, rg = oracle_all(c, nthreads=16)
    errs = {"o": relerr(to64(o), ro), "state": relerr(to64(st), rst), "ckpt": relerr(to64(ck), rck)}
    for n in GRADS:
        errs[n] = relerr(to64(g[n]), rg[n])
    vs_chunk = {"o": relerr(to64(o), to64(o1)), "state": relerr(to64(st), to64(st1)),
                "ckpt": relerr(to64(ck), to64(ck1))}
    for n in ("dq", "dk", "dv", "dstate"):
        vs_chunk[n] = relerr(to64(g[n]), to64(g1[n]))
    say("[tpar] errors " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    say("[tpar] vs single pass " + " ".join("%s=%.2e" % kv for kv in vs_chunk.items()))
    assert vs_chunk["state"] > 0.0, "the segments must change the rounding (long memory)"
    assert vs_chunk["dstate"] > 0.0, "the backward's segments must change the rounding"
    bad = {n: e for n, e in list(errs.items()) + [("chunk_" + k, v) for k, v in vs_chunk.items()]
           if not e <= TOL["bf16"]}
    assert not bad, bad


def test_tpar_saved_record_and_repeat():
    c = inputs.make_case("tpar_save", 1, 4096, 1, 2, 128, 64, "bf16", 505, A_log_range=(-7.0, -4.0))
    assert segmented(c)
    say("[tpar] saved record + repeat")
    t = upload(c)
    runs = []
    for _ in range(2):
        o, st, ck = gpu_fwd(t, algo=TPAR, save=True)
        g = gpu_bwd(t, ck, algo=TPAR, save=True)
        runs.append([o, st] + [g[n] for n in GRADS])
    torch.cuda.synchronize()
    for x, y in zip(*runs):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)
    ro, rst, _, rg = oracle_all(c, nthreads=16)
    o, st = runs[0][0], runs[0][1]
    assert relerr(to64(o), ro) <= TOL["bf16"] and relerr(to64(st), rst) <= TOL["bf16"]
    for n, x in zip(GRADS, runs[0][2:]):
        assert relerr(to64(x), rg[n]) <= TOL["bf16"], n


@pytest.mark.parametrize("kind", ["masked_segment", "extreme"])
def test_tpar_degenerate_segments(kind):
    """A segment whose steps are all masked (its map is the identity: the
    state passes through it) and extreme gates (every map close to 0)."""
    B, T = 1, 4096
    if kind == "masked_segment":
        mask = np.ones((B, T), dtype=np.uint8)
        mask[0, 1024:2048] = 0   # two whole 512-step segments (8 chunks each)
        c = inputs.make_case("tpar_" + kind, B, T, 1, 2, 128, 64, "bf16", 506, mask=mask,
                             A_log_range=(-7.0, -4.0))
    else:
        c = inputs.make_case("tpar_" + kind, B, T, 1, 2, 128, 64, "bf16", 507, extreme=True)
    assert segmented(c)
    say("[tpar] case=%s" % c.name)
    t = upload(c)
    o, st, ck = gpu_fwd(t, algo=TPAR)
    g = gpu_bwd(t, ck, algo=TPAR)
    torch.cuda.synchronize()
    ro, rst, rck, rg = oracle_all(c, nthreads=16)
    errs = {"o": relerr(to64(o), ro), "state": relerr(to64(st), rst), "ckpt": relerr(to64(ck), rck)}
    for n in GRADS:
        errs[n] = relerr(to64(g[n]), rg[n])
    say("[tpar] errors " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for n, x in list(g.items()) + [("o", o), ("state", st)]:
        assert torch.isfinite(x.float()).all(), n
    bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad

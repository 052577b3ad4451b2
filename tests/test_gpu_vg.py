"""GPU parity of the per-key-channel gate (gdn_fwd_vg / gdn_bwd_vg through
the C ABI) against the fp64 oracle (oracle.fwd_vg / oracle.bwd_vg).

Tolerances as for the scalar gate (normwise per tensor, max|x - ref| /
max|ref|): 1e-4 for fp32 workloads, 2e-2 for bf16.  The fp32 cases run the
scan kernels and cover every lane layout of the reverse sweep (Dk = 16 .. 256:
one to four rows per lane, rows padded below 64; Dv with one or four waves
per workgroup), ragged chunk tails and recompute blocks, masks.  The bf16
cases run the chunk form (AUTO or CHUNK): every built (Dk, Dv) with ragged
tails and masks, sequences of 1 .. 129 steps, gates that do not decay, that
underflow, that decay strongly or slowly over 2048 steps, the Qwen3.5-9B
layer shape at T = 256 and 2048 with a per-channel gate, a Kimi-Linear-like
shape (32 heads of 128; the pages name the model but not its sizes, so the
sizes are an assumption), and a forward of one family with a backward of the
other.  Repeated runs must be bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, dev_tensor, relerr, say, to64
from linear_attention_recurrence_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu
VG_GRADS = ("dq", "dk", "dv", "dlg", "db", "dstate")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()


def upload_vg(case):
    t = {n: dev_tensor(case, n) for n in ("q", "k", "v", "lg", "b", "state0", "dO", "dS_final")}
    t["mask"] = None if case.mask is None else torch.from_numpy(case.mask).cuda()
    return t


def run_vg(t, algo=binding.ALGO_AUTO, bwd_algo=None, save=False):
    o, st, ck = binding.fwd_vg(t["q"], t["k"], t["v"], t["lg"], t["b"], t["state0"], t["mask"], algo=algo,
                               save=save)
    g = binding.bwd_vg(t["q"], t["k"], t["v"], t["lg"], t["b"], t["state0"], t["mask"], ck,
                       t["dO"], t["dS_final"], algo=algo if bwd_algo is None else bwd_algo, save=save)
    return o, st, ck, g


def compare_vg(case, nthreads=8, algo=binding.ALGO_AUTO, bwd_algo=None, save=False):
    tol = TOL[case.dtype]
    say("[vg] case=%s B=%d T=%d Hk=%d Hv=%d Dk=%d Dv=%d dtype=%s algo=%d/%d save=%d" % (
        case.name, case.B, case.T, case.Hk, case.Hv, case.Dk, case.Dv, case.dtype, algo,
        algo if bwd_algo is None else bwd_algo, save))
    t = upload_vg(case)
    o, st, ck, g = run_vg(t, algo, bwd_algo, save)
    torch.cuda.synchronize()
    v = case.vals
    ro, rst, rck = oracle.fwd_vg(*case.vg_args(), nthreads=nthreads)
    rg = oracle.bwd_vg(*case.vg_args(), v["dO"], v.get("dS_final"), nthreads=nthreads)
    errs = {"o": relerr(to64(o), ro), "state": relerr(to64(st), rst)}
    if rck.shape[0] and not save:  # the fp32 states (the saved record holds none)
        errs["ckpt"] = relerr(to64(ck), rck)
    for n in VG_GRADS:
        errs[n] = relerr(to64(g[n]), rg[n])
    say("[vg] errors " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for n, x in list(g.items()) + [("o", o), ("state", st)]:
        assert torch.isfinite(x.float()).all(), n
    if case.mask is not None:   # masked steps: exact zeros
        m = torch.from_numpy(case.mask == 0)
        for n in ("dlg", "db", "dv"):
            assert torch.all(g[n].cpu()[m] == 0), n
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    return t, (o, st, ck, g)


def test_vg_tiny():
    compare_vg(inputs.vg_tiny())


@pytest.mark.parametrize("T", [1, 3, 64, 65, 130, 1024])
@pytest.mark.parametrize("masked", [False, True])
def test_vg_edge(T, masked):
    compare_vg(inputs.vg_edge(T, masked=masked))


@pytest.mark.parametrize("Dk,Dv,dtype", [(16, 8, "f32"), (32, 16, "f32"), (32, 24, "bf16"),
                                         (128, 64, "bf16"), (256, 32, "f32"), (256, 8, "f32"),
                                         (192, 96, "f32")])
def test_vg_shapes(Dk, Dv, dtype):
    B, T = 2, 77
    mask = np.ones((B, T), dtype=np.uint8)
    mask[1, 40:] = 0
    mask[0, 5] = 0
    c = inputs.make_vg_case("vg_Dk%d_Dv%d_%s" % (Dk, Dv, dtype), B, T, 2, 4, Dk, Dv, dtype,
                            9000 + Dk + Dv, mask=mask)
    compare_vg(c)


def test_vg_kimi_like():
    compare_vg(inputs.make_vg_case("vg_kimi_like", 1, 256, 32, 32, 128, 128, "bf16", 9100,
                                   state_std=None, dS_final=False))


def test_vg_qwen35_9b_t256():
    compare_vg(inputs.vg_qwen35_9b(256))


def test_vg_qwen35_9b_t2048():
    compare_vg(inputs.vg_qwen35_9b(2048), nthreads=16)


def test_vg_deterministic_repeat():
    c = inputs.vg_qwen35_9b(256)
    say("[vg determinism] case=%s" % c.name)
    t = upload_vg(c)
    outs = []
    for _ in range(3):
        o, st, ck, g = run_vg(t)
        outs.append([o, st, ck] + [g[n] for n in VG_GRADS])
    torch.cuda.synchronize()
    for other in outs[1:]:
        for x, y in zip(outs[0], other):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


@pytest.mark.parametrize("T", [1, 70])
def test_vg_state_in_place(T):
    """state_out may alias state0 exactly: the same bits as a separate output."""
    c = inputs.make_vg_case("vg_inplace_T%d" % T, 2, T, 2, 4, 64, 32, "f32", 9200 + T)
    say("[vg in-place] case=%s" % c.name)
    t = upload_vg(c)
    o, st, _ = binding.fwd_vg(t["q"], t["k"], t["v"], t["lg"], t["b"], t["state0"], None)
    s = t["state0"].clone()
    o2, st2, _ = binding.fwd_vg(t["q"], t["k"], t["v"], t["lg"], t["b"], s, None, state_out=s)
    torch.cuda.synchronize()
    assert st2.data_ptr() == s.data_ptr()
    assert torch.equal(o, o2) and torch.equal(st, s)


def test_vg_empty_sequence():
    """T = 0: the state passes through, dstate = dS_final, nothing else."""
    c = inputs.make_vg_case("vg_empty", 2, 0, 2, 4, 64, 32, "f32", 9300)
    say("[vg empty] case=%s" % c.name)
    t = upload_vg(c)
    o, st, ck, g = run_vg(t)
    torch.cuda.synchronize()
    assert o.numel() == 0 and g["dlg"].numel() == 0
    assert torch.equal(st, t["state0"]) and torch.equal(g["dstate"], t["dS_final"])


@pytest.mark.parametrize("kind", ["no_decay", "underflow"])
def test_vg_extreme_gates(kind):
    """lg = 0 (g = 1: the delta rule without decay) and lg = -200 on every
    other channel (g underflows to 0: those rows are wiped each step); the
    gradients stay finite and match the oracle."""
    c = inputs.make_vg_case("vg_" + kind, 2, 130, 2, 4, 64, 32, "f32", 9400, mask=None)
    if kind == "no_decay":
        c.vals["lg"][...] = 0.0
    else:
        c.vals["lg"][..., ::2] = -200.0
    compare_vg(c)


# ---- the chunk form (bf16)

@pytest.mark.parametrize("Dk,Dv", [(64, 32), (64, 128), (128, 64), (128, 96), (192, 32), (192, 128)])
def test_vg_chunk_shapes(Dk, Dv):
    """Three chunks with a ragged tail (64 + 64 + 13 steps) and masked steps,
    two value heads per key head, for every built head size."""
    B, T = 2, 141
    mask = np.ones((B, T), dtype=np.uint8)
    mask[0, 5] = 0
    mask[0, 63:66] = 0
    mask[1, 100:] = 0
    c = inputs.make_vg_case("vg_chunk_Dk%d_Dv%d" % (Dk, Dv), B, T, 2, 4, Dk, Dv, "bf16",
                            9600 + Dk + Dv, mask=mask)
    compare_vg(c, algo=binding.ALGO_CHUNK)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129])
def test_vg_chunk_edges(T):
    compare_vg(inputs.vg_edge(T, masked=True, dtype="bf16"), algo=binding.ALGO_CHUNK)


@pytest.mark.parametrize("kind", ["no_decay", "underflow", "strong"])
def test_vg_chunk_extreme_gates(kind):
    """lg = 0 (no decay), lg = -200 on every other channel (those rows are
    wiped every step: e^{G} underflows inside the chunk products) and lg = -30
    on a third of the channels with slow decays elsewhere."""
    c = inputs.make_vg_case("vg_chunk_" + kind, 2, 150, 2, 4, 128, 64, "bf16", 9700)
    if kind == "no_decay":
        c.vals["lg"][...] = 0.0
    elif kind == "underflow":
        c.vals["lg"][..., ::2] = -200.0
    else:
        c.vals["lg"][...] = -0.01
        c.vals["lg"][..., ::3] = -30.0
    compare_vg(c, algo=binding.ALGO_CHUNK)


def test_vg_chunk_long_memory():
    """Slow decays (median e^-0.0025 per step) over 2048 steps: the bf16
    rounding of the chunk products carried through 32 chunk boundaries."""
    c = inputs.make_vg_case("vg_chunk_long_memory", 1, 2048, 2, 4, 128, 128, "bf16", 9800,
                            lg_mu=-6.0, lg_sigma=1.0)
    compare_vg(c, nthreads=16, algo=binding.ALGO_CHUNK)


@pytest.mark.parametrize("fwd,bwd", [(binding.ALGO_CHUNK, binding.ALGO_SCAN),
                                     (binding.ALGO_SCAN, binding.ALGO_CHUNK)])
def test_vg_families_interchange(fwd, bwd):
    """Both families write the same fp32 checkpoints, so a forward of one pairs
    with a backward of the other."""
    mask = np.ones((2, 150), dtype=np.uint8)
    mask[1, 70:90] = 0
    c = inputs.make_vg_case("vg_interchange", 2, 150, 2, 4, 128, 64, "bf16", 9900, mask=mask)
    compare_vg(c, algo=fwd, bwd_algo=bwd)


def test_vg_chunk_state_in_place():
    c = inputs.make_vg_case("vg_chunk_inplace", 2, 70, 2, 4, 64, 32, "bf16", 9950)
    say("[vg chunk in-place] case=%s" % c.name)
    t = upload_vg(c)
    o, st, _ = binding.fwd_vg(t["q"], t["k"], t["v"], t["lg"], t["b"], t["state0"], None,
                              algo=binding.ALGO_CHUNK)
    s = t["state0"].clone()
    o2, st2, _ = binding.fwd_vg(t["q"], t["k"], t["v"], t["lg"], t["b"], s, None, state_out=s,
                                algo=binding.ALGO_CHUNK)
    torch.cuda.synchronize()
    assert st2.data_ptr() == s.data_ptr()
    assert torch.equal(o, o2) and torch.equal(st, s)


# ---- the chunk form's saved record (save=True: the forward writes the rows,
# matrices and X the backward reads, the backward recomputes none of them)

@pytest.mark.parametrize("Dk,Dv", [(64, 32), (64, 128), (128, 64), (128, 96), (192, 32), (192, 128)])
def test_vg_saved_shapes(Dk, Dv):
    B, T = 2, 141
    mask = np.ones((B, T), dtype=np.uint8)
    mask[0, 5] = 0
    mask[0, 63:66] = 0
    mask[1, 100:] = 0
    c = inputs.make_vg_case("vg_saved_Dk%d_Dv%d" % (Dk, Dv), B, T, 2, 4, Dk, Dv, "bf16",
                            9600 + Dk + Dv, mask=mask)
    compare_vg(c, algo=binding.ALGO_CHUNK, save=True)


@pytest.mark.parametrize("T", [1, 64, 65])
def test_vg_saved_edges(T):
    compare_vg(inputs.vg_edge(T, masked=True, dtype="bf16"), algo=binding.ALGO_CHUNK, save=True)


def test_vg_saved_qwen35_9b_t256():
    compare_vg(inputs.vg_qwen35_9b(256), save=True)


def test_vg_saved_long_memory():
    c = inputs.make_vg_case("vg_saved_long_memory", 1, 2048, 2, 4, 128, 128, "bf16", 9800,
                            lg_mu=-6.0, lg_sigma=1.0)
    compare_vg(c, nthreads=16, algo=binding.ALGO_CHUNK, save=True)


def test_vg_saved_repeat_and_unsaved():
    """Saved runs are bit-identical to each other, and agree with the path that
    recomputes (same tolerance as against the oracle: the two compute X in
    different kernels, with different accumulation orders)."""
    c = inputs.vg_qwen35_9b(256)
    say("[vg saved] case=%s" % c.name)
    t = upload_vg(c)
    runs = [run_vg(t, save=True) for _ in range(2)]
    base = run_vg(t)
    torch.cuda.synchronize()
    (o1, s1, c1, g1), (o2, s2, c2, g2) = runs
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(c1, c2)
    for n in VG_GRADS:
        assert torch.equal(g1[n], g2[n]), n
    o0, s0, _, g0 = base
    errs = {"o": relerr(to64(o1), to64(o0)), "state": relerr(to64(s1), to64(s0))}
    for n in VG_GRADS:
        errs[n] = relerr(to64(g1[n]), to64(g0[n]))
    say("[vg saved vs recomputed] " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    assert all(e <= TOL["bf16"] for e in errs.values()), errs

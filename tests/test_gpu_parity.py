"""GPU parity: libgdn.so (through its C ABI) against the fp64 oracle.

Tolerances (normwise per tensor, max|x - ref| / max|ref|): 1e-4 for fp32
workloads, 2e-2 for bf16 workloads.  Workloads: the PR's toy shape, the edge
and masking sweep (T in {1, 64, 65, 1024}, masks, extreme gates), the
Qwen3.5-9B GDN layer shape at T = 256 and T = 2048 (every element compared),
ragged shapes, and the decode chain.  Repeated runs must be bit-identical.
The first group runs the sequential scan (ALGO_SCAN; AUTO for fp32), the
second the chunked form (ALGO_CHUNK, bf16), which AUTO picks for bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import GRADS, TOL, dev_tensor, gpu_bwd, gpu_fwd, oracle_all, relerr, report, say, to64, upload
from linear_attention_recurrence_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()  # a GPU without the built library is an error, not a skip


def run_and_compare(case, tol=None, algo=binding.ALGO_AUTO, nthreads=8):
    tol = tol if tol is not None else TOL[case.dtype]
    say("[parity] case=%s B=%d T=%d Hk=%d Hv=%d Dk=%d Dv=%d dtype=%s algo=%d" % (
        case.name, case.B, case.T, case.Hk, case.Hv, case.Dk, case.Dv, case.dtype, algo))
    t = upload(case)
    o, st, ck = gpu_fwd(t, algo=algo)
    g = gpu_bwd(t, ck, algo=algo)
    torch.cuda.synchronize()
    ro, rst, rck, rg = oracle_all(case, nthreads=nthreads)
    pairs = [("o", to64(o), ro), ("state", to64(st), rst)]
    if rck.shape[0]:
        pairs.append(("ckpt", to64(ck), rck))
    pairs += [(n, to64(g[n]), rg[n]) for n in GRADS]
    errs = report("parity", pairs)
    for n, x in list(g.items()) + [("o", o), ("state", st)]:
        assert torch.isfinite(x.float()).all(), n
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    return t, (o, st, ck, g)


def test_tiny():
    run_and_compare(inputs.tiny())


@pytest.mark.parametrize("T", [1, 64, 65, 1024])
@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("extreme", [False, True])
def test_edge(T, masked, extreme):
    run_and_compare(inputs.edge(T, masked=masked, extreme=extreme))


SCAN = binding.ALGO_SCAN


def test_ragged_dk128():
    c = inputs.make_case("ragged_dk128", 2, 200, 2, 4, 128, 64, "bf16", 77)
    run_and_compare(c, algo=SCAN)


def test_ragged_dk32_dv16_fp32():
    c = inputs.make_case("ragged_dk32", 3, 70, 1, 3, 32, 16, "f32", 78,
                         mask=np.array([[1] * 70, [1] * 35 + [0] * 35, [0] + [1] * 69]))
    run_and_compare(c)


def test_qwen35_9b_t256():
    run_and_compare(inputs.qwen35_9b(256), algo=SCAN)


def test_qwen35_9b_t2048():
    run_and_compare(inputs.qwen35_9b(2048), algo=SCAN, nthreads=16)


def test_deterministic_repeat():
    c = inputs.qwen35_9b(256)
    say("[determinism] case=%s" % c.name)
    t = upload(c)
    outs = []
    for _ in range(3):
        o, st, ck = gpu_fwd(t, algo=SCAN)
        g = gpu_bwd(t, ck, algo=SCAN)
        outs.append([o, st, ck] + [g[n] for n in GRADS])
    torch.cuda.synchronize()
    for other in outs[1:]:
        for x, y in zip(outs[0], other):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def test_mask_invariants_on_gpu():
    """All-valid mask == no mask (bitwise), and a half-masked row's final state
    equals the final state of its unmasked prefix (bitwise), on the GPU."""
    c = inputs.edge(65, masked=False)
    say("[mask] case=%s" % c.name)
    t = upload(c)
    o0, s0, _ = gpu_fwd(t)
    t1 = dict(t)
    t1["mask"] = torch.ones((c.B, c.T), dtype=torch.uint8, device="cuda")
    o1, s1, _ = gpu_fwd(t1)
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    t2 = dict(t)
    t2["mask"] = torch.from_numpy(inputs.edge_mask(c.B, c.T)).cuda()
    _, s2, _ = gpu_fwd(t2)
    n = c.T // 2
    tp = {k_: (v_[:, :n].contiguous() if k_ in ("q", "k", "v", "a", "b", "dO") else v_)
          for k_, v_ in t.items()}
    _, sp, _ = gpu_fwd(tp)
    assert torch.equal(s2[1], sp[1]) and torch.equal(s2[3], sp[3])
    assert torch.equal(s2[0], s0[0])


def test_decode_chain():
    """64 single-step calls with the state updated in place equal the oracle's
    64-step run (outputs of every step and the final state)."""
    c = inputs.decode(64)
    say("[decode] case=%s B=%d steps=%d" % (c.name, c.B, c.T))
    t = upload(c)
    state = t["state0"].clone()
    outs = []
    for i in range(c.T):
        sl = {n: t[n][:, i:i + 1].contiguous() for n in ("q", "k", "v", "a", "b")}
        o, st, ck = binding.fwd(sl["q"], sl["k"], sl["v"], sl["a"], sl["b"], t["A_log"],
                                t["dt_bias"], state, None, need_ckpt=False, state_out=state)
        assert st.data_ptr() == state.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    o_gpu = to64(torch.cat(outs, dim=1))
    ro, rst, _ = oracle.fwd(*c.oracle_args(), nthreads=8)
    e_o, e_s = relerr(o_gpu, ro), relerr(to64(state), rst)
    say("[decode] errors o=%.2e state=%.2e" % (e_o, e_s))
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


def test_empty_sequence():
    c = inputs.make_case("empty", 2, 0, 1, 2, 16, 8, "f32", 33)
    say("[empty] case=%s" % c.name)
    t = upload(c)
    o, st, ck = gpu_fwd(t)
    g = gpu_bwd(t, ck)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 8)
    assert torch.equal(st, t["state0"])
    assert torch.equal(g["dstate"], t["dS_final"])
    assert torch.all(g["dA_log"] == 0) and torch.all(g["ddt_bias"] == 0)


# ---------------------------------------------------------------- chunk form

CHUNK = binding.ALGO_CHUNK


@pytest.mark.parametrize("T", [1, 64, 65, 1024])
@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("extreme", [False, True])
def test_chunk_edge_bf16(T, masked, extreme):
    run_and_compare(inputs.edge(T, masked=masked, extreme=extreme, dtype="bf16"), algo=CHUNK)


def test_chunk_ragged_dk128():
    c = inputs.make_case("chunk_ragged_dk128", 2, 200, 2, 4, 128, 64, "bf16", 79)
    run_and_compare(c, algo=CHUNK)


def test_chunk_ragged_dk256_g1():
    c = inputs.make_case("chunk_ragged_dk256", 1, 130, 2, 2, 256, 32, "bf16", 80)
    run_and_compare(c, algo=CHUNK)


def test_chunk_dk64_g4():
    c = inputs.make_case("chunk_dk64_g4", 2, 150, 2, 8, 64, 96, "bf16", 81)
    run_and_compare(c, algo=CHUNK)


def test_chunk_qwen35_9b_t256():
    run_and_compare(inputs.qwen35_9b(256), algo=CHUNK)


def test_chunk_qwen35_9b_t2048():
    run_and_compare(inputs.qwen35_9b(2048), algo=CHUNK, nthreads=16)


def test_chunk_deterministic_repeat():
    c = inputs.qwen35_9b(256)
    say("[determinism] chunk case=%s" % c.name)
    t = upload(c)
    outs = []
    for _ in range(3):
        o, st, ck = gpu_fwd(t, algo=CHUNK)
        g = gpu_bwd(t, ck, algo=CHUNK)
        outs.append([o, st, ck] + [g[n] for n in GRADS])
    torch.cuda.synchronize()
    for other in outs[1:]:
        for x, y in zip(outs[0], other):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def test_auto_runs_chunk_for_bf16():
    """AUTO on a bf16 workload gives the chunk form's bits exactly."""
    c = inputs.qwen35_9b(256)
    say("[auto] case=%s" % c.name)
    t = upload(c)
    o1, s1, k1 = gpu_fwd(t)
    g1 = gpu_bwd(t, k1)
    o2, s2, k2 = gpu_fwd(t, algo=CHUNK)
    g2 = gpu_bwd(t, k2, algo=CHUNK)
    torch.cuda.synchronize()
    for x, y in [(o1, o2), (s1, s2), (k1, k2)] + [(g1[n], g2[n]) for n in GRADS]:
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def test_chunk_checkpoint_interchange():
    """A checkpoint from the scan forward drives the chunk backward (and the
    reverse) to the oracle's gradients within the bf16 bound."""
    c = inputs.qwen35_9b(256)
    say("[interchange] case=%s" % c.name)
    t = upload(c)
    ro, rst, rck, rg = oracle_all(c, nthreads=8)
    for fa, ba in ((SCAN, CHUNK), (CHUNK, SCAN)):
        _, _, ck = gpu_fwd(t, algo=fa)
        g = gpu_bwd(t, ck, algo=ba)
        torch.cuda.synchronize()
        errs = {n: relerr(to64(g[n]), rg[n]) for n in GRADS}
        say("[interchange] fwd=%d bwd=%d errors " % (fa, ba) +
            " ".join("%s=%.2e" % kv for kv in errs.items()))
        assert all(e <= TOL["bf16"] for e in errs.values()), errs


@pytest.mark.parametrize("case", ["9b_t256", "ragged_dk128", "ragged_dk256_g1", "dk64_g4", "edge65_masked", "edge1"])
def test_chunk_saved_matrices_bitwise(case):
    """Under gdn_dims.save the forward saves the chunk matrices, the bf16
    chunk-start states and X of every step, and the backward uses them instead
    of recomputing the matrices and X and converting the fp32 checkpoints:
    every output and every gradient is bit-identical to the run without save
    (each head size has its own gradient-pass kernel for the saved path)."""
    c = {"9b_t256": lambda: inputs.qwen35_9b(256),
         "ragged_dk128": lambda: inputs.make_case("chunk_ragged_dk128", 2, 200, 2, 4, 128, 64, "bf16", 79),
         "ragged_dk256_g1": lambda: inputs.make_case("chunk_ragged_dk256", 1, 130, 2, 2, 256, 32, "bf16", 80),
         "dk64_g4": lambda: inputs.make_case("chunk_dk64_g4", 2, 150, 2, 8, 64, 96, "bf16", 81),
         "edge65_masked": lambda: inputs.edge(65, masked=True, extreme=False, dtype="bf16"),
         "edge1": lambda: inputs.edge(1, masked=False, extreme=False, dtype="bf16")}[case]()
    say("[saved] case=%s" % c.name)
    t = upload(c)
    o1, s1, k1 = gpu_fwd(t, algo=CHUNK)
    g1 = gpu_bwd(t, k1, algo=CHUNK)
    o2, s2, k2 = gpu_fwd(t, algo=CHUNK, save=True)
    g2 = gpu_bwd(t, k2, algo=CHUNK, save=True)
    torch.cuda.synchronize()
    for x, y in [(o1, o2), (s1, s2)] + [(g1[n], g2[n]) for n in GRADS]:
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


# Groups of more than four value heads per key head: the gradient pass takes
# the per-head scalars in batches of four, and value heads 4, 8, ... start a
# new batch.  Ragged T, a mask with invalid steps, with and without the saved
# record (G = 9 also leaves a last batch of one head).
GROUPS = {
    "g6_dk128": (1, 150, 1, 6, 128, 64, 91),
    "g8_dk192": (2, 100, 1, 8, 192, 32, 92),
    "g9_dk64": (1, 70, 1, 9, 64, 32, 93),
    "g5_dk256": (1, 90, 1, 5, 256, 32, 94),
}


def _group_case(name):
    B, T, Hk, Hv, Dk, Dv, seed = GROUPS[name]
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    mask = (rng.random((B, T)) > 0.2).astype(np.uint8)
    return inputs.make_case("chunk_" + name, B, T, Hk, Hv, Dk, Dv, "bf16", seed, mask=mask)


@pytest.mark.parametrize("save", [False, True])
@pytest.mark.parametrize("name", list(GROUPS))
def test_chunk_many_heads_per_group(name, save):
    c = _group_case(name)
    say("[groups] case=%s B=%d T=%d Hk=%d Hv=%d Dk=%d Dv=%d save=%d" % (c.name, c.B, c.T, c.Hk, c.Hv, c.Dk,
                                                                      c.Dv, save))
    t = upload(c)
    o, st, ck = gpu_fwd(t, algo=CHUNK, save=save)
    g = gpu_bwd(t, ck, algo=CHUNK, save=save)
    torch.cuda.synchronize()
    ro, rst, rck, rg = oracle_all(c, nthreads=8)
    pairs = [("o", to64(o), ro), ("state", to64(st), rst)]
    pairs += [(n, to64(g[n]), rg[n]) for n in GRADS]
    errs = report("groups", pairs)
    for n, x in list(g.items()) + [("o", o), ("state", st)]:
        assert torch.isfinite(x.float()).all(), n
    bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad


def test_chunk_many_heads_saved_bitwise():
    """With more than four value heads per key head the saved record still
    gives the bits of the run without it."""
    c = _group_case("g6_dk128")
    say("[groups saved] case=%s" % c.name)
    t = upload(c)
    o1, s1, k1 = gpu_fwd(t, algo=CHUNK)
    g1 = gpu_bwd(t, k1, algo=CHUNK)
    o2, s2, k2 = gpu_fwd(t, algo=CHUNK, save=True)
    g2 = gpu_bwd(t, k2, algo=CHUNK, save=True)
    torch.cuda.synchronize()
    for x, y in [(o1, o2), (s1, s2)] + [(g1[n], g2[n]) for n in GRADS]:
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)

"""GPU parity of the decode step with the preceding conv update
(gdn_decode_conv, through the C ABI) against the fp64 oracle
(oracle.decode_conv: the conv update, then the single-step recurrence).

Tolerances as the other parity tests (normwise per tensor: 1e-4 fp32,
2e-2 bf16).  The carried conv samples are copies of inputs, so they must match
bit for bit.  Shapes cover G = 1, 2, 4, key widths 16 .. 256, value widths 32 ..
128, 2 .. 8 taps, masked rows, in-place chains of calls, and repeat runs.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, relerr, say, to64
from linear_attention_recurrence_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()


def upload(c):
    def dev(name):
        x = c.store(name)
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).cuda()
    t = {n: dev(n) for n in ("x", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state0")}
    t["mask"] = None if c.mask is None else torch.from_numpy(c.mask).cuda()
    return t


def gpu_step(c, t, i, conv_state, state0, **kw):
    return binding.decode_conv(t["x"][:, i].contiguous(), t["conv_w"], conv_state, t["a"][:, i].contiguous(),
                               t["b"][:, i].contiguous(), t["A_log"], t["dt_bias"], c.Hk, c.Dk, c.Hv, c.Dv,
                               state0, t["mask"], **kw)


def oracle_step(c, i, conv_state, state0):
    v = c.vals
    return oracle.decode_conv(v["x"][:, i], conv_state, v["conv_w"], v["a"][:, i], v["b"][:, i], v["A_log"],
                              v["dt_bias"], c.Hk, c.Dk, c.Hv, c.Dv, state0=state0, mask=c.mask)


SHAPES = [  # dtype, Hk, Hv, Dk, Dv, K, masked
    ("bf16", 2, 4, 64, 32, 4, False),
    ("bf16", 2, 4, 64, 32, 4, True),
    ("f32", 1, 1, 128, 128, 2, False),
    ("bf16", 2, 8, 128, 64, 4, False),
    ("f32", 4, 8, 16, 32, 8, True),
    ("f32", 2, 2, 32, 64, 1, False),
    ("bf16", 1, 2, 256, 32, 3, False),
    ("bf16", 1, 1, 192, 128, 4, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s_hk%d_hv%d_dk%d_dv%d_k%d%s" % (s[:6] + ("_m" if s[6] else "",)))
def test_decode_conv_parity(shape):
    dtype, Hk, Hv, Dk, Dv, K, masked = shape
    B = 4
    c = inputs.make_conv_case("dconv", B, 1, Hk, Hv, Dk, Dv, K, dtype, 70 + Dk + K,
                              mask=np.array([1, 0, 1, 0]) if masked else None)
    say("[decode_conv] B=%d Hk=%d Hv=%d Dk=%d Dv=%d K=%d dtype=%s masked=%s" % (B, Hk, Hv, Dk, Dv, K, dtype, masked))
    t = upload(c)
    o, st, cs = gpu_step(c, t, 0, t["conv_state"], t["state0"])
    torch.cuda.synchronize()
    ro, rst, rcs = oracle_step(c, 0, c.vals["conv_state"], c.vals["state0"])
    errs = {"o": relerr(to64(o), ro), "state": relerr(to64(st), rst)}
    say("[decode_conv] errors " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    assert np.array_equal(to64(cs), rcs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_conv_in_place_chain(dtype):
    """Eight calls, each updating the conv state and the state in place, follow
    the oracle's eight steps; a repeat of the chain is bit-identical."""
    B, Hk, Hv, Dk, Dv, K, steps = 3, 2, 4, 64, 64, 4, 8
    c = inputs.make_conv_case("dconv_chain", B, steps, Hk, Hv, Dk, Dv, K, dtype, 91, mask=np.array([1, 1, 0]))
    say("[decode_conv chain] dtype=%s steps=%d" % (dtype, steps))
    runs = []
    for rep in range(2):
        t = upload(c)
        cs, st = t["conv_state"], t["state0"]
        outs = []
        for i in range(steps):
            o, st2, cs2 = gpu_step(c, t, i, cs, st, conv_state_out=cs, state_out=st)
            assert cs2.data_ptr() == cs.data_ptr() and st2.data_ptr() == st.data_ptr()
            outs.append(o.clone())
        torch.cuda.synchronize()
        runs.append((torch.stack(outs), st.clone(), cs.clone()))
    rcs, rst = c.vals["conv_state"], c.vals["state0"]
    for i in range(steps):
        ro, rst, rcs = oracle_step(c, i, rcs, rst)
        e = relerr(to64(runs[0][0][i]), ro)
        assert e <= TOL[dtype], (i, e)
    assert relerr(to64(runs[0][1]), rst) <= TOL[dtype]
    assert np.array_equal(to64(runs[0][2]), rcs)
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)

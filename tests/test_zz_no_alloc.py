"""gdn_fwd_noalloc (the forward whose workspace is the library's static device
array) against gdn_fwd (the same forward with a caller-allocated workspace),
through the C ABI: two calls in a row, the second on a smaller input, so the
second runs on the scratch contents the first left behind.  Both routes run
the same kernels in the same order, so the outputs must agree bit for bit
(stronger than the bf16 / fp32 parity bars); the first case is also checked
against the oracle.  Cases: the chunk form with the saved record, the fp32
scan, the T-parallel chunk form, and an in-place state update."""
import numpy as np
import pytest
import torch

from helpers import TOL, gpu_fwd, oracle_all, relerr, say, to64, upload
from linear_attention_recurrence_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()


def bits(x):
    return x.view(torch.uint8) if x.dtype == torch.bfloat16 else x


def noalloc(t, algo, save, in_place=False):
    B, T, Hk, Dk = t["q"].shape
    Hv, Dv = t["v"].shape[2], t["v"].shape[3]
    d = binding.make_dims(B, T, Hk, Hv, Dk, Dv, t["q"].dtype, algo, save)
    assert binding.fwd_workspace_bytes(d) <= binding.NOALLOC_SCRATCH_BYTES
    o = torch.empty((B, T, Hv, Dv), dtype=t["q"].dtype, device="cuda")
    st = t["state0"] if in_place else torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device="cuda")
    n = binding.ckpt_elems(d)
    ck = torch.empty((n,), dtype=torch.float32, device="cuda") if n else None
    binding.fwd_noalloc(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"], t["dt_bias"], t["state0"],
                        t["mask"], o=o, state_out=st, ckpt=ck, algo=algo, save=save)
    return o, st, ck


PAIRS = [
    # (large case, small case, algo, save)
    (("na_chunk_big", 2, 700, 2, 4, 128, 64, "bf16", 801), ("na_chunk_small", 1, 130, 1, 2, 64, 32, "bf16", 802),
     binding.ALGO_CHUNK, True),
    (("na_scan_big", 2, 300, 2, 4, 64, 32, "f32", 803), ("na_scan_small", 1, 70, 1, 1, 16, 8, "f32", 804),
     binding.ALGO_SCAN, False),
    (("na_tpar_big", 1, 8192, 1, 2, 128, 64, "bf16", 805), ("na_tpar_small", 1, 4096, 1, 1, 64, 32, "bf16", 806),
     binding.ALGO_CHUNK_TPAR, False),
]


@pytest.mark.parametrize("big,small,algo,save", PAIRS)
def test_noalloc_matches_gdn_fwd(big, small, algo, save):
    cases = [inputs.make_case(*big, A_log_range=(-7.0, -4.0)), inputs.make_case(*small, A_log_range=(-7.0, -4.0))]
    ts = [upload(c) for c in cases]
    ref = [gpu_fwd(t, algo=algo, save=save) for t in ts]
    torch.cuda.synchronize()
    for c, t, r in zip(cases, ts, ref):
        say("[noalloc] case=%s algo=%d save=%d" % (c.name, algo, save))
        o, st, ck = noalloc(t, algo, save)
        torch.cuda.synchronize()
        assert torch.equal(bits(o), bits(r[0])), c.name
        assert torch.equal(st, r[1]), c.name
        if ck is not None:
            assert torch.equal(ck.view(-1), r[2].reshape(-1)), c.name
    ro, rst, _, _ = oracle_all(cases[0], nthreads=16)
    tol = TOL[cases[0].dtype]
    o, st, _ = noalloc(ts[0], algo, save)
    torch.cuda.synchronize()
    assert relerr(to64(o), ro) <= tol and relerr(to64(st), rst) <= tol


def test_noalloc_in_place_and_too_big():
    """state_out == state0 (the single pass, as gdn_fwd), then a call whose
    workspace exceeds the static array: refused with GDN_ERR_WORKSPACE and
    nothing written."""
    c = inputs.make_case("na_inplace", 1, 8192, 1, 2, 128, 64, "bf16", 807, A_log_range=(-7.0, -4.0))
    t = upload(c)
    t_ref = dict(t, state0=t["state0"].clone())
    r = gpu_fwd(t_ref, algo=binding.ALGO_CHUNK)
    o, st, _ = noalloc(t, binding.ALGO_CHUNK_TPAR, False, in_place=True)
    torch.cuda.synchronize()
    assert st.data_ptr() == t["state0"].data_ptr()
    assert torch.equal(bits(o), bits(r[0])) and torch.equal(st, r[1])
    big = inputs.make_case("na_big", 1, 2048, 16, 64, 192, 128, "bf16", 808, state_std=None, dS_final=False)
    tb = upload(big)
    d = binding.make_dims(1, 2048, 16, 64, 192, 128, torch.bfloat16, binding.ALGO_CHUNK, True)
    assert binding.fwd_workspace_bytes(d) <= binding.NOALLOC_SCRATCH_BYTES  # the 9B layer at T=2048 fits
    huge = binding.make_dims(1, 16384, 16, 64, 192, 128, torch.bfloat16, binding.ALGO_CHUNK, False)
    assert binding.fwd_workspace_bytes(huge) > binding.NOALLOC_SCRATCH_BYTES
    o = torch.zeros((1, 2048, 64, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((1, 64, 192, 128), dtype=torch.float32, device="cuda")
    n = binding.ckpt_elems(d)
    ck = torch.empty((n,), dtype=torch.float32, device="cuda")
    binding.fwd_noalloc(tb["q"], tb["k"], tb["v"], tb["a"], tb["b"], tb["A_log"], tb["dt_bias"], None, None,
                        o=o, state_out=st, ckpt=ck, algo=binding.ALGO_CHUNK, save=True)
    r9 = gpu_fwd(tb, algo=binding.ALGO_CHUNK, save=True)
    torch.cuda.synchronize()
    assert torch.equal(bits(o), bits(r9[0])) and torch.equal(st, r9[1])
    lib = binding.lib()
    import ctypes
    p = [ctypes.c_void_p(tb["q"].data_ptr())] * 12
    rc = lib.gdn_fwd_noalloc(ctypes.byref(huge), *p, None)
    assert rc == 3

"""C ABI of libgdn.so on the CPU: the library loads, exports every entry point
include/gdn.h declares, and validates arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_fwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(gdn_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = declared()
    assert set(names) == set(B.EXPORTS)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gdn_version().startswith(b"gdn-mi355x")


def test_status_strings():
    lib = B.lib()
    for code in range(5):
        assert lib.gdn_status_string(code)
    assert lib.gdn_status_string(99) == b"unknown status"


def test_size_queries():
    d = B.make_dims(1, 2048, 16, 64, 192, 128, B.GDN_BF16)
    assert B.ckpt_elems(d) == 31 * 64 * 192 * 128
    d = B.make_dims(4, 65, 4, 8, 64, 32, B.GDN_F32)
    assert B.ckpt_elems(d) == 1 * 4 * 8 * 64 * 32
    for T in (0, 1, 64):
        assert B.ckpt_elems(B.make_dims(4, T, 4, 8, 64, 32, B.GDN_F32)) == 0
    assert B.fwd_workspace_bytes(d) > 0
    assert B.bwd_workspace_bytes(d) > B.fwd_workspace_bytes(d)


@pytest.mark.parametrize("dims,code", [
    ((1, 8, 3, 4, 16, 8), 1),        # Hv % Hk != 0
    ((0, 8, 2, 4, 16, 8), 1),        # B < 1
    ((1, -1, 2, 4, 16, 8), 1),       # T < 0
    ((1, 8, 2, 4, 48, 8), 2),        # Dk not built
    ((1, 8, 2, 4, 16, 12), 2),       # Dv not a multiple of 8
    ((1, 8, 2, 4, 16, 40), 2),       # Dv > 24 and not a multiple of 32
])
def test_bad_dims(dims, code):
    with pytest.raises(B.GdnError) as e:
        B.fwd_workspace_bytes(B.make_dims(*dims, B.GDN_F32))
    assert e.value.code == code


def test_bad_dtype_and_algo():
    with pytest.raises(B.GdnError) as e:
        B.fwd_workspace_bytes(B.make_dims(1, 8, 2, 4, 16, 8, 7))
    assert e.value.code == 2
    with pytest.raises(B.GdnError) as e:
        B.fwd_workspace_bytes(B.make_dims(1, 8, 2, 4, 16, 8, B.GDN_F32, 9))
    assert e.value.code == 1


def _fake(n):
    return [ctypes.c_void_p(4096 * (i + 1)) for i in range(n)]


def test_fwd_rejects_before_launch():
    """Null required pointers and a short workspace are reported without any
    kernel launch (the pointers here are never dereferenced)."""
    lib = B.lib()
    d = B.make_dims(1, 8, 2, 4, 16, 8, B.GDN_F32)
    need = B.fwd_workspace_bytes(d)
    p = _fake(13)  # q k v a b A_log dt_bias state0 mask o state_out ckpt ws
    args = list(p)
    args[0] = None  # q
    assert lib.gdn_fwd(ctypes.byref(d), *args, need, None) == 1
    args = list(p)
    args[10] = None  # state_out
    assert lib.gdn_fwd(ctypes.byref(d), *args, need, None) == 1
    assert lib.gdn_fwd(ctypes.byref(d), *p, need - 1, None) == 3
    assert lib.gdn_fwd(ctypes.byref(d), *p[:12], None, need, None) == 3
    assert lib.gdn_fwd(None, *p, need, None) == 1


def test_bwd_rejects_before_launch():
    lib = B.lib()
    d = B.make_dims(1, 130, 2, 4, 16, 8, B.GDN_F32)
    need = B.bwd_workspace_bytes(d)
    p = _fake(21)  # ... ckpt(9) dO dS_final dq dk dv(14) da db dA_log ddt_bias dstate ws
    args = list(p)
    args[9] = None  # ckpt is required when T > 64
    assert lib.gdn_bwd(ctypes.byref(d), *args, need, None) == 1
    args = list(p)
    args[14] = None  # dv
    assert lib.gdn_bwd(ctypes.byref(d), *args, need, None) == 1
    assert lib.gdn_bwd(ctypes.byref(d), *p, need - 1, None) == 3


def test_auto_selects_chunk_for_bf16():
    """AUTO runs the chunk form for bf16 with a built head size and T > 1 (its
    workspace equals CHUNK's), and the scan otherwise."""
    def ws(T, dtype, Dk, algo):
        d = B.make_dims(1, T, 16, 64, Dk, 128, dtype, algo)
        return B.fwd_workspace_bytes(d), B.bwd_workspace_bytes(d)
    assert ws(2048, B.GDN_BF16, 192, B.ALGO_AUTO) == ws(2048, B.GDN_BF16, 192, B.ALGO_CHUNK)
    assert ws(2048, B.GDN_BF16, 192, B.ALGO_AUTO) != ws(2048, B.GDN_BF16, 192, B.ALGO_SCAN)
    assert ws(2048, B.GDN_F32, 192, B.ALGO_AUTO) == ws(2048, B.GDN_F32, 192, B.ALGO_SCAN)
    assert ws(1, B.GDN_BF16, 192, B.ALGO_AUTO) == ws(1, B.GDN_BF16, 192, B.ALGO_SCAN)
    assert ws(2048, B.GDN_BF16, 32, B.ALGO_AUTO) == ws(2048, B.GDN_BF16, 32, B.ALGO_SCAN)


@pytest.mark.parametrize("dtype,Dk,Dv", [(B.GDN_F32, 192, 128), (B.GDN_BF16, 32, 128),
                                         (B.GDN_BF16, 192, 16)])
def test_chunk_unsupported(dtype, Dk, Dv):
    with pytest.raises(B.GdnError) as e:
        B.fwd_workspace_bytes(B.make_dims(1, 128, 2, 4, Dk, Dv, dtype, B.ALGO_CHUNK))
    assert e.value.code == 2


def test_saved_chunk_matrices_sizes():
    """gdn_dims.save (chunk family) turns the checkpoint buffer into the
    library's own: the chunk-start states in bf16 (one slot per chunk, chunk 0
    included) and the saved chunk matrices, which leave the workspaces; the
    scan family ignores it."""
    plain = B.make_dims(1, 2048, 16, 64, 192, 128, B.GDN_BF16)
    saved = B.make_dims(1, 2048, 16, 64, 192, 128, B.GDN_BF16, save=True)
    states = 31 * 64 * 192 * 128
    mats = 64 * 32 * 64 * 64 // 2        # one bf16 64x64 matrix per (head, chunk), in fp32 elements
    qts = 16 * 32 * 192 * 64 // 2       # the chunk's q rows transposed, bf16
    scal = 64 * 32 * 12 * 64
    assert B.ckpt_elems(plain) == states
    slots = 32 * 64 * 192 * 128 // 2     # bf16, in fp32 elements
    xs = 2048 * 64 * 128 // 2            # X of every step, bf16
    assert B.ckpt_elems(saved) == slots + 2 * mats + qts + scal + xs  # Tx and P^T
    assert B.bwd_workspace_bytes(saved) < B.bwd_workspace_bytes(plain)
    assert B.fwd_workspace_bytes(saved) < B.fwd_workspace_bytes(plain)
    f32 = B.make_dims(1, 2048, 16, 64, 192, 128, B.GDN_F32, save=True)
    assert B.ckpt_elems(f32) == states
    assert B.bwd_workspace_bytes(f32) == B.bwd_workspace_bytes(B.make_dims(1, 2048, 16, 64, 192, 128, B.GDN_F32))
    one = B.make_dims(1, 1, 16, 64, 192, 128, B.GDN_BF16, B.ALGO_CHUNK, save=True)
    assert B.ckpt_elems(one) > 0      # the initial state's slot and the saved matrices


def test_saved_needs_the_checkpoint_buffer():
    lib = B.lib()
    d = B.make_dims(1, 32, 2, 4, 64, 32, B.GDN_BF16, B.ALGO_CHUNK, save=True)
    p = _fake(13)
    need = B.fwd_workspace_bytes(d)
    args = list(p)
    args[11] = None  # ckpt
    assert lib.gdn_fwd(ctypes.byref(d), *args, need, None) == 1
    need = B.bwd_workspace_bytes(d)
    p = _fake(21)
    args = list(p)
    args[9] = None  # ckpt (T <= 64, but the saved matrices live there)
    assert lib.gdn_bwd(ctypes.byref(d), *args, need, None) == 1


def test_decode_conv_rejects_before_launch():
    """gdn_decode_conv validates T == 1, the tap count, the head sizes and the
    required pointers before any launch (the pointers here are never
    dereferenced)."""
    lib = B.lib()
    p = _fake(13)  # x conv_w conv_state conv_state_out | a b A_log dt_bias state0 mask o state_out stream

    def call(d, k=4, args=None):
        a = list(p) if args is None else args
        return lib.gdn_decode_conv(ctypes.byref(d), a[0], a[1], a[2], a[3], k, a[4], a[5], a[6], a[7],
                                   a[8], a[9], a[10], a[11], None)
    ok = B.make_dims(2, 1, 2, 4, 64, 32, B.GDN_BF16)
    assert call(B.make_dims(2, 2, 2, 4, 64, 32, B.GDN_BF16)) == 1   # T != 1
    assert call(ok, k=0) == 1 and call(ok, k=9) == 1                # taps
    assert call(B.make_dims(2, 1, 2, 4, 48, 32, B.GDN_BF16)) == 2   # Dk not built
    assert call(B.make_dims(2, 1, 2, 4, 64, 40, B.GDN_BF16)) == 2   # Dv not a multiple of 32
    for i in (0, 1, 2, 3, 4, 5, 6, 7, 10, 11):                      # required pointers
        args = list(p)
        args[i] = None
        assert call(ok, args=args) == 1, i


def test_vg_rejects_before_launch():
    """gdn_fwd_vg / gdn_bwd_vg: the chunk form of the per-channel gate exists
    for bf16 with Dk 64 / 128 / 192 only, and not T-parallel; required
    pointers and the workspace are checked before any launch (the pointers
    here are never dereferenced)."""
    lib = B.lib()
    out = ctypes.c_size_t(0)
    chunk = B.make_dims(1, 128, 2, 4, 64, 32, B.GDN_BF16, B.ALGO_CHUNK)
    assert lib.gdn_fwd_vg_workspace_bytes(ctypes.byref(chunk), ctypes.byref(out)) == 0
    assert lib.gdn_bwd_vg_workspace_bytes(ctypes.byref(chunk), ctypes.byref(out)) == 0
    for bad in (B.make_dims(1, 128, 2, 4, 256, 32, B.GDN_BF16, B.ALGO_CHUNK),
                B.make_dims(1, 128, 2, 4, 64, 32, B.GDN_F32, B.ALGO_CHUNK),
                B.make_dims(1, 128, 2, 4, 64, 32, B.GDN_BF16, B.ALGO_CHUNK_TPAR)):
        assert lib.gdn_fwd_vg_workspace_bytes(ctypes.byref(bad), ctypes.byref(out)) == 2
        assert lib.gdn_bwd_vg_workspace_bytes(ctypes.byref(bad), ctypes.byref(out)) == 2
    d = B.make_dims(1, 128, 2, 4, 64, 32, B.GDN_F32)
    assert lib.gdn_fwd_vg_workspace_bytes(ctypes.byref(d), ctypes.byref(out)) == 0
    fws = out.value
    assert lib.gdn_bwd_vg_workspace_bytes(ctypes.byref(d), ctypes.byref(out)) == 0
    bws = out.value
    # sub-checkpoints (every 4 steps of a chunk, rows padded to 64) + partials
    assert bws >= fws + 4 * (1 * 4 * 32 * 64 * 16 + 1 * 128 * 4 * 1 * 3 * 64)
    f = _fake(10)  # q k v lg b state0 mask o state_out ckpt
    for i in (0, 1, 2, 3, 4, 7, 8):
        args = list(f)
        args[i] = None
        assert lib.gdn_fwd_vg(ctypes.byref(d), *args, f[0], fws, None) == 1, i
    assert lib.gdn_fwd_vg(ctypes.byref(d), *f, f[0], fws - 1, None) == 3
    g = _fake(16)  # q k v lg b state0 mask ckpt dO dS dq dk dv dlg db dstate
    for i in (0, 1, 2, 3, 4, 7, 8, 10, 11, 12, 13, 14, 15):
        args = list(g)
        args[i] = None
        assert lib.gdn_bwd_vg(ctypes.byref(d), *args, g[0], bws, None) == 1, i
    assert lib.gdn_bwd_vg(ctypes.byref(d), *g, g[0], bws - 1, None) == 3


def test_vg_saved_record_sizes():
    """gdn_vg_ckpt_elems: the fp32 states without save (and on the scan family,
    which ignores save); with save on the chunk form, the record: the bf16
    state at every chunk start, then per (chunk, head) four bf16 row blocks of
    64 x Dk, two 64 x 64 bf16 matrices (Tx, P^T) and the chunk scalars, and X of every
    step (each region 256-byte aligned).  The saved workspaces are smaller than the unsaved
    ones by what moved into the record, and a NULL ckpt is refused."""
    lib = B.lib()
    out = ctypes.c_size_t(0)
    Bn, T, Hk, Hv, Dk, Dv = 1, 200, 2, 4, 128, 64
    nc = (T + 63) // 64
    states = (nc - 1) * Bn * Hv * Dk * Dv
    for dtype, algo, save, want in ((B.GDN_BF16, B.ALGO_CHUNK, 0, states), (B.GDN_F32, B.ALGO_AUTO, 1, states),
                                    (B.GDN_BF16, B.ALGO_SCAN, 1, states)):
        d = B.make_dims(Bn, T, Hk, Hv, Dk, Dv, dtype, algo, save)
        assert lib.gdn_vg_ckpt_elems(ctypes.byref(d), ctypes.byref(out)) == 0
        assert out.value == want
    d = B.make_dims(Bn, T, Hk, Hv, Dk, Dv, B.GDN_BF16, B.ALGO_CHUNK, 1)
    assert lib.gdn_vg_ckpt_elems(ctypes.byref(d), ctypes.byref(out)) == 0
    bhc = Bn * Hv * nc
    pieces = [bhc * Dk * Dv // 2] + [bhc * 64 * Dk // 2] * 4 + [bhc * 64 * 64 // 2] * 2 + [bhc * 8 * 64, Bn * T * Hv * Dv // 2]
    assert out.value == sum((p * 4 + 255) // 256 * 64 for p in pieces)
    assert lib.gdn_vg_ckpt_bytes(ctypes.byref(d), ctypes.byref(out)) == 0
    assert out.value == sum((p * 4 + 255) // 256 * 256 for p in pieces)
    ws = {}
    for save in (0, 1):
        dd = B.make_dims(Bn, T, Hk, Hv, Dk, Dv, B.GDN_BF16, B.ALGO_CHUNK, save)
        for fn in ("gdn_fwd_vg_workspace_bytes", "gdn_bwd_vg_workspace_bytes"):
            assert getattr(lib, fn)(ctypes.byref(dd), ctypes.byref(out)) == 0
            ws[fn, save] = out.value
    for fn in ("gdn_fwd_vg_workspace_bytes", "gdn_bwd_vg_workspace_bytes"):
        assert ws[fn, 1] < ws[fn, 0]
    f = _fake(10)
    args = list(f)
    args[9] = None  # ckpt
    assert lib.gdn_fwd_vg(ctypes.byref(d), *args, f[0], ws["gdn_fwd_vg_workspace_bytes", 1], None) == 1
    g = _fake(16)
    args = list(g)
    args[7] = None
    assert lib.gdn_bwd_vg(ctypes.byref(d), *args, g[0], ws["gdn_bwd_vg_workspace_bytes", 1], None) == 1


def test_tpar_segments_only_when_they_pay():
    """GDN_ALGO_CHUNK_TPAR splits a long sequence into segments (more
    workspace: the segment maps and start states) only when the single pass
    leaves most compute units idle; at the 9B shape it is the single pass."""
    def ws(algo, dims):
        return B.fwd_workspace_bytes(B.make_dims(*dims, B.GDN_BF16, algo))
    head = (1, 2048, 16, 64, 192, 128)
    assert ws(B.ALGO_CHUNK_TPAR, head) == ws(B.ALGO_CHUNK, head)
    long1 = (1, 32768, 2, 4, 128, 128)
    extra = ws(B.ALGO_CHUNK_TPAR, long1) - ws(B.ALGO_CHUNK, long1)
    # 16 segments (512 chunks / 32 each): maps [16, 4, 128, 256] + starts [15, 4, 128, 128]
    assert extra == 4 * (16 * 4 * 128 * 256 + 15 * 4 * 128 * 128) + 256
    bws = lambda algo, dims: B.bwd_workspace_bytes(B.make_dims(*dims, B.GDN_BF16, algo))
    assert bws(B.ALGO_CHUNK_TPAR, long1) - bws(B.ALGO_CHUNK, long1) == extra
    assert bws(B.ALGO_CHUNK_TPAR, head) == bws(B.ALGO_CHUNK, head)
    assert B.ckpt_elems(B.make_dims(*long1, B.GDN_BF16, B.ALGO_CHUNK_TPAR)) == \
        B.ckpt_elems(B.make_dims(*long1, B.GDN_BF16, B.ALGO_CHUNK))


@pytest.mark.parametrize("dims", [
    (64, 65536, 4, 8, 64, 32),      # 64x64 chunk matrices: 64*8*1024*8192 B = 4 GiB
    (24, 262144, 4, 8, 64, 32),     # 6 GiB of chunk matrices
    (4096, 65, 16, 16, 256, 32),    # transposed k rows of the ragged chunks: 4096*16*2*256*128 B = 4 GiB
])
def test_chunk_rejects_tensors_past_4gib(dims):
    """The chunk kernels reach their per-chunk tensors through buffer
    descriptors with 32-bit byte offsets; a shape whose chunk matrices or
    transposed k / q rows would reach 4 GiB is refused by CHUNK and
    CHUNK_TPAR (GDN_ERR_UNSUPPORTED) and runs the scan under AUTO, instead of
    wrapping its offsets."""
    for algo in (B.ALGO_CHUNK, B.ALGO_CHUNK_TPAR):
        for save in (False, True):
            d = B.make_dims(*dims, B.GDN_BF16, algo, save=save)
            for q in (B.fwd_workspace_bytes, B.bwd_workspace_bytes, B.ckpt_elems):
                with pytest.raises(B.GdnError) as e:
                    q(d)
                assert e.value.code == 2
    auto = B.make_dims(*dims, B.GDN_BF16, B.ALGO_AUTO, save=True)
    scan = B.make_dims(*dims, B.GDN_BF16, B.ALGO_SCAN)
    assert B.fwd_workspace_bytes(auto) == B.fwd_workspace_bytes(scan)
    assert B.ckpt_elems(auto) == B.ckpt_elems(scan)


def test_chunk_accepts_just_below_4gib():
    """One chunk fewer than the 4 GiB matrices: still the chunk form."""
    d = B.make_dims(64, 65536 - 64, 4, 8, 64, 32, B.GDN_BF16, B.ALGO_CHUNK)
    assert B.fwd_workspace_bytes(d) > 0
    auto = B.make_dims(64, 65536 - 64, 4, 8, 64, 32, B.GDN_BF16, B.ALGO_AUTO)
    assert B.fwd_workspace_bytes(auto) == B.fwd_workspace_bytes(d)


def test_in_place_forward_takes_the_single_pass():
    """state_out == state0 with a long few-head sequence: the T-parallel
    output pass would read state0 in its first segment while its last segment
    writes state_out, so the call runs the single pass.  Its workspace is the
    single pass's, so the T-parallel size is more than enough and a buffer of
    exactly the single pass's size is accepted (validated on the host; the
    short workspace check is the only one that depends on the route)."""
    lib = B.lib()
    dims = (1, 32768, 2, 4, 128, 128)
    dt = B.make_dims(*dims, B.GDN_BF16, B.ALGO_CHUNK_TPAR)
    single = B.fwd_workspace_bytes(B.make_dims(*dims, B.GDN_BF16, B.ALGO_CHUNK))
    assert B.fwd_workspace_bytes(dt) > single
    p = _fake(13)  # q k v a b A_log dt_bias state0 mask o state_out ckpt ws
    args = list(p)
    args[10] = None  # state_out missing: rejected before any launch either way
    assert lib.gdn_fwd(ctypes.byref(dt), *args, single, None) == 1
    args = list(p)
    args[10] = args[7]  # in place; a workspace one byte short of the single pass is refused
    assert lib.gdn_fwd(ctypes.byref(dt), *args, single - 1, None) == 3
    args = list(p)  # not in place: the T-parallel route needs its larger workspace
    assert lib.gdn_fwd(ctypes.byref(dt), *args, single, None) == 3


def test_byte_and_combined_size_queries():
    """gdn_ckpt_bytes = 4 * gdn_ckpt_elems; gdn_workspace_bytes(d, for_bwd)
    is the forward's or the backward's workspace query."""
    lib = B.lib()
    out = ctypes.c_size_t(0)
    for dims in [(1, 2048, 16, 64, 192, 128, B.GDN_BF16), (4, 65, 4, 8, 64, 32, B.GDN_F32)]:
        for save in (False, True):
            d = B.make_dims(*dims, save=save)
            assert lib.gdn_ckpt_bytes(ctypes.byref(d), ctypes.byref(out)) == 0
            assert out.value == 4 * B.ckpt_elems(d)
            assert lib.gdn_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(out)) == 0
            assert out.value == B.fwd_workspace_bytes(d)
            assert lib.gdn_workspace_bytes(ctypes.byref(d), 1, ctypes.byref(out)) == 0
            assert out.value == B.bwd_workspace_bytes(d)
    bad = B.make_dims(1, 8, 3, 4, 16, 8, B.GDN_F32)
    assert lib.gdn_ckpt_bytes(ctypes.byref(bad), ctypes.byref(out)) == 1
    assert lib.gdn_workspace_bytes(ctypes.byref(bad), 1, ctypes.byref(out)) == 1

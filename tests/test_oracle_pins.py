"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these re-types the oracle's own step: each compares it with a closed
form, a textbook special case, central differences, an identity that holds for
any correct implementation, or a second route to the same quantity.  Sources:
mlx-lm PR "Add gated_delta_update VJP" (sections "Numerical correctness" and
"Covered corner cases", "Design notes"; its extension "Associative prefix-scan
scaffold"); torch-to-nnef GDN page ("Op contract").
"""
import math

import numpy as np
import pytest

import oracle
from linear_attention_recurrence_fwd_amd import inputs

EPS = 1e-6


def rel(x, ref):
    x, ref = np.asarray(x), np.asarray(ref)
    den = np.max(np.abs(ref))
    return np.max(np.abs(x - ref)) / (den if den > 0 else 1.0)


def unit_rows(rng, shape):
    """Rows with |x|^2 + 1e-6 == 1, so the op's L2 normalisation leaves them
    unchanged (to rounding): the tests can then state results in terms of the
    raw vectors without re-deriving the normalisation."""
    x = rng.standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x * math.sqrt(1.0 - EPS)


# ----------------------------------------------------------------- gates

def test_gate_constants():
    """g = exp(-exp(A_log) softplus(a+dt_bias)), beta = sigmoid(b) at points
    where the value is a known constant (op contract's log-decay / beta)."""
    g, ell, beta = oracle.gates(0.0, 0.0, 0.0, 0.0)   # softplus(0) = ln 2
    assert g == pytest.approx(0.5, rel=1e-15) and beta == 0.5
    assert ell == pytest.approx(-math.log(2.0), rel=1e-15)
    g, _, beta = oracle.gates(0.0, math.log(3.0), math.log(2.0), 0.0)
    assert g == pytest.approx(0.25, rel=1e-15) and beta == pytest.approx(0.75, rel=1e-15)
    g, _, beta = oracle.gates(-1.0, 0.0, 0.0, 1.0)    # dt_bias enters additively
    assert g == pytest.approx(0.5, rel=1e-15)
    g, _, beta = oracle.gates(-800.0, 40.0, 1.0, 0.0)  # no decay, full write
    assert g == 1.0 and beta == 1.0


def test_softplus_clamp_upper_20():
    """The PR's clamp of the softplus argument: the argument is capped at 20 (read
    as an upper bound only).  Values at and above 20 give the same gate."""
    g20 = oracle.gates(20.0, 0.0, 0.0, 0.0)
    assert oracle.gates(25.0, 0.0, 0.0, 0.0) == g20
    assert oracle.gates(15.0, 0.0, 0.0, 5.0) == g20
    assert oracle.gates(19.5, 0.0, 0.0, 0.0)[1] > g20[1]
    # softplus(20) = 20 + log1p(e^-20)
    assert -g20[1] == pytest.approx(20.0 + math.log1p(math.exp(-20.0)), rel=1e-15)


# ------------------------------------------------------- T = 1 closed form

def t1_case(rng, Dk=16, Dv=8, A_log=0.0, b=0.0):
    q = unit_rows(rng, (1, 1, 1, Dk))
    k = unit_rows(rng, (1, 1, 1, Dk))
    v = rng.standard_normal((1, 1, 1, Dv))
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    a = np.zeros((1, 1, 1))
    bb = np.full((1, 1, 1), b)
    return q, k, v, a, bb, np.array([A_log]), np.zeros(1), S0


@pytest.mark.parametrize("A_log,b,g,beta", [(0.0, 0.0, 0.5, 0.5),
                                            (math.log(2.0), math.log(3.0), 0.25, 0.75)])
def test_t1_closed_form(A_log, b, g, beta):
    """One step from S0:  with P = I - beta k k^T,
    S1 = g P S0 + beta k v^T  and  o = S1^T q / sqrt(Dk)
    (decay, read, correct, write, then read out from the updated state)."""
    rng = np.random.default_rng(11)
    q, k, v, a, bb, Al, dt, S0 = t1_case(rng, A_log=A_log, b=b)
    Dk = q.shape[-1]
    o, S1, ck = oracle.fwd(q, k, v, a, bb, Al, dt, S0)
    kk, qq, vv, S = k[0, 0, 0], q[0, 0, 0], v[0, 0, 0], S0[0, 0]
    P = np.eye(Dk) - beta * np.outer(kk, kk)
    S1_ref = g * P @ S + beta * np.outer(kk, vv)
    o_ref = S1_ref.T @ qq / math.sqrt(Dk)
    assert rel(S1[0, 0], S1_ref) < 1e-13
    assert rel(o[0, 0, 0], o_ref) < 1e-13
    assert ck.shape[0] == 0


def test_t1_closed_form_gradients():
    """VJP of the single step, written from the closed form above:
    with M = dS1 + q dO^T (q already scaled), the pieces that do not involve
    the normalisation are  dv = beta M^T k,  dS0 = g P M."""
    rng = np.random.default_rng(12)
    q, k, v, a, bb, Al, dt, S0 = t1_case(rng)
    g, beta = 0.5, 0.5
    Dk = q.shape[-1]
    dO = rng.standard_normal(v.shape)
    dS = rng.standard_normal(S0.shape)
    gr = oracle.bwd(q, k, v, a, bb, Al, dt, S0, None, dO, dS)
    kk, qq = k[0, 0, 0], q[0, 0, 0] / math.sqrt(Dk)
    M = dS[0, 0] + np.outer(qq, dO[0, 0, 0])
    P = np.eye(Dk) - beta * np.outer(kk, kk)
    assert rel(gr["dv"][0, 0, 0], beta * M.T @ kk) < 1e-12
    assert rel(gr["dstate"][0, 0], g * P @ M) < 1e-12


def test_eps_inside_the_square_root():
    """Op contract: q/k are L2-normalised with eps 1e-6; read as
    x (|x|^2 + eps)^(-1/2).  For |q|^2 = eps the normalised q is q_unit/sqrt(2)
    (rms_norm-style eps*Dk, or eps outside the root, would give other ratios).
    o is linear in the normalised q, so o(q) / o(q_unit) pins the placement."""
    rng = np.random.default_rng(13)
    q, k, v, a, bb, Al, dt, S0 = t1_case(rng)
    qu = q / np.linalg.norm(q)                      # |qu| = 1
    qs = qu * math.sqrt(EPS)                        # |qs|^2 = eps
    o_u = oracle.fwd(qu, k, v, a, bb, Al, dt, S0)[0]
    o_s = oracle.fwd(qs, k, v, a, bb, Al, dt, S0)[0]
    ratio = math.sqrt(EPS) / math.sqrt(2 * EPS) * math.sqrt(1 + EPS)
    assert rel(o_s, ratio * o_u) < 1e-12


# ------------------------------------------------------------ FD, all grads

def loss(case_vals, mask, o, ST):
    L = np.sum(o * case_vals["dO"])
    if case_vals.get("dS_final") is not None:
        L += np.sum(ST * case_vals["dS_final"])
    return L


def fd_check(c, names=("q", "k", "v", "a", "b", "A_log", "dt_bias", "state0"),
             h=2.0 ** -20, tol=2e-7):
    vals = {n: x.copy() for n, x in c.vals.items()}
    gr = oracle.bwd(*c.oracle_args(), vals["dO"], vals.get("dS_final"))
    gmap = dict(q="dq", k="dk", v="dv", a="da", b="db", A_log="dA_log",
                dt_bias="ddt_bias", state0="dstate")

    def L():
        args = (vals["q"], vals["k"], vals["v"], vals["a"], vals["b"], vals["A_log"],
                vals["dt_bias"], vals.get("state0"), c.mask)
        o, st, _ = oracle.fwd(*args)
        return loss(vals, c.mask, o, st)

    for n in names:
        x = vals[n]
        fd = np.empty_like(x)
        flat, ff = x.reshape(-1), fd.reshape(-1)
        for i in range(flat.size):
            x0 = flat[i]
            flat[i] = x0 + h
            lp = L()
            flat[i] = x0 - h
            lm = L()
            flat[i] = x0
            ff[i] = (lp - lm) / (2 * h)
        err = rel(gr[gmap[n]], fd)
        assert err < tol, (n, err)
    return gr


def test_fd_tiny_all_gradients():
    """The PR's toy shape (B=1,T=8,Hk=2,Hv=4,Dk=16,Dv=8) checked against
    central differences for all eight gradients, here in fp64 (step 2^-20)."""
    fd_check(inputs.tiny())


def test_fd_masked_and_clamped():
    """FD through the masked path (PR: "FD through masked path") and across
    the softplus clamp (steps with a+dt_bias > 20 get da = 0)."""
    c = inputs.make_case("fdmask", 2, 6, 1, 2, 8, 4, "f32", 21,
                         mask=np.array([[1, 1, 0, 1, 0, 0], [1, 1, 1, 1, 1, 1]]))
    c.vals["a"][0, 1, :] = 30.0     # clamped step, valid
    c.vals["a"][1, 3, 1] = 19.0     # close below the clamp
    gr = fd_check(c)
    assert np.all(gr["da"][0, 1, :] == 0.0)
    assert np.all(gr["da"][0, [2, 4, 5], :] == 0.0)
    assert np.all(gr["db"][0, [2, 4, 5], :] == 0.0)
    assert np.all(gr["dv"][0, [2, 4, 5]] == 0.0)
    assert abs(gr["da"][1, 3, 1]) > 0.0


# --------------------------------------------------- chunking and masking

def test_chunked_equals_unchunked_bitwise():
    """Checkpointing every 64 steps and recomputing inside a chunk changes
    only the blocking, not the arithmetic (PR "Design notes"; torch-to-nnef:
    chunked and recurrent forms agree up to reordering)."""
    c = inputs.edge(65, masked=True)
    ref = oracle.bwd(*c.oracle_args(), c.vals["dO"], c.vals["dS_final"], chunk=0)
    for ch in (64, 7, 1):
        got = oracle.bwd(*c.oracle_args(), c.vals["dO"], c.vals["dS_final"], chunk=ch)
        for n in ref:
            assert np.array_equal(ref[n], got[n]), (ch, n)


def test_ckpt_is_prefix_state():
    """The checkpoint after 64c steps equals the final state of a run over
    the first 64c steps, bit for bit."""
    c = inputs.edge(130, masked=True)
    v = c.vals
    o, st, ck = oracle.fwd(*c.oracle_args())
    assert ck.shape[0] == 2
    for i, n in enumerate((64, 128)):
        sl = lambda x: x[:, :n]
        _, st_n, _ = oracle.fwd(sl(v["q"]), sl(v["k"]), sl(v["v"]), sl(v["a"]), sl(v["b"]),
                                v["A_log"], v["dt_bias"], v["state0"], c.mask[:, :n])
        assert np.array_equal(ck[i], st_n)


def test_mask_all_true_equals_unmasked():
    c = inputs.edge(65, masked=False)
    args = list(c.oracle_args())
    o0, s0, _ = oracle.fwd(*args)
    args[-1] = np.ones((c.B, c.T), np.uint8)
    o1, s1, _ = oracle.fwd(*args)
    assert np.array_equal(o0, o1) and np.array_equal(s0, s1)
    g0 = oracle.bwd(*c.oracle_args(), c.vals["dO"], c.vals["dS_final"])
    g1 = oracle.bwd(*args, c.vals["dO"], c.vals["dS_final"])
    for n in g0:
        assert np.array_equal(g0[n], g1[n]), n


def test_half_mask_final_state_is_prefix_state():
    """PR "Covered corner cases": a half-masked sequence's final state equals
    the state after its unmasked prefix only."""
    c = inputs.edge(65, masked=True)
    v = c.vals
    _, st, _ = oracle.fwd(*c.oracle_args())
    n = c.T // 2
    sl = lambda x: x[:, :n]
    _, st_p, _ = oracle.fwd(sl(v["q"]), sl(v["k"]), sl(v["v"]), sl(v["a"]), sl(v["b"]),
                            v["A_log"], v["dt_bias"], v["state0"])
    assert np.array_equal(st[1], st_p[1]) and np.array_equal(st[3], st_p[3])


def test_masked_step_equals_identity_step():
    """A masked step leaves S unchanged and reads o from it; the same happens
    for a valid step with g = 1 and beta = 0 exactly (a = b = -800 in fp64),
    so the two runs agree in every output and gradient."""
    c = inputs.edge(65, masked=True)
    v = c.vals
    gm = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    om, sm, _ = oracle.fwd(*c.oracle_args())
    a2, b2 = v["a"].copy(), v["b"].copy()
    off = c.mask == 0
    a2[off] = -800.0
    b2[off] = -800.0
    args = (v["q"], v["k"], v["v"], a2, b2, v["A_log"], v["dt_bias"], v["state0"], None)
    oi, si, _ = oracle.fwd(*args)
    gi = oracle.bwd(*args, v["dO"], v["dS_final"])
    assert np.array_equal(om, oi) and np.array_equal(sm, si)
    for n in gm:
        assert rel(gi[n], gm[n]) < 1e-15, n


# -------------------------------------------------------- extreme gates

@pytest.mark.parametrize("masked", [False, True])
def test_extreme_gates_finite_and_exact(masked):
    """PR: A_log = 5, a = 15 gives no NaN/Inf.  There g underflows to exactly
    0, so every valid step starts from the zero state: o_t does not depend on
    anything before t, the final state is rank one along k_T, and the gate
    gradients vanish."""
    c = inputs.edge(65, masked=masked, extreme=True)
    v = c.vals
    o, st, _ = oracle.fwd(*c.oracle_args())
    gr = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    assert np.isfinite(o).all() and np.isfinite(st).all()
    for n, x in gr.items():
        assert np.isfinite(x).all(), n
    assert np.all(gr["da"] == 0) and np.all(gr["dA_log"] == 0) and np.all(gr["ddt_bias"] == 0)
    # independence from the past: perturb state0 and all inputs before t = 40
    v2 = {n: x.copy() for n, x in v.items()}
    v2["state0"] += 1.0
    v2["v"][:, :40] += 1.0
    o2, st2, _ = oracle.fwd(v2["q"], v2["k"], v2["v"], v2["a"], v2["b"], v2["A_log"],
                            v2["dt_bias"], v2["state0"], c.mask)
    valid = np.ones((c.B, c.T), bool) if c.mask is None else c.mask.astype(bool)
    # a valid step t >= 40 sees only itself
    sel = valid.copy()
    sel[:, :40] = False
    assert np.array_equal(o[sel], o2[sel])
    # final state of an all-valid row is beta_T * khat_T v_T^T (rank one)
    kT = v["k"][0, -1]
    for h in range(c.Hv):
        S = st[0, h]
        kk = kT[h // c.G]
        coef = S.T @ kk / (kk @ kk)
        assert rel(S, np.outer(kk, coef)) < 1e-14
        assert rel(coef, coef @ v["v"][0, -1, h] / (v["v"][0, -1, h] @ v["v"][0, -1, h])
                   * v["v"][0, -1, h]) < 1e-14


# ------------------------------------------------------------- identities

@pytest.mark.parametrize("case", ["tiny", "edge65"])
def test_euler_homogeneity(case):
    """(o, S_T) are jointly linear in (v, S0), so
    sum <dv, v> + <dstate, S0> = sum <dO, o> + <dS_final, S_T>."""
    c = inputs.tiny() if case == "tiny" else inputs.edge(65, masked=True)
    v = c.vals
    o, st, _ = oracle.fwd(*c.oracle_args())
    gr = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    lhs = np.sum(gr["dv"] * v["v"]) + np.sum(gr["dstate"] * v["state0"])
    rhs = np.sum(v["dO"] * o) + np.sum(v["dS_final"] * st)
    assert abs(lhs - rhs) <= 1e-12 * (abs(rhs) + np.sum(np.abs(v["dO"] * o)))


def test_qk_scale_invariance():
    """The output depends on q, k only through their directions (up to eps),
    so <dq, q> and <dk, k> vanish per row to O(eps/|x|^2)."""
    c = inputs.edge(64, masked=True)
    v = c.vals
    gr = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    for x, dx in ((v["q"], gr["dq"]), (v["k"], gr["dk"])):
        dots = np.sum(x * dx, axis=-1)
        scale = np.linalg.norm(x, axis=-1) * np.linalg.norm(dx, axis=-1)
        bound = 4 * EPS / np.sum(x * x, axis=-1) + 1e-13
        assert np.all(np.abs(dots) <= bound * scale + 1e-300)


def test_associative_affine_composition():
    """PR extension "Associative prefix-scan scaffold": a valid step is the
    affine map S -> A_t S + B_t with A_t = g_t (I - beta_t k_t k_t^T) and
    B_t = beta_t k_t v_t^T; composing the maps in a tree bracketing must give
    the scan's final state.  Gates are chosen with known values: x = 0 so
    softplus = ln 2 and g = 2^-exp(A_log); beta from b in {0, ln 3, -ln 3}."""
    rng = np.random.default_rng(14)
    B, T, Hk, Hv, Dk, Dv = 1, 13, 1, 2, 8, 5
    k = unit_rows(rng, (B, T, Hk, Dk))
    q = unit_rows(rng, (B, T, Hk, Dk))
    v = rng.standard_normal((B, T, Hv, Dv))
    bsel = rng.integers(0, 3, (B, T, Hv))
    b = np.array([0.0, math.log(3.0), -math.log(3.0)])[bsel]
    beta = np.array([0.5, 0.75, 0.25])[bsel]
    a = np.zeros((B, T, Hv))
    A_log = np.array([0.0, math.log(2.0)])
    gval = np.array([0.5, 0.25])
    S0 = rng.standard_normal((B, Hv, Dk, Dv))
    _, st, _ = oracle.fwd(q, k, v, a, b, A_log, np.zeros(Hv), S0)
    for h in range(Hv):
        maps = []
        for t in range(T):
            kk = k[0, t, 0]
            maps.append((gval[h] * (np.eye(Dk) - beta[0, t, h] * np.outer(kk, kk)),
                         beta[0, t, h] * np.outer(kk, v[0, t, h])))
        while len(maps) > 1:   # (A2,B2) o (A1,B1) = (A2 A1, A2 B1 + B2), pairwise
            nxt = []
            for i in range(0, len(maps) - 1, 2):
                (A1, B1), (A2, B2) = maps[i], maps[i + 1]
                nxt.append((A2 @ A1, A2 @ B1 + B2))
            if len(maps) % 2:
                nxt.append(maps[-1])
            maps = nxt
        A, Bm = maps[0]
        assert rel(st[0, h], A @ S0[0, h] + Bm) < 1e-13


def test_delta_rule_textbook_lms():
    """With g = 1 and beta = 1 the step is the classic delta (Widrow-Hoff)
    rule: writing values under orthogonal keys into an empty state and reading
    one back returns it, and rewriting a key replaces its value; with the
    keys' norm |k|^2 = 1 - eps the reads carry the known factor 1 - eps."""
    Dk, Dv = 6, 3
    rng = np.random.default_rng(15)
    c = math.sqrt(1.0 - EPS)
    T = Dk + 2
    k = np.zeros((1, T, 1, Dk))
    q = np.zeros((1, T, 1, Dk))
    for t in range(Dk):
        k[0, t, 0, t] = c
    k[0, Dk, 0, 0] = c            # rewrite key 0
    k[0, Dk + 1, 0, 3] = c        # rewrite key 3
    q[0, :, 0, 0] = 1.0           # always read key 0
    v = rng.standard_normal((1, T, 1, Dv))
    a = np.full((1, T, 1), -800.0)
    b = np.full((1, T, 1), 40.0)
    o, st, _ = oracle.fwd(q, k, v, a, b, np.zeros(1), np.zeros(1))
    qs = 1.0 / math.sqrt(1.0 + EPS) / math.sqrt(Dk)   # normalised, scaled q
    v0, v0new = v[0, 0, 0], v[0, Dk, 0]
    assert rel(o[0, 0, 0], c * qs * v0) < 1e-14
    assert rel(o[0, Dk - 1, 0], c * qs * v0) < 1e-14
    # after the rewrite: S^T k0 = c^2 v' + c^2 (1 - c^2) v0
    expect = c * qs * (v0new + (1 - c * c) * v0)
    assert rel(o[0, Dk, 0], expect) < 1e-12
    # rewriting key 3 does not disturb key 0
    assert rel(o[0, Dk + 1, 0], expect) < 1e-12


def test_gqa_equals_repeated_heads():
    """Op contract: value head h reads q/k head h // G, and q/k are not
    repeated at the boundary.  Running with q/k repeat-interleaved to Hv heads
    (G = 1) gives the same outputs, and the shared-head gradients are the sums
    over the copies."""
    c = inputs.tiny()
    v = c.vals
    G = c.G
    rep = lambda x: np.repeat(x, G, axis=2)
    args_r = (rep(v["q"]), rep(v["k"]), v["v"], v["a"], v["b"], v["A_log"], v["dt_bias"],
              v["state0"], None)
    o, st, _ = oracle.fwd(*c.oracle_args())
    o_r, st_r, _ = oracle.fwd(*args_r)
    assert np.array_equal(o, o_r) and np.array_equal(st, st_r)
    g = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    g_r = oracle.bwd(*args_r, v["dO"], v["dS_final"])
    for n in ("dq", "dk"):
        summed = g_r[n].reshape(c.B, c.T, c.Hk, G, c.Dk).sum(axis=3)
        assert rel(g[n], summed) < 1e-13
    for n in ("dv", "da", "db", "dA_log", "ddt_bias", "dstate"):
        assert rel(g[n], g_r[n]) < 1e-14


def test_state_carry_segments():
    """fwd over [0, T1) then over [T1, T) from its final state equals one run
    over [0, T), bit for bit; the backward chains through dstate."""
    c = inputs.edge(65, masked=True)
    v = c.vals
    T1 = 23
    o, st, _ = oracle.fwd(*c.oracle_args())
    s1 = lambda x: x[:, :T1]
    s2 = lambda x: x[:, T1:]
    a1 = (s1(v["q"]), s1(v["k"]), s1(v["v"]), s1(v["a"]), s1(v["b"]), v["A_log"],
          v["dt_bias"], v["state0"], s1(c.mask))
    o1, st1, _ = oracle.fwd(*a1)
    a2 = (s2(v["q"]), s2(v["k"]), s2(v["v"]), s2(v["a"]), s2(v["b"]), v["A_log"],
          v["dt_bias"], st1, s2(c.mask))
    o2, st2, _ = oracle.fwd(*a2)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o) and np.array_equal(st2, st)
    g = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    g2 = oracle.bwd(*a2, s2(v["dO"]), v["dS_final"])
    g1 = oracle.bwd(*a1, s1(v["dO"]), g2["dstate"])
    assert np.array_equal(g["dstate"], g1["dstate"])
    for n in ("dq", "dk", "dv", "da", "db"):
        assert np.array_equal(g[n], np.concatenate([g1[n], g2[n]], axis=1)), n
    for n in ("dA_log", "ddt_bias"):
        assert rel(g[n], g1[n] + g2[n]) < 1e-13


def test_decode_steps_equal_one_call():
    """Decode: T single-step calls, each starting from the previous state,
    reproduce one call over all T steps."""
    c = inputs.make_case("dec_small", 3, 9, 2, 4, 16, 8, "bf16", 31, dS_final=False)
    v = c.vals
    o, st, _ = oracle.fwd(*c.oracle_args())
    S = v["state0"]
    for t in range(c.T):
        sl = lambda x: x[:, t:t + 1]
        o_t, S, _ = oracle.fwd(sl(v["q"]), sl(v["k"]), sl(v["v"]), sl(v["a"]), sl(v["b"]),
                               v["A_log"], v["dt_bias"], S)
        assert np.array_equal(o_t, o[:, t:t + 1])
    assert np.array_equal(S, st)


def test_empty_sequence():
    """T = 0: the state passes through, nothing else is produced."""
    c = inputs.make_case("empty", 2, 0, 1, 2, 8, 4, "f32", 32)
    v = c.vals
    o, st, ck = oracle.fwd(*c.oracle_args())
    assert o.shape == (2, 0, 2, 4) and np.array_equal(st, v["state0"]) and ck.shape[0] == 0
    g = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    assert np.array_equal(g["dstate"], v["dS_final"])
    assert np.all(g["dA_log"] == 0) and np.all(g["ddt_bias"] == 0)


# ------------------------------------------------- conv update (decode path)
# Depthwise causal conv1d + SiLU with a k-sample carry state (torch-to-nnef
# GDN page, the causal-conv-update drop-in: hidden_states [b, C, S],
# conv_state [b, C, k], weight [C, k] -> out [b, C, S], final_state [b, C, k]).

def silu_ref(z):
    return z / (1.0 + np.exp(-z))


def test_silu_closed_form():
    """SiLU(0) = 0 and SiLU(ln 3) = (3/4) ln 3 (sigmoid(ln 3) = 3/4): a zero
    state and a single unit tap turn the conv update into SiLU of the input."""
    x = np.array([0.0, math.log(3.0), -math.log(3.0)]).reshape(1, 3, 1)
    w = np.zeros((3, 2))
    w[:, 1] = 1.0
    out, _ = oracle.conv_update(x, np.zeros((1, 3, 2)), w)
    assert out[0, 0, 0] == 0.0
    assert abs(out[0, 1, 0] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(out[0, 2, 0] + 0.25 * math.log(3.0)) < 1e-15


def test_conv_delta_taps_shift_the_state():
    """Taps (0, .., 0, 1): the output is SiLU of the newest sample, and the
    state shifts by one sample per step with the new sample appended."""
    rng = np.random.default_rng(60)
    B, C, K = 2, 5, 4
    x = rng.standard_normal((B, C, 1))
    st = rng.standard_normal((B, C, K))
    w = np.zeros((C, K))
    w[:, -1] = 1.0
    out, fin = oracle.conv_update(x, st, w)
    assert np.allclose(out, silu_ref(x), rtol=1e-15, atol=0)
    assert np.array_equal(fin[:, :, :-1], st[:, :, 1:]) and np.array_equal(fin[:, :, -1], x[:, :, 0])


def test_conv_matches_library_convolution():
    """Brute force against numpy's convolution of the carried samples followed
    by the new ones: output s is the 'valid' convolution at position s + 1
    (the window of the k newest samples ending at new sample s)."""
    rng = np.random.default_rng(61)
    B, C, K, S = 2, 3, 4, 6
    x = rng.standard_normal((B, C, S))
    st = rng.standard_normal((B, C, K))
    w = rng.standard_normal((C, K))
    out, fin = oracle.conv_update(x, st, w)
    for bi in range(B):
        for c in range(C):
            ext = np.concatenate([st[bi, c], x[bi, c]])
            z = np.convolve(ext, w[c][::-1], mode="valid")[1:]
            assert np.allclose(out[bi, c], silu_ref(z), rtol=1e-13, atol=1e-15)
            assert np.array_equal(fin[bi, c], ext[-K:])


def test_conv_single_steps_equal_one_call():
    """S single-sample updates, each from the previous final state, reproduce
    one update over the S samples."""
    rng = np.random.default_rng(62)
    B, C, K, S = 2, 4, 3, 7
    x = rng.standard_normal((B, C, S))
    st = rng.standard_normal((B, C, K))
    w = rng.standard_normal((C, K))
    out, fin = oracle.conv_update(x, st, w)
    cur = st
    for s in range(S):
        o1, cur = oracle.conv_update(x[:, :, s:s + 1], cur, w)
        assert np.array_equal(o1[:, :, 0], out[:, :, s])
    assert np.array_equal(cur, fin)


def test_decode_conv_masked_row_keeps_both_states():
    """A masked batch row of the decode step with conv update keeps its conv
    state and its recurrent state; the unmasked rows equal the unmasked call."""
    rng = np.random.default_rng(63)
    B, Hk, Hv, Dk, Dv, K = 3, 1, 2, 8, 4, 4
    C = 2 * Hk * Dk + Hv * Dv
    x = rng.standard_normal((B, C))
    cs = rng.standard_normal((B, C, K))
    w = rng.standard_normal((C, K)) * 0.5
    a, b = rng.standard_normal((B, Hv)), rng.standard_normal((B, Hv))
    A_log, dt_bias = rng.uniform(0, 2, Hv), rng.standard_normal(Hv) * 0.5
    s0 = rng.standard_normal((B, Hv, Dk, Dv)) * 0.1
    mask = np.array([1, 0, 1])
    o, st, fin = oracle.decode_conv(x, cs, w, a, b, A_log, dt_bias, Hk, Dk, Hv, Dv, state0=s0, mask=mask)
    o1, st1, fin1 = oracle.decode_conv(x, cs, w, a, b, A_log, dt_bias, Hk, Dk, Hv, Dv, state0=s0)
    assert np.array_equal(fin[1], cs[1]) and np.array_equal(st[1], s0[1])
    for r in (0, 2):
        assert np.array_equal(fin[r], fin1[r]) and np.array_equal(st[r], st1[r]) and np.array_equal(o[r], o1[r])


# ------------------------------------------ per-key-channel (vector) gates
#
# mlx-lm PR, "Models covered" / "Scope and follow-ups": Kimi-Linear runs the
# rule with a gate per key channel (g.ndim == 4).  The gate vector g_t scales
# the rows of the state; the caller gives lg = log g.

def _nrm(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def vg_brute_fwd(q, k, v, lg, b, state0, mask):
    """The step as a transition map, S_t = (I - beta k k^T) diag(g) S + beta k v^T,
    o_t = S_t^T q / sqrt(Dk), with dense numpy products per (b, h); masked steps
    are the identity map.  Returns (o, S_T, states at t = 64, 128, ...)."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    G = Hv // Hk
    kn, qn = _nrm(k), _nrm(q) / math.sqrt(Dk)
    beta = 1.0 / (1.0 + np.exp(-b))
    o = np.zeros((B, T, Hv, Dv))
    ST = np.zeros((B, Hv, Dk, Dv))
    nck = max((T + 63) // 64 - 1, 0)
    ck = np.zeros((nck, B, Hv, Dk, Dv))
    for bi in range(B):
        for h in range(Hv):
            S = np.zeros((Dk, Dv)) if state0 is None else state0[bi, h].copy()
            for t in range(T):
                if mask is None or mask[bi, t]:
                    kk = kn[bi, t, h // G]
                    A = (np.eye(Dk) - beta[bi, t, h] * np.outer(kk, kk)) @ np.diag(np.exp(lg[bi, t, h]))
                    S = A @ S + beta[bi, t, h] * np.outer(kk, v[bi, t, h])
                o[bi, t, h] = S.T @ qn[bi, t, h // G]
                if (t + 1) % 64 == 0 and t + 1 < T:
                    ck[(t + 1) // 64 - 1, bi, h] = S
            ST[bi, h] = S
    return o, ST, ck


def test_vg_matches_transition_map_form():
    """Forward with per-channel gates equals the dense transition-map form,
    including masked steps and a checkpoint (T = 70)."""
    c = inputs.make_vg_case("vgb", 2, 70, 1, 2, 8, 5, "f32", 31,
                            mask=np.array([[1] * 70, [1] * 30 + [0, 1] * 20]))
    args = c.vg_args()
    o, st, ck = oracle.fwd_vg(*args)
    o_r, st_r, ck_r = vg_brute_fwd(*args)
    assert rel(o, o_r) < 1e-12 and rel(st, st_r) < 1e-12
    assert ck.shape == ck_r.shape and rel(ck, ck_r) < 1e-12


def test_vg_t1_closed_form_gradients():
    """One step, S1 = P diag(g) S0 + beta k v^T with P = I - beta k k^T.  With
    M = dS1 + q dO^T: dS0 = diag(g) P M and d(lg)_i = g_i ((P M) o S0)_i summed
    over the row, dv = beta M^T k.  Distinct gates per channel, so a gate
    applied to columns, a missing g_i factor or a gradient taken against the
    decayed state all show."""
    rng = np.random.default_rng(32)
    Dk, Dv = 6, 4
    q = unit_rows(rng, (1, 1, 1, Dk))
    k = unit_rows(rng, (1, 1, 1, Dk))
    v = rng.standard_normal((1, 1, 1, Dv))
    lg = -rng.uniform(0.05, 2.0, (1, 1, 1, Dk))
    b = np.full((1, 1, 1), math.log(3.0))   # beta = 3/4
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    dO = rng.standard_normal((1, 1, 1, Dv))
    dS = rng.standard_normal((1, 1, Dk, Dv))
    beta, g = 0.75, np.exp(lg[0, 0, 0])
    kk, qq = k[0, 0, 0], q[0, 0, 0] / math.sqrt(Dk)
    P = np.eye(Dk) - beta * np.outer(kk, kk)
    S1 = P @ np.diag(g) @ S0[0, 0] + beta * np.outer(kk, v[0, 0, 0])
    o, st, _ = oracle.fwd_vg(q, k, v, lg, b, S0)
    assert rel(st[0, 0], S1) < 1e-13 and rel(o[0, 0, 0], S1.T @ qq) < 1e-13
    gr = oracle.bwd_vg(q, k, v, lg, b, S0, None, dO, dS)
    M = dS[0, 0] + np.outer(qq, dO[0, 0, 0])
    assert rel(gr["dstate"][0, 0], np.diag(g) @ P @ M) < 1e-12
    assert rel(gr["dlg"][0, 0, 0], g * np.sum((P @ M) * S0[0, 0], axis=1)) < 1e-12
    assert rel(gr["dv"][0, 0, 0], beta * M.T @ kk) < 1e-12


def fd_check_vg(c, h=2.0 ** -20, tol=2e-7):
    vals = {n: x.copy() for n, x in c.vals.items()}
    gr = oracle.bwd_vg(*c.vg_args(), vals["dO"], vals.get("dS_final"))
    gmap = dict(q="dq", k="dk", v="dv", lg="dlg", b="db", state0="dstate")

    def L():
        o, st, _ = oracle.fwd_vg(vals["q"], vals["k"], vals["v"], vals["lg"], vals["b"],
                                 vals.get("state0"), c.mask)
        return loss(vals, c.mask, o, st)

    for n in gmap:
        x = vals[n]
        fd = np.empty_like(x)
        flat, ff = x.reshape(-1), fd.reshape(-1)
        for i in range(flat.size):
            x0 = flat[i]
            flat[i] = x0 + h
            lp = L()
            flat[i] = x0 - h
            lm = L()
            flat[i] = x0
            ff[i] = (lp - lm) / (2 * h)
        err = rel(gr[gmap[n]], fd)
        assert err < tol, (n, err)
    return gr


def test_vg_fd_all_gradients():
    """Central differences for all six gradients of the per-channel-gate form
    on the PR's toy shape."""
    fd_check_vg(inputs.vg_tiny())


def test_vg_fd_masked():
    """FD through masked steps; masked steps get dv = dlg = db = 0."""
    c = inputs.make_vg_case("vgfdm", 2, 6, 1, 2, 8, 4, "f32", 33,
                            mask=np.array([[1, 1, 0, 1, 0, 0], [1, 1, 1, 1, 1, 1]]))
    gr = fd_check_vg(c)
    assert np.all(gr["dlg"][0, [2, 4, 5]] == 0.0)
    assert np.all(gr["db"][0, [2, 4, 5]] == 0.0)
    assert np.all(gr["dv"][0, [2, 4, 5]] == 0.0)


def test_vg_uniform_channels_equal_scalar_gate():
    """With every channel's log-gate equal to the scalar gate's l, the
    per-channel form is the scalar one: same o and state, and the channel sum
    of d(lg) equals dl = da / (-exp(A_log) sigmoid(x)) (x below the clamp)."""
    c = inputs.edge(65, masked=True)
    v = c.vals
    B, T, Hv, Dk = c.B, c.T, c.Hv, c.Dk
    ell = np.empty((B, T, Hv))
    for bi in range(B):
        for t in range(T):
            for h in range(Hv):
                ell[bi, t, h] = oracle.gates(v["a"][bi, t, h], 0.0, v["A_log"][h], v["dt_bias"][h])[1]
    lg = np.repeat(ell[..., None], Dk, axis=3)
    o, st, ck = oracle.fwd(*c.oracle_args())
    o2, st2, ck2 = oracle.fwd_vg(v["q"], v["k"], v["v"], lg, v["b"], v["state0"], c.mask)
    assert rel(o2, o) < 1e-13 and rel(st2, st) < 1e-13 and rel(ck2, ck) < 1e-13
    g1 = oracle.bwd(*c.oracle_args(), v["dO"], v["dS_final"])
    g2 = oracle.bwd_vg(v["q"], v["k"], v["v"], lg, v["b"], v["state0"], c.mask, v["dO"],
                       v["dS_final"])
    for n in ("dq", "dk", "dv", "db", "dstate"):
        assert rel(g2[n], g1[n]) < 1e-12, n
    x = v["a"] + v["dt_bias"]
    dl = g1["da"] / (-np.exp(v["A_log"]) / (1.0 + np.exp(-x)))
    assert rel(g2["dlg"].sum(axis=3), dl) < 1e-10


def test_vg_chunked_equals_unchunked_bitwise():
    c = inputs.vg_edge(65, masked=True)
    ref = oracle.bwd_vg(*c.vg_args(), c.vals["dO"], c.vals["dS_final"], chunk=0)
    for ch in (64, 5):
        got = oracle.bwd_vg(*c.vg_args(), c.vals["dO"], c.vals["dS_final"], chunk=ch)
        for n in ref:
            assert np.array_equal(ref[n], got[n]), (ch, n)


def test_vg_euler_homogeneity():
    """(o, S_T) are jointly linear in (v, S0) for any gates."""
    c = inputs.vg_edge(65, masked=True)
    v = c.vals
    o, st, _ = oracle.fwd_vg(*c.vg_args())
    gr = oracle.bwd_vg(*c.vg_args(), v["dO"], v["dS_final"])
    lhs = np.sum(gr["dv"] * v["v"]) + np.sum(gr["dstate"] * v["state0"])
    rhs = np.sum(v["dO"] * o) + np.sum(v["dS_final"] * st)
    assert abs(lhs - rhs) <= 1e-12 * (abs(rhs) + np.sum(np.abs(v["dO"] * o)))

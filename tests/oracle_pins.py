"""Pins that tie the fp64 oracle to what the sources and the mathematics fix.

Each ``pin_*`` takes the oracle module and raises AssertionError (or any
exception) when the oracle disagrees with something independent of it:
exact rational identities between *different* algorithms (Theorem 2 of
"Dion3: Full-Stack Orthogonal Updates"), closed forms built from the
definition p_t(x) = a_t x + b_t x^3 + c_t x^5 with numpy's polynomial and SVD
routines, the textbook polar factor, printed FLOP counts and invariants.

The same pins are run against deliberately broken copies of the oracle in
``test_oracle_mutations.py`` to show that a plausible mistake anywhere in it
is caught.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction as F

import numpy as np
from numpy.polynomial import Polynomial

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Distinct coefficients per iteration, so that any mix-up of the iteration
# index or of the (a, b, c) roles changes the result.
SCHED3 = [(F(3, 2), F(-1, 2), F(1, 8)),
          (F(15, 8), F(-10, 8), F(3, 8)),
          (F("3.4445"), F("-4.7750"), F("2.0315"))]
SCHED4 = SCHED3 + [(F(2), F(-3, 2), F(1, 2))]
EPS = F(1, 10 ** 7)

# 3 x 5 integer matrix with ||X||_F = 9 and 2 x 2 with ||X||_F = 7.
X35 = [[-1, -2, 4, 1, 4], [-1, 0, 0, 2, 0], [4, -3, 0, -2, 3]]
X22 = [[2, 4], [5, 2]]


def load_schedules():
    out = {}
    with open(os.path.join(GOLDEN, "coefficients.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                out[line[0]] = tuple(F(v) for v in line[1:4])
    return out


def _exact(rows):
    return np.array([[F(v) for v in r] for r in rows], dtype=object)


def _eq(A, B):
    A, B = np.asarray(A), np.asarray(B)
    return A.shape == B.shape and all(a == b for a, b in zip(A.ravel(), B.ravel()))


def _rel(A, B):
    return float(np.linalg.norm(A - B) / max(np.linalg.norm(B), 1e-300))


def _phi(coeffs):
    """The composition p_T o ... o p_1, each p_t a numpy.polynomial built
    from its definition and evaluated stage by stage (composing the power
    series to degree 5^T would lose everything to cancellation)."""
    stages = [Polynomial([0.0, float(a), 0.0, float(b), 0.0, float(c)])
              for a, b, c in coeffs]

    def phi(x):
        for p in stages:
            x = p(x)
        return x
    return phi


def _closed_form(X, coeffs, eps=1e-7):
    """U phi(s) V^T for the thin SVD of X/(||X||_F + eps)."""
    Y = X / (np.linalg.norm(X) + eps)
    U, s, Vt = np.linalg.svd(Y, full_matrices=False)
    return (U * _phi(coeffs)(s)) @ Vt


def _randn(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# P1: exact rational equality of the different algorithms (Theorem 2)
# ---------------------------------------------------------------------------
def pin_exact_equivalence(O):
    X = _exact(X35)
    ref = O.standard_ns(X, SCHED3, eps=EPS)
    for rs in [(), (1,), (2,), (1, 2)]:
        for alg in ("stabilized", "naive"):
            got = O.gram_ns(X, SCHED3, restarts=rs, algebra=alg, eps=EPS)
            assert _eq(got, ref), f"Gram NS ({alg}, restarts {rs}) != standard NS exactly"


def pin_exact_equivalence_t4(O):
    X = _exact(X22)
    ref = O.standard_ns(X, SCHED4, eps=EPS)
    for rs in [(2,), (1, 3)]:
        got = O.gram_ns(X, SCHED4, restarts=rs, eps=EPS)
        assert _eq(got, ref), f"T=4 Gram NS (restarts {rs}) != standard NS exactly"


def pin_restart_semantics(O):
    """A restart after iteration s replaces the input by X_s = Q_s X, which
    must equal s steps of standard NS exactly (Theorem 2 proof: q_t = x_t/x_0);
    R is re-formed from it and Q starts again from I, so Q_{s+1} = h_{s+1}(R).
    Restarts leave the output unchanged, so only the trace can pin where one
    happens."""
    X = _exact(X35)
    for s in (1, 2):
        _, trace = O.gram_ns_trace(X, SCHED3, restarts=(s,), eps=EPS)
        where = [st["t"] for st in trace if "restart_X" in st]
        assert where == [s + 1], where
        Xs = trace[s]["restart_X"]
        assert _eq(Xs, O.standard_ns(X, SCHED3[:s], eps=EPS))
        a, b, c = SCHED3[s]
        R = Xs @ Xs.T
        I = _exact([[int(i == j) for j in range(R.shape[0])] for i in range(R.shape[0])])
        assert _eq(trace[s]["Q"], a * I + b * R + c * (R @ R))


# ---------------------------------------------------------------------------
# P1b: rank-one closed form, exact.  For a single row x the only singular
# value of x/(|x| + eps) is s = |x|/(|x| + eps), so T steps give
# (p_T o ... o p_1)(s) * x/|x| (Dion3 §2.2); evaluated here by hand-written
# Horner steps of each p_t, in rationals.
# ---------------------------------------------------------------------------
def pin_rank_one_exact(O):
    x = _exact([[1, 2, 2]])                  # |x| = 3
    s = F(3) / (F(3) + EPS)
    y = s
    for a, b, c in SCHED3:
        y2 = y * y
        y = y * (a + y2 * (b + y2 * c))
    expect = x * (y / 3)
    assert _eq(O.standard_ns(x, SCHED3, eps=EPS), expect)
    assert _eq(O.gram_ns(x, SCHED3, restarts=(1,), eps=EPS), expect)
    # Printed Muon quintic, one step, eps = 0: p(1) = a + b + c = 0.701.
    sched = load_schedules()
    got = O.standard_ns(x, [sched["muon_ns5"]], eps=F(0))
    assert _eq(got, x * (F("0.701") / 3))


# ---------------------------------------------------------------------------
# P2: Theorem 2, scalar recurrence vs composed polynomial (exact + fp64)
# ---------------------------------------------------------------------------
def pin_theorem2(O):
    for k in range(0, 11):
        x = F(k, 10)
        y = x
        for a, b, c in SCHED4:
            y = a * y + b * y ** 3 + c * y ** 5
        assert O.theorem2_q(SCHED4, x) * x == y
        assert O.composed_poly(SCHED4, x) == y
    xs = np.linspace(0.0, 1.0, 1001)
    ref = _phi(SCHED4)(xs)
    assert np.max(np.abs(O.theorem2_q(SCHED4, xs) * xs - ref)) <= 1e-12
    assert np.max(np.abs(O.composed_poly(SCHED4, xs) - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# P4: spectral closed form with numpy SVD + numpy.polynomial (fp64)
# ---------------------------------------------------------------------------
def pin_spectral(O):
    sched = load_schedules()
    ns5 = [tuple(float(v) for v in sched["muon_ns5"])] * 5
    mixed = [tuple(float(v) for v in row) for row in SCHED4] + [ns5[0]]
    # wide, square, and tall shapes (a tall X goes through its transpose; the
    # closed form uses the SVD of the tall matrix itself)
    for seed, (n, m) in enumerate([(24, 60), (17, 17), (9, 40), (40, 9), (60, 24)]):
        X = 3.0 * _randn((n, m), seed)
        for co in (ns5, mixed):
            cf = _closed_form(X, co)
            assert _rel(O.standard_ns(X, co), cf) <= 1e-10
            assert _rel(O.gram_ns(X, co, restarts=(2,)), cf) <= 1e-10
            assert _rel(O.gram_ns(X, co, restarts=(), algebra="naive"), cf) <= 1e-10
            assert _rel(O.spectral_map(X, co), cf) <= 1e-12


# ---------------------------------------------------------------------------
# P5: the convergent schedule drives X to the textbook polar factor U V^T
# ---------------------------------------------------------------------------
def pin_polar_limit(O):
    sched = load_schedules()
    conv = [tuple(float(v) for v in sched["convergent"])] * 40
    rng = np.random.default_rng(7)
    n, m = 8, 20
    U, _ = np.linalg.qr(rng.standard_normal((n, n)))
    V, _ = np.linalg.qr(rng.standard_normal((m, n)))
    s = np.linspace(1.0, 0.1, n)
    X = (U * s) @ V.T
    polar = U @ V.T
    assert _rel(O.standard_ns(X, conv), polar) <= 1e-12
    assert _rel(O.gram_ns(X, conv, restarts=(5, 10, 15, 20, 25, 30, 35)), polar) <= 1e-12
    assert _rel(O.polar(X), polar) <= 1e-12
    # the tall matrix X^T = V S U^T has polar factor V U^T
    assert _rel(O.standard_ns(X.T, conv), polar.T) <= 1e-12
    assert _rel(O.gram_ns(X.T, conv, restarts=(5, 10, 15, 20, 25, 30, 35)), polar.T) <= 1e-12


# ---------------------------------------------------------------------------
# FLOP model against the printed counts
# ---------------------------------------------------------------------------
def pin_flop_model(O):
    with open(os.path.join(GOLDEN, "flop_model.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    n = 64
    for key, T, alpha, val in rows:
        T, alpha, val = int(T), int(alpha), float(val)
        m = alpha * n
        if key == "standard_plain":
            got = O.flops_standard(n, m, T, symmetric=False) / n ** 3
        elif key == "standard_sym":
            got = O.flops_standard(n, m, T, symmetric=True) / n ** 3
        elif key == "gram_naive":
            got = O.flops_gram(n, m, T, 0) / n ** 3
        elif key == "restart_extra":
            got = (O.flops_gram(n, m, T, 1) - O.flops_gram(n, m, T, 0)) / n ** 3
        elif key == "saving_vs_sym":
            got = round(100 * (1 - O.flops_gram(n, m, T, 0) / O.flops_standard(n, m, T, True)))
        elif key == "saving_vs_plain":
            got = round(100 * (1 - O.flops_gram(n, m, T, 0) / O.flops_standard(n, m, T, False)))
        else:
            raise KeyError(key)
        assert abs(got - val) < 1e-9, (key, got, val)


# ---------------------------------------------------------------------------
# P6: invariants
# ---------------------------------------------------------------------------
def pin_invariants(O):
    sched = load_schedules()
    ns5 = [tuple(float(v) for v in sched["muon_ns5"])] * 5
    X = _randn((12, 30), 3)
    out, trace = O.gram_ns_trace(X, ns5, restarts=(2,))
    R0 = (X / (np.linalg.norm(X) + 1e-7))
    R0 = R0 @ R0.T
    assert np.linalg.eigvalsh(R0).min() >= -1e-14 * np.linalg.norm(R0)
    for st in trace:
        for key in ("R", "Z", "Q"):
            M = st[key]
            assert np.linalg.norm(M - M.T) <= 1e-13 * np.linalg.norm(M), (st["t"], key)
        assert np.linalg.norm(st["Q"] @ st["R"] - st["R"] @ st["Q"]) <= 1e-12 * (
            np.linalg.norm(st["Q"]) * np.linalg.norm(st["R"]))
    # row permutation + sign flips and column permutation equivariance
    rng = np.random.default_rng(11)
    P = np.eye(12)[rng.permutation(12)] * rng.choice([-1.0, 1.0], size=12)[:, None]
    Pi = np.eye(30)[:, rng.permutation(30)]
    assert _rel(O.gram_ns(P @ X, ns5), P @ out) <= 1e-12
    assert _rel(O.gram_ns(X @ Pi, ns5), out @ Pi) <= 1e-12
    assert _rel(O.standard_ns(P @ X @ Pi, ns5), P @ O.standard_ns(X, ns5) @ Pi) <= 1e-12
    # zero matrix -> exactly zero (eps keeps the normalisation finite)
    Z0 = np.zeros((4, 9))
    assert np.all(O.gram_ns(Z0, ns5) == 0.0) and np.all(O.standard_ns(Z0, ns5) == 0.0)
    # scale invariance up to the eps effect
    assert _rel(O.gram_ns(1024.0 * X, ns5), out) <= 1e-6
    # singular values of the output are phi(singular values of the input)
    s_in = np.linalg.svd(X / (np.linalg.norm(X) + 1e-7), compute_uv=False)
    s_out = np.linalg.svd(out, compute_uv=False)
    assert np.max(np.abs(np.sort(s_out) - np.sort(np.abs(_phi(ns5)(s_in))))) <= 1e-12


# ---------------------------------------------------------------------------
# P7: Dion3 fractional rows
# ---------------------------------------------------------------------------
def pin_dion3(O):
    sched = load_schedules()
    ns5 = [tuple(float(v) for v in sched["muon_ns5"])] * 5
    X = _randn((10, 24), 5)
    init = _randn((10, 24), 6)
    perm = np.random.default_rng(1).permutation(10)
    full = O.dion3_rows(X, init, perm, ns5)
    assert _rel(full, O.gram_ns(X, ns5)) <= 1e-12            # f = 1 reduces to Muon
    rows = [7, 2, 4]
    part = O.dion3_rows(X, init, rows, ns5)
    keep = [i for i in range(10) if i not in rows]
    assert np.array_equal(part[keep], init[keep])              # untouched rows
    sub = X[rows]
    assert _rel(part[rows], _closed_form(sub, ns5)) <= 1e-10   # own normalisation


# ---------------------------------------------------------------------------
# Dion3 selection: brute force over every k-subset on tiny integer matrices
# ---------------------------------------------------------------------------
def pin_dion3_select(O):
    import itertools
    rng = np.random.default_rng(11)
    for trial in range(40):
        n, m = int(rng.integers(1, 8)), int(rng.integers(1, 5))
        # small integers (many exact ties), signs mixed
        M = rng.integers(-3, 4, size=(n, m)).astype(np.float64)
        for k in range(1, n + 1):
            got = O.dion3_select(M, k)
            norms = [sum(abs(int(v)) for v in M[i]) for i in range(n)]
            # the subset with the largest total norm; among equals, the
            # lexicographically smallest index tuple
            best = max(itertools.combinations(range(n), k),
                       key=lambda S: (sum(norms[i] for i in S), [-i for i in S]))
            assert list(got) == list(best), (M, k, got, best)
    # k = n takes every row; a row permutation permutes the selection
    M = _randn((30, 12), 3)
    assert list(O.dion3_select(M, 30)) == list(range(30))
    perm = np.random.default_rng(2).permutation(30)
    sel = set(O.dion3_select(M, 9))
    assert set(O.dion3_select(M[perm], 9)) == {int(np.where(perm == i)[0][0]) for i in sel}


# ---------------------------------------------------------------------------
# The whole Dion3 update (Algorithm 4 with the NorMuon steps of eq. (2))
# ---------------------------------------------------------------------------
def pin_dion3_step(O):
    from fractions import Fraction
    sched = load_schedules()
    ns5 = [tuple(float(v) for v in sched["muon_ns5"])] * 5
    n, m, lr = 12, 40, 0.03
    W, G, M = _randn((n, m), 21), _randn((n, m), 22), _randn((n, m), 23)
    Msum32 = np.float32(M) + np.float32(G)          # the stored fp32 momentum sum
    Msum = Msum32.astype(np.float64)
    v0 = np.abs(_randn(n, 24)) + 0.1

    # k = n, no NorMuon, no decay: W moves by -lr times the closed form of
    # the finite iteration on M + G (thin SVD), M becomes momentum * (M + G)
    r = O.dion3_step(W, G, M, v0, n, ns5, lr=lr, weight_decay=0.0, momentum=0.5, normuon=False)
    assert list(r["S"]) == list(range(n))
    assert _rel(W - r["W"], lr * _closed_form(Msum, ns5)) <= 1e-10
    assert np.array_equal(r["M"], 0.5 * Msum) and np.array_equal(r["v"], v0)

    # selection on the momentum sum: exact rational l1 norms of the fp32 values
    k = 5
    r = O.dion3_step(W, G, M, v0, k, ns5, lr=lr, weight_decay=0.1, momentum=0.25, normuon=False)
    exact = [sum(abs(Fraction(float(x))) for x in Msum32[i]) for i in range(n)]
    top = sorted(sorted(range(n), key=lambda i: -exact[i])[:k])
    assert list(r["S"]) == top
    rest = [i for i in range(n) if i not in top]
    decay = 1.0 - lr * 0.1
    assert np.array_equal(r["W"][rest], decay * W[rest])          # decay only
    assert np.array_equal(r["M"][rest], Msum[rest])                # momentum sum kept
    assert np.array_equal(r["M"][top], 0.25 * Msum[top])           # error feedback
    cf = _closed_form(Msum[top], ns5)
    assert _rel(decay * W[top] - r["W"][top], lr * cf) <= 1e-10   # own normalisation of M[S]

    # lr * weight_decay = 1 zeroes the unselected rows; momentum 0 zeroes the
    # selected momentum rows
    r = O.dion3_step(W, G, M, v0, k, ns5, lr=lr, weight_decay=1.0 / lr, momentum=0.0, normuon=False)
    assert not r["W"][rest].any() and not r["M"][top].any()
    assert _rel(-r["W"][top], lr * cf) <= 1e-10

    # NorMuon, beta2 = 0: the second moment is this step's row mean square, so
    # every row ends with the same norm, and the rescale keeps ||O||_F
    r = O.dion3_step(W, G, M, v0, k, ns5, lr=lr, momentum=0.9, beta2=0.0, eps=1e-12, normuon=True)
    rn = np.linalg.norm(r["O"], axis=1)
    assert np.max(np.abs(rn / rn[0] - 1.0)) <= 1e-9
    assert abs(np.linalg.norm(r["O"]) / np.linalg.norm(cf) - 1.0) <= 1e-10
    assert np.allclose(r["v"][top], np.mean(cf * cf, axis=1), rtol=1e-10, atol=0)
    assert np.array_equal(r["v"][rest], v0[rest])

    # NorMuon, beta2 = 1: v stays as given and row i is divided by
    # sqrt(v_i) + eps before the common rescale
    v1 = v0.copy()
    v1[top] = [1.0, 4.0, 9.0, 16.0, 25.0]
    r = O.dion3_step(W, G, M, v1, k, ns5, lr=lr, beta2=1.0, eps=0.0, normuon=True)
    assert np.array_equal(r["v"], v1)
    ratio = np.linalg.norm(r["O"], axis=1) / np.linalg.norm(cf, axis=1)
    assert np.allclose(ratio * np.array([1.0, 2.0, 3.0, 4.0, 5.0]), ratio[0], rtol=1e-10, atol=0)
    assert abs(np.linalg.norm(r["O"]) / np.linalg.norm(cf) - 1.0) <= 1e-10

    # NorMuon, beta2 = 1/2: the new second moment averages the old one and
    # the row mean square of the orthogonalised rows
    r = O.dion3_step(W, G, M, v1, k, ns5, lr=lr, beta2=0.5, eps=1e-8, normuon=True)
    assert np.allclose(r["v"][top], 0.5 * v1[top] + 0.5 * np.mean(cf * cf, axis=1), rtol=1e-10, atol=0)

    # a zero momentum sum: every key ties at 0, so the first k rows are
    # taken; Newton-Schulz of zero is zero, NorMuon leaves it zero (the
    # Frobenius rescale is 0/0 there), W only decays and v only decays
    Z = np.zeros((n, m))
    r = O.dion3_step(W, Z, Z, v1, k, ns5, lr=lr, weight_decay=0.5, beta2=0.5, eps=1e-8, normuon=True)
    assert list(r["S"]) == list(range(k))
    assert np.all(np.isfinite(r["O"])) and not r["O"].any()
    assert np.array_equal(r["W"], (1.0 - lr * 0.5) * W)
    assert np.array_equal(r["v"][:k], 0.5 * v1[:k]) and np.array_equal(r["v"][k:], v1[k:])
    assert not r["M"].any()


# ---------------------------------------------------------------------------
# Where to restart: the scalar model and sweep of Dion3 App. B.2.1
# ---------------------------------------------------------------------------
def pin_restart_sweep(O):
    sched = load_schedules()
    ns5 = [tuple(float(v) for v in sched["muon_ns5"])] * 5
    stab = [tuple(float(v) for v in sched["convergent"])]
    # (a) no corruption and no spurious eigenvalue: restarts are exact, so the
    # output singular value is phi(x_0) whatever the schedule (Theorem 2)
    x0 = np.linspace(0.0, 1.0, 401)
    for rs in ((), (1,), (2,), (1, 3), (4,)):
        _, q_trace, xT = O.restart_model(ns5, rs, x0 * x0, r_min=0.0)
        assert len(q_trace) == 5
        assert np.max(np.abs(xT - _phi(ns5)(x0))) <= 1e-12
    # (b) a spurious negative eigenvalue grows by at least (15/8)^2 per step
    # under h(x) = 15/8 - 10/8 x + 3/8 x^2 (App. B.1.2), never restarted
    r_trace, _, _ = O.restart_model(stab * 6, (), np.array([-4e-4, -1e-6]), r_min=-4e-4)
    for r_prev, r_next in zip(r_trace[:-1], r_trace[1:]):
        assert np.all(r_next < 0) and np.all(r_next / r_prev >= (15 / 8) ** 2)
    # (c) the 10-step study of App. B.2 restarts after step 5 (Figs. 16-17);
    # for a constant schedule the sweep puts one restart in the middle and
    # two restarts of 15 steps after 5 and 10
    assert O.restart_sweep(stab * 10, 1, points=2001)[0] == (5,)
    assert O.restart_sweep(stab * 15, 2, points=2001)[0] == (5, 10)
    # (d) App. B.2.1, Fig. 18: without a restart the printed quintic blows up
    # from R_0's -4e-4; one restart after iteration 2 keeps every eigenvalue
    # of R above -0.4 and of Q below 100, a restart after 1 or 4 does not
    _, none = O.restart_sweep(ns5, 0)
    assert none[0]["restarts"] == () and none[0]["max_cond_q"] > 1e6 and none[0]["min_r"] < -10
    best, rows = O.restart_sweep(ns5, 1)
    by = {r["restarts"]: r for r in rows}
    assert sorted(by) == [(1,), (2,), (3,), (4,)]
    assert by[(2,)]["min_r"] > -0.4 and by[(2,)]["max_q"] < 100
    for bad in ((1,), (4,)):
        assert by[bad]["min_r"] < -0.4 or by[bad]["max_q"] > 100
    assert by[best]["max_cond_q"] == min(r["max_cond_q"] for r in rows)
    # without corruption the condition numbers follow from Theorem 2 alone:
    # q_t = phi_t(x_0) / x_0 on every direction, (a_1 ... a_t) at x_0 = 0
    pts = 2001
    _, rows0 = O.restart_sweep(ns5, 0, r_min=0.0, points=pts)
    xs = np.sqrt(np.linspace(0.0, 1.0, pts))
    want = 0.0
    for t in range(1, 6):
        with np.errstate(invalid="ignore", divide="ignore"):
            qt = _phi(ns5[:t])(xs) / xs
        qt[0] = np.prod([c[0] for c in ns5[:t]])
        want = max(want, np.max(np.abs(qt)) / np.min(np.abs(qt)))
    assert abs(rows0[0]["max_cond_q"] / want - 1.0) <= 1e-9
    # ... and after an exact restart after 2, Q restarts from I on x_2 =
    # phi_2(x_0): q_t = phi_t(x_0) / phi_2(x_0) for t > 2 (its smallest value
    # lies inside the grid, where x_2^2 reaches the vertex of h)
    _, rows2 = O.restart_sweep(ns5, 1, r_min=0.0, points=pts)
    with np.errstate(invalid="ignore", divide="ignore"):
        qs = [_phi(ns5[:t])(xs) / xs for t in (1, 2)]
        qs += [_phi(ns5[:t])(xs) / _phi(ns5[:2])(xs) for t in (3, 4, 5)]
    qs[0][0], qs[1][0] = ns5[0][0], ns5[0][0] * ns5[1][0]
    for i, t in enumerate((3, 4, 5)):
        qs[2 + i][0] = np.prod([c[0] for c in ns5[2:t]])
    want2 = max(np.max(np.abs(q)) / np.min(np.abs(q)) for q in qs)
    assert 0 < np.argmin(np.abs(qs[2])) < pts - 1
    assert abs([r for r in rows2 if r["restarts"] == (2,)][0]["max_cond_q"] / want2 - 1.0) <= 1e-9
    # the re-formed R's smallest eigenvalue is the corruption itself (the
    # zero directions of X stay zero)
    r_trace, _, _ = O.restart_model(ns5, (2,), np.array([-4e-4, 0.25, 1.0]))
    assert len(r_trace) == 5 and r_trace[2][0] == -4e-4 and r_trace[2][2] > 0


FAST_PINS = [pin_exact_equivalence, pin_restart_semantics, pin_rank_one_exact, pin_theorem2, pin_spectral,
             pin_polar_limit, pin_flop_model, pin_invariants, pin_dion3, pin_dion3_select, pin_dion3_step,
             pin_restart_sweep]
ALL_PINS = FAST_PINS + [pin_exact_equivalence_t4]

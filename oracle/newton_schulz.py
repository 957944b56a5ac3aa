"""Reference oracle for Newton-Schulz orthogonalisation (fp64 CPU).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code with the HIP library.

Every routine follows the written description in
"Dion3: Full-Stack Orthogonal Updates" (Amsel et al.):

* ``standard_ns``   -- §2.2, Algorithm 1 (standard Newton-Schulz).
* ``gram_ns``       -- §4, Algorithm 2 (naive Gram Newton-Schulz) and §4.2,
                       Algorithm 3 (stabilised Gram Newton-Schulz, with the
                       reformulated quadratic of Appendix B.2.3), with the
                       restart generalised to any set of iterations
                       (Appendix B.2: restart every few iterations).
* ``theorem2_q``    -- §4, Theorem 2 (scalar r/q/z recurrence).
* ``composed_poly`` -- §2.2: the composed odd polynomial p_T o ... o p_1.
* ``spectral_map``  -- §2.2: NS acts on the SVD as U (p_T o...o p_1)(S) V^T.
* ``polar``         -- §2.1, Definition 1: polar(X) = U V^T.
* ``dion3_select``  -- §6, Algorithm 4, selection: the k rows of largest l1
                       norm.
* ``dion3_rows``    -- §6, Algorithm 4: orthogonalise the selected rows M[S,:]
                       as one k x m matrix and write them back.
* ``normuon_rows``  -- the NorMuon steps of Algorithm 4 (§2.1 eq. (2)).
* ``dion3_step``    -- §6, Algorithm 4 in full (momentum sum, selection,
                       orthogonalisation, the optional NorMuon steps of §2.1
                       eq. (2), weight decay, update of the selected rows,
                       error feedback).
* ``flops_*``       -- §2.2 and §4.1 FLOP models, §4.2 restart surcharge.
* ``restart_model``, ``restart_sweep``
                    -- Appendix B.2.1: the scalar model of Gram Newton-Schulz
                       on every eigen-direction of R_0, with spurious negative
                       eigenvalues and a corruption at every re-formed R, and
                       the sweep over restart schedules that keeps the
                       condition number of Q_t smallest.

Arithmetic is float64 numpy (BLAS matmul) for float inputs.  For inputs of
dtype ``object`` holding ``fractions.Fraction`` the very same code runs in
exact rational arithmetic; the Frobenius norm then must be rational (the
square root is taken exactly), which is how the tests pin the algebra
bit-exactly.  Dion3 runs these iterations in half precision; the oracle
deliberately does not emulate any rounding.

Readings of the sources taken here (each also listed in the design notes):
* normalisation is X / (||X||_F + eps) with eps = 1e-7 added to the norm;
* "restart after iteration s" means: before computing Z_{s+1}, replace X by
  Q_s X, re-form R from it and reset Q to I (X is not renormalised);
* the coefficient triple of iteration t is (a_t, b_t, c_t) with
  p_t(x) = a_t x + b_t x^3 + c_t x^5 and h_t(y) = a_t + b_t y + c_t y^2;
* NorMuon divides each selected row by the square root of its second moment
  plus eps (the root sign is lost in the extracted text of Algorithm 4 and
  eq. (2); the recap describes an Adam-style second moment); weight decay
  scales every row of W, the update and the error feedback touch the
  selected rows only (Algorithm 4 marks those two lines "for i in S");
* the one stored value the selection reads, the momentum sum M + G, is
  formed as an fp32 addition, as the caller's fp32 buffer holds it; all
  later steps are fp64;
* Dion3 (§2) takes n <= m without loss of generality; a tall X (n > m) is
  orthogonalised through its transpose: the iteration runs on X^T and the
  result is transposed back (polar(X) = polar(X^T)^T, and each odd
  polynomial step commutes with transposition).
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction
from typing import Iterable, Sequence

import numpy as np

EPS = 1e-7

__all__ = [
    "EPS", "frobenius_normalize", "standard_ns", "gram_ns", "theorem2_q",
    "composed_poly", "spectral_map", "polar", "dion3_select", "dion3_rows", "dion3_step",
    "flops_standard", "flops_gram", "gram_ns_trace", "restart_model", "restart_sweep",
]


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def _is_exact(x: np.ndarray) -> bool:
    return x.dtype == object


def _exact_sqrt(v: Fraction) -> Fraction:
    """Square root of a non-negative rational that must be a perfect square."""
    v = Fraction(v)
    if v < 0:
        raise ValueError("negative")
    p, q = v.numerator, v.denominator
    rp, rq = math.isqrt(p), math.isqrt(q)
    if rp * rp != p or rq * rq != q:
        raise ValueError(f"{v} is not the square of a rational")
    return Fraction(rp, rq)


def _eye(n: int, like: np.ndarray) -> np.ndarray:
    if _is_exact(like):
        e = np.empty((n, n), dtype=object)
        for i in range(n):
            for j in range(n):
                e[i, j] = Fraction(int(i == j))
        return e
    return np.eye(n, dtype=np.float64)


def _as_work(X) -> np.ndarray:
    X = np.asarray(X)
    if X.dtype == object:
        return np.vectorize(Fraction, otypes=[object])(X)
    return X.astype(np.float64)


def _coef(c, exact: bool):
    return Fraction(c) if exact else float(c)


def _coeff_list(coeffs, exact: bool):
    out = []
    for row in coeffs:
        a, b, c = row
        out.append((_coef(a, exact), _coef(b, exact), _coef(c, exact)))
    if not out:
        raise ValueError("need at least one iteration")
    return out


# --------------------------------------------------------------------------
# normalisation (Algorithms 1-3, first step)
# --------------------------------------------------------------------------
def frobenius_normalize(X, eps=EPS) -> np.ndarray:
    """X / (||X||_F + eps): puts every singular value in [0, 1)."""
    X = _as_work(X)
    if _is_exact(X):
        s = sum((v * v for v in X.ravel()), Fraction(0))
        return X / (_exact_sqrt(s) + Fraction(eps))
    return X / (np.sqrt(np.sum(X * X)) + eps)


# --------------------------------------------------------------------------
# Algorithm 1: standard Newton-Schulz
# --------------------------------------------------------------------------
def standard_ns(X, coeffs, eps=EPS) -> np.ndarray:
    """Standard Newton-Schulz (Dion3 §2.2, Algorithm 1).

    Each iteration forms the n x n matrix A = X X^T, the quadratic
    B = b A + c A^2 and updates X <- a X + B X, which maps every singular
    value x to p_t(x) = a x + b x^3 + c x^5.
    """
    X = _as_work(X)
    n, m = X.shape
    if n > m:                        # n <= m without loss of generality
        return standard_ns(X.T, coeffs, eps).T
    exact = _is_exact(X)
    Y = frobenius_normalize(X, eps)
    for a, b, c in _coeff_list(coeffs, exact):
        A = Y @ Y.T
        B = b * A + c * (A @ A)
        Y = a * Y + B @ Y
    return Y


# --------------------------------------------------------------------------
# Algorithms 2 and 3: Gram Newton-Schulz
# --------------------------------------------------------------------------
def gram_ns_trace(X, coeffs, restarts: Iterable[int] = (2,),
                  algebra: str = "stabilized", eps=EPS):
    """Gram Newton-Schulz, returning the output and every intermediate.

    algebra="stabilized": Dion3 §4.2 Algorithm 3 / Appendix B.2.3.  The
        quadratic is Z_t = b R + c R^2 and a_t enters each product through
        an explicit a * (.) term:  Q_t = Q Z + a Q,  RZ = R Z + a R,
        R_t = Z RZ + a RZ.
    algebra="naive":      Dion3 §4 Algorithm 2.  Z_t = a I + b R + c R^2,
        Q_t = Q Z, R_t = Z R Z.

    ``restarts`` holds the iterations s after which the method restarts
    (Dion3 §4.2; Appendix B.2): at the start of iteration s+1 the input is
    replaced by Q_s X, R is re-formed as X X^T and Q is reset to I.  The
    pages' default is a single restart after iteration 2.  An empty set gives
    the un-restarted iteration.

    Returns (output, trace) where trace is a list of dicts with the values of
    R, Z, Q after each iteration (and the restarted X when one happens).
    A tall X (n > m) runs on X^T; the output is transposed back and the
    trace holds the m x m iterates of the transposed problem.
    """
    X = _as_work(X)
    n, m = X.shape
    if n > m:                        # n <= m without loss of generality
        out, trace = gram_ns_trace(X.T, coeffs, restarts, algebra, eps)
        return out.T, trace
    exact = _is_exact(X)
    cl = _coeff_list(coeffs, exact)
    T = len(cl)
    rs = sorted(set(int(s) for s in restarts))
    for s in rs:
        if not 1 <= s <= T - 1:
            raise ValueError(f"restart after iteration {s} is outside [1, T-1]")
    if algebra not in ("stabilized", "naive"):
        raise ValueError(algebra)

    Y = frobenius_normalize(X, eps)
    R = Y @ Y.T                      # Gram matrix R_0
    Q = _eye(n, Y)                   # Q_0 = I
    trace = []
    for t in range(1, T + 1):
        a, b, c = cl[t - 1]
        step = {"t": t}
        if (t - 1) in rs:            # restart after iteration t-1
            Y = Q @ Y
            R = Y @ Y.T
            Q = _eye(n, Y)
            step["restart_X"] = Y
        if algebra == "stabilized":
            Z = b * R + c * (R @ R)
            Q = Q @ Z + a * Q
            RZ = R @ Z + a * R
            R = Z @ RZ + a * RZ
        else:
            Z = a * _eye(n, Y) + b * R + c * (R @ R)
            Q = Q @ Z
            R = Z @ R @ Z
        step.update(R=R, Z=Z, Q=Q)
        trace.append(step)
    return Q @ Y, trace


def gram_ns(X, coeffs, restarts: Iterable[int] = (2,),
            algebra: str = "stabilized", eps=EPS) -> np.ndarray:
    """Gram Newton-Schulz output Q_T X (see :func:`gram_ns_trace`)."""
    return gram_ns_trace(X, coeffs, restarts, algebra, eps)[0]


# --------------------------------------------------------------------------
# Theorem 2 and the spectral picture
# --------------------------------------------------------------------------
def composed_poly(coeffs, x):
    """(p_T o ... o p_1)(x) with p_t(x) = a_t x + b_t x^3 + c_t x^5 (§2.2)."""
    exact = isinstance(x, Fraction) or (isinstance(x, np.ndarray) and x.dtype == object)
    y = x
    for a, b, c in _coeff_list(coeffs, exact):
        y = a * y + b * y ** 3 + c * y ** 5
    return y


def theorem2_q(coeffs, x):
    """q_T from Theorem 2: r_0 = x^2, q_0 = 1, z_t = h_t(r_{t-1}),
    r_t = r_{t-1} z_t^2, q_t = q_{t-1} z_t, with h_t(y) = a + b y + c y^2.
    The theorem states (p_T o ... o p_1)(x) = q_T x."""
    exact = isinstance(x, Fraction) or (isinstance(x, np.ndarray) and x.dtype == object)
    r = x * x
    q = Fraction(1) if exact else 1.0
    for a, b, c in _coeff_list(coeffs, exact):
        z = a + b * r + c * r * r
        r = r * z * z
        q = q * z
    return q


def spectral_map(X, coeffs, eps=EPS) -> np.ndarray:
    """U diag(phi(s)) V^T for the thin SVD of X/(||X||_F+eps), phi the
    composed polynomial: the exact result of T Newton-Schulz steps (§2.2)."""
    Y = frobenius_normalize(np.asarray(X, dtype=np.float64), eps)
    U, s, Vt = np.linalg.svd(Y, full_matrices=False)
    return (U * composed_poly(coeffs, s)) @ Vt


def polar(X) -> np.ndarray:
    """polar(X) = U V^T for the thin SVD X = U S V^T (Dion3 Definition 1)."""
    U, _, Vt = np.linalg.svd(np.asarray(X, dtype=np.float64), full_matrices=False)
    return U @ Vt


# --------------------------------------------------------------------------
# Dion3 fractional rows (Algorithm 4, orthogonalisation of M[S,:])
# --------------------------------------------------------------------------
def dion3_select(M, k: int) -> np.ndarray:
    """Selection step of the Dion3 update (Dion3 §6, Algorithm 4): the
    indices of the k rows of M with the largest l1 norm, in ascending order.

    A row's norm is the exact sum of |M_ij| rounded once to float64
    (math.fsum).  Rows with equal norms are taken in index order, the smaller
    index first (Dion3's Algorithm 4 does not say how ties break).
    """
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[0]
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    keys = [math.fsum(np.abs(M[i])) for i in range(n)]
    order = sorted(range(n), key=lambda i: (-keys[i], i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def dion3_rows(X, out_init, rows: Sequence[int], coeffs, restarts=(2,),
               algebra="stabilized", eps=EPS) -> np.ndarray:
    """Orthogonalise rows ``rows`` of X as one k x m matrix (normalised by its
    own Frobenius norm) with Gram Newton-Schulz and write the result to the
    same rows of a copy of ``out_init``; all other rows are left as given."""
    X = np.asarray(X)
    rows = [int(r) for r in rows]
    if len(set(rows)) != len(rows):
        raise ValueError("row indices must be distinct")
    out = np.array(out_init, dtype=np.float64, copy=True)
    out[rows, :] = gram_ns(X[rows, :], coeffs, restarts, algebra, eps)
    return out


def normuon_rows(O, v_rows, beta2=0.95, eps=1e-8):
    """The optional NorMuon steps of Dion3 Algorithm 4 (from NorMuon, §2.1
    eq. (2)) on the k x m update O, whose row i has second moment v_rows[i]:
    v_i <- beta2 v_i + (1 - beta2) mean_j O_ij^2, O_ij <- O_ij / (sqrt(v_i)
    + eps), then O is rescaled to the Frobenius norm it had before that
    division.  Returns (O, v_rows), both new float64 arrays."""
    O = np.asarray(O, dtype=np.float64)
    second = beta2 * np.asarray(v_rows, dtype=np.float64) + (1.0 - beta2) * np.mean(O * O, axis=1)
    On = O / (np.sqrt(second) + eps)[:, None]
    # the rescale to ||O||_F is 0/0 when the selected rows orthogonalise to
    # zero (a zero momentum sum); the update then stays zero
    norm_on = np.linalg.norm(On)
    O = On * (np.linalg.norm(O) / norm_on) if norm_on > 0 else On
    return O, second


def dion3_step(W, G, M, v, k: int, coeffs, restarts=(2,), lr=0.02, weight_decay=0.0,
               momentum=0.95, beta2=0.95, eps=1e-8, normuon=True, algebra="stabilized"):
    """One Dion3 update of one weight matrix (Dion3 §6, Algorithm 4), with
    Gram Newton-Schulz as its polar step and, when ``normuon``, the NorMuon
    steps of §2.1 eq. (2).  In order:

    1. the momentum takes the gradient: M + G (an fp32 addition: the caller's
       momentum buffer is fp32, and the selection reads the stored sum);
    2. S = the k rows of that sum with the largest l1 norm (dion3_select);
    3. O = Gram Newton-Schulz of the k x m submatrix of those rows;
    4. NorMuon: v_i <- beta2 v_i + (1 - beta2) mean_j O_ij^2 for i in S,
       O_ij <- O_ij / (sqrt(v_i) + eps), then O is rescaled to the Frobenius
       norm it had before that division (a zero O stays zero: Algorithm 4's
       ratio is 0/0 there);
    5. weight decay on every row: W <- (1 - lr * weight_decay) W;
    6. the selected rows move: W[S] <- W[S] - lr * O;
    7. error feedback on the selected rows: M[S] <- momentum * M[S].

    Returns a dict with W, M, v (fp64 arrays; v untouched without NorMuon),
    S (int64, ascending) and O (the k x m update direction after step 4).
    """
    W = np.asarray(W, dtype=np.float64)
    Msum = (np.asarray(M, dtype=np.float32) + np.asarray(G, dtype=np.float32)).astype(np.float64)
    n, m = Msum.shape
    S = dion3_select(Msum, k)
    O = gram_ns(Msum[S, :], coeffs, restarts, algebra)
    v_new = np.array(v, dtype=np.float64, copy=True) if v is not None else None
    if normuon:
        O, v_new[S] = normuon_rows(O, v_new[S], beta2, eps)
    W_new = (1.0 - lr * weight_decay) * W
    W_new[S, :] -= lr * O
    M_new = Msum.copy()
    M_new[S, :] *= momentum
    return {"W": W_new, "M": M_new, "v": v_new, "S": S, "O": O}


# --------------------------------------------------------------------------
# FLOP models (2 FLOPs per multiply-add)
# --------------------------------------------------------------------------
def flops_standard(n: int, m: int, T: int, symmetric: bool) -> float:
    """Standard NS: per iteration X X^T (2mn^2), A^2 (2n^3), B X (2mn^2)
    (§2.2); the symmetric kernels halve the two symmetric products (§2.3)."""
    if symmetric:
        return T * (3.0 * m * n * n + n ** 3)
    return T * (4.0 * m * n * n + 2.0 * n ** 3)


def flops_gram(n: int, m: int, T: int, n_restarts: int) -> float:
    """Gram NS with symmetric kernels (§4.1): four n^3 products per iteration,
    mn^2 for the Gram matrix, 2mn^2 for the final Q X, minus the free Q_1 and
    the skipped R_T (3n^3); each restart adds Q X (2mn^2) and a Gram matrix
    (mn^2) and again makes one Q update free and one R update skippable
    (3n^3), i.e. +3(alpha-1) n^3 (§4.2)."""
    base = T * 4.0 * n ** 3 + 3.0 * m * n * n - 3.0 * n ** 3
    return base + n_restarts * (3.0 * m * n * n - 3.0 * n ** 3)


# --------------------------------------------------------------------------
# Where to restart (Appendix B.2.1)
# --------------------------------------------------------------------------
def restart_model(coeffs, restarts: Iterable[int], r0, r_min: float = -4e-4):
    """Gram Newton-Schulz on one eigen-direction at a time (Appendix B.2.1).

    R_0, Q_t and R_t share eigenvectors in exact arithmetic (Theorem 2), so
    each eigenvalue r_0 of R_0 evolves on its own: z_t = h_t(r_{t-1}),
    q_t = q_{t-1} z_t, r_t = r_{t-1} z_t^2.  r0 holds eigenvalues of R_0 in
    [r_min, 1]; a negative one is spurious (Appendix B.1.2): its direction
    has singular value 0, so the input component is x_0 = sqrt(max(r_0, 0)).
    A restart before iteration t (t - 1 in ``restarts``) replaces X by Q X
    (x <- q x), re-forms R = X X^T with r_min added to every eigenvalue (the
    pages subtract 4e-4 I to model rounding at each re-formation), and resets
    Q to I.  The last R update is not needed and not taken.

    Returns (r_trace, q_trace, x_T): r_trace lists R's eigenvalues as each
    R is formed or updated (R_0, re-formed R's, R_1 .. R_{T-1} unless a
    restart replaces them), q_trace lists Q_1 .. Q_T, and x_T = q_T x is the
    output's singular value for each direction."""
    co = [tuple(float(v) for v in row) for row in coeffs]
    T = len(co)
    rs = set(int(s) for s in restarts)
    r = np.asarray(r0, dtype=np.float64).copy()
    x = np.sqrt(np.maximum(r, 0.0))
    q = np.ones_like(r)
    r_trace, q_trace = [r.copy()], []
    for t in range(1, T + 1):
        if (t - 1) in rs:
            x = q * x
            r = x * x + r_min
            q = np.ones_like(r)
            r_trace.append(r.copy())
        a, b, c = co[t - 1]
        z = a + b * r + c * r * r
        q = q * z
        q_trace.append(q.copy())
        if t < T and t not in rs:
            r = r * (z * z)
            r_trace.append(r.copy())
    return r_trace, q_trace, q * x


def restart_sweep(coeffs, n_restarts: int = 1, r_min: float = -4e-4, points: int = 20001):
    """The restart-schedule sweep of Appendix B.2.1: for every set of
    ``n_restarts`` restart iterations in [1, T-1], run :func:`restart_model`
    on a uniform grid of R_0 eigenvalues over [r_min, 1] and record the
    largest condition number of Q_t over t (max |q_t| / min |q_t| over the
    grid), the largest |q_t| and the smallest eigenvalue of any R.  Returns
    (best, rows): rows holds one dict per schedule in lexicographic order,
    best is the schedule with the smallest largest condition number (the
    pages' choice rule)."""
    T = len(coeffs)
    grid = np.linspace(r_min, 1.0, points)
    rows = []
    def cond(q):          # an overflowed or singular Q counts as unbounded
        aq = np.abs(q)
        if not np.all(np.isfinite(aq)) or np.min(aq) == 0.0:
            return math.inf
        return float(np.max(aq) / np.min(aq))

    with np.errstate(over="ignore", invalid="ignore"):
        for sched in itertools.combinations(range(1, T), n_restarts):
            r_trace, q_trace, _ = restart_model(coeffs, sched, grid, r_min)
            rows.append({"restarts": tuple(sched), "max_cond_q": max(cond(q) for q in q_trace),
                         "max_q": max(float(np.max(np.abs(q))) if np.all(np.isfinite(q)) else math.inf
                                      for q in q_trace),
                         "min_r": min(float(np.min(r)) if np.all(np.isfinite(r)) else -math.inf
                                      for r in r_trace)})
    best = min(rows, key=lambda d: d["max_cond_q"])["restarts"]
    return best, rows

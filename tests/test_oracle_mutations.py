"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one of them (CPU only; the real oracle is never modified)."""
import os
import types

import pytest

from oracle_pins import FAST_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "newton_schulz.py")

MUTATIONS = {
    "Q update drops a*Q": ("Q = Q @ Z + a * Q", "Q = Q @ Z"),
    "RZ sign flipped": ("RZ = R @ Z + a * R", "RZ = R @ Z - a * R"),
    "R update wrong operand": ("R = Z @ RZ + a * RZ", "R = RZ @ RZ + a * RZ"),
    "quadratic b/c swapped (Gram)": ("Z = b * R + c * (R @ R)", "Z = c * R + b * (R @ R)"),
    "quadratic b/c swapped (standard)": ("B = b * A + c * (A @ A)", "B = c * A + b * (A @ A)"),
    "standard update transposed product": ("Y = a * Y + B @ Y", "Y = a * Y + B.T @ B @ Y"),
    "restart off by one": ("if (t - 1) in rs:", "if t in rs:"),
    "restart forgets Q": ("            Y = Q @ Y\n", "            Y = Y\n"),
    "restart keeps Q": ("            Q = _eye(n, Y)\n            step[", "            step["),
    "eps dropped": ("return X / (np.sqrt(np.sum(X * X)) + eps)", "return X / np.sqrt(np.sum(X * X))"),
    "eps inside sqrt": ("return X / (np.sqrt(np.sum(X * X)) + eps)", "return X / np.sqrt(np.sum(X * X) + eps)"),
    "exact eps dropped": ("(_exact_sqrt(s) + Fraction(eps))", "_exact_sqrt(s)"),
    "naive Q uses Z only": ("            Q = Q @ Z\n            R = Z @ R @ Z", "            Q = Z\n            R = Z @ R @ Z"),
    "naive R misses a Z": ("R = Z @ R @ Z", "R = Z @ R"),
    "naive forgets aI": ("Z = a * _eye(n, Y) + b * R", "Z = b * R"),
    "iterations reversed": ("for a, b, c in _coeff_list(coeffs, exact):\n        A", "for a, b, c in reversed(_coeff_list(coeffs, exact)):\n        A"),
    "theorem2 z drops square": ("z = a + b * r + c * r * r", "z = a + b * r + c * r"),
    "theorem2 r update": ("r = r * z * z", "r = r * z"),
    "polynomial degree": ("y = a * y + b * y ** 3 + c * y ** 5", "y = a * y + b * y ** 3 + c * y ** 4"),
    "final apply transposed": ("return Q @ Y, trace", "return Q.T @ Q @ Y, trace"),
    "flops sym": ("return T * (3.0 * m * n * n + n ** 3)", "return T * (3.0 * m * n * n + 2 * n ** 3)"),
    "flops restart": ("n_restarts * (3.0 * m * n * n - 3.0 * n ** 3)", "n_restarts * (3.0 * m * n * n)"),
    "dion3 keeps X rows": ("out[rows, :] = gram_ns(X[rows, :]", "out[rows, :] = gram_ns(X[sorted(rows), :]"),
    "identity wrong": ("return np.eye(n, dtype=np.float64)", "return 2.0 * np.eye(n, dtype=np.float64)"),
    "tall standard not transposed back": ("return standard_ns(X.T, coeffs, eps).T", "return standard_ns(X.T, coeffs, eps)"),
    "tall gram not transposed back": ("return out.T, trace", "return out, trace"),
    "select ties to larger index": ("key=lambda i: (-keys[i], i))", "key=lambda i: (-keys[i], -i))"),
    "select smallest rows": ("key=lambda i: (-keys[i], i))", "key=lambda i: (keys[i], i))"),
    "select l2 instead of l1": ("keys = [math.fsum(np.abs(M[i])) for i in range(n)]", "keys = [math.fsum(M[i] * M[i]) for i in range(n)]"),
    "step momentum not added": ("np.asarray(M, dtype=np.float32) + np.asarray(G, dtype=np.float32)",
                                "np.asarray(M, dtype=np.float32) + 0 * np.asarray(G, dtype=np.float32)"),
    "step selects before the sum": ("S = dion3_select(Msum, k)", "S = dion3_select(np.asarray(M, dtype=np.float64), k)"),
    "normuon root dropped": ("On = O / (np.sqrt(second) + eps)[:, None]", "On = O / (second + eps)[:, None]"),
    "normuon no rescale": ("O = On * (np.linalg.norm(O) / norm_on) if norm_on > 0 else On", "O = On"),
    "normuon zero rescale gives nan": ("O = On * (np.linalg.norm(O) / norm_on) if norm_on > 0 else On",
                                       "O = On * (np.linalg.norm(O) / norm_on) if norm_on >= 0 else On"),
    "normuon sum not mean": ("np.mean(O * O, axis=1)", "np.sum(O * O, axis=1)"),
    "normuon beta swapped": ("second = beta2 * np.asarray(v_rows, dtype=np.float64) + (1.0 - beta2) * np.mean",
                             "second = (1.0 - beta2) * np.asarray(v_rows, dtype=np.float64) + beta2 * np.mean"),
    "decay on selected rows only": ("W_new = (1.0 - lr * weight_decay) * W\n",
                                    "W_new = W.copy()\n    W_new[S, :] *= 1.0 - lr * weight_decay\n"),
    "update sign": ("W_new[S, :] -= lr * O", "W_new[S, :] += lr * O"),
    "error feedback on every row": ("M_new[S, :] *= momentum", "M_new *= momentum"),
    "sweep drops the corruption": ("r = x * x + r_min", "r = x * x"),
    "sweep restart forgets Q": ("            x = q * x\n", "            x = x\n"),
    "sweep R update not squared": ("r = r * (z * z)", "r = r * z"),
    "sweep picks the worst": ("best = min(rows, key=", "best = max(rows, key="),
    "sweep condition from one end": ("return float(np.max(aq) / np.min(aq))", "return float(np.max(aq) / aq[-1])"),
    "sweep spurious direction kept": ("x = np.sqrt(np.maximum(r, 0.0))", "x = np.sqrt(np.abs(r))"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _caught(mod):
    for pin in FAST_PINS:
        try:
            pin(mod)
        except Exception:
            return pin.__name__
    return None


def test_unmutated_copy_passes():
    with open(SRC) as f:
        src = f.read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    assert _caught(mod) is None


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert _caught(_mutant(old, new)) is not None, f"pins missed mutation: {name}"

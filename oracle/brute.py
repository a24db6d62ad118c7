"""Exact-rational brute force of the gated delta rule, for tiny sizes.

TEST INFRASTRUCTURE ONLY.  Materialises the literal matrix form of the update,
S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T and o_t = S_t q_t,
as explicit d x d products of ``fractions.Fraction`` values (no rounding at
all).  It takes alpha and beta directly so the exponentials of the gates are
bypassed, and it shares nothing with the f64 oracle, whose u = S k form it pins.
Pure Python loops: use d <= 4, T <= 6.
"""
from fractions import Fraction


def _matmul(X, Y):
    n, m, p = len(X), len(Y), len(Y[0])
    return [[sum((X[i][l] * Y[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _identity(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def recurrence_exact(q, k, v, alpha, beta, S0=None):
    """Single head.  q, k: T lists of dk Fractions; v: T lists of dv Fractions;
    alpha, beta: T Fractions; S0: dv x dk Fractions or None.
    Returns (o: T lists of dv, S: dv x dk)."""
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = [[Fraction(0)] * dk for _ in range(dv)] if S0 is None else [list(r) for r in S0]
    outs = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        # I - beta k k^T
        M = _identity(dk)
        for i in range(dk):
            for j in range(dk):
                M[i][j] -= Fraction(beta[t]) * kt[i] * kt[j]
        SM = _matmul(S, M)
        S = [[Fraction(alpha[t]) * SM[i][j] + Fraction(beta[t]) * Fraction(v[t][i]) * kt[j]
              for j in range(dk)] for i in range(dv)]
        qt = [[Fraction(x)] for x in q[t]]
        outs.append([row[0] for row in _matmul(S, qt)])
    return outs, S

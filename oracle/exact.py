"""Exact rational brute force of the KDA recurrence -- TEST INFRASTRUCTURE ONLY.

The recurrence of "Ling-3.1-flash: Grouped Routing and Two Different MLA Caches"
(flozi.net), section "KDA replaces a token list with a recurrent matrix" --
retention, corrected delta write, read after the write -- uses only products
and sums once the retention factors alpha = exp(g) are given. With rational
alpha, beta, q, k, v the whole computation is exact in ``fractions.Fraction``:
no rounding at all. Used on tiny inputs (T <= 6, d <= 4) to pin the FP64 oracle.
"""
from fractions import Fraction


def kda_exact(q, k, v, alpha, beta, S0=None, scale=Fraction(1)):
    """q, k, alpha: T lists of dk Fractions; v: T lists of dv Fractions;
    beta: T Fractions. Returns (o: T lists of dv Fractions, S: dk x dv)."""
    T = len(q)
    dk = len(q[0])
    dv = len(v[0])
    S = [[Fraction(0)] * dv for _ in range(dk)] if S0 is None else [list(r) for r in S0]
    outs = []
    for t in range(T):
        # retention of each key-channel row
        S = [[alpha[t][c] * S[c][j] for j in range(dv)] for c in range(dk)]
        # corrected write
        pred = [sum(k[t][c] * S[c][j] for c in range(dk)) for j in range(dv)]
        u = [beta[t] * (v[t][j] - pred[j]) for j in range(dv)]
        S = [[S[c][j] + k[t][c] * u[j] for j in range(dv)] for c in range(dk)]
        # read
        outs.append([scale * sum(q[t][c] * S[c][j] for c in range(dk)) for j in range(dv)])
    return outs, S

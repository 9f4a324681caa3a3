"""Exact rational gated delta rule: an independent, rounding-free cross-check.

The Circuit.LLM.Mixer step ("Delta rule", "Gated memory") written out with
Python ``fractions.Fraction`` scalars in plain nested loops -- no NumPy, no
floating point -- on a preactivated core: rational alpha (scalar or per key
channel), rational beta, rational v, and keys/queries chosen rational
(e.g. Pythagorean unit vectors such as (3/5, 4/5, 0, ...)).  With such
inputs every intermediate is exact, so the float64 oracle must agree to
within its own rounding.  Imports nothing from ``recurrence``.
"""
from fractions import Fraction


def _F(x):
    return x if isinstance(x, Fraction) else Fraction(x)


def exact_scan(S0, Q, Kh, V, alpha, beta):
    """S0: K x Vd nested lists; Q, Kh: T x K; V: T x Vd; alpha: T scalars or T x K; beta: T.

    Returns (O as T x Vd lists of Fractions, final state K x Vd).
    """
    Kd = len(S0)
    Vd = len(S0[0])
    S = [[_F(x) for x in row] for row in S0]
    outs = []
    for t in range(len(Kh)):
        a_t = alpha[t]
        a_row = [_F(a_t[i]) for i in range(Kd)] if isinstance(a_t, (list, tuple)) else [_F(a_t)] * Kd
        # decay the previous state, row i (key channel i) by a_row[i]
        S = [[a_row[i] * S[i][j] for j in range(Vd)] for i in range(Kd)]
        k = [_F(x) for x in Kh[t]]
        q = [_F(x) for x in Q[t]]
        b = _F(beta[t])
        # what the key already retrieves, then the write strength per value column
        v_old = [sum(k[i] * S[i][j] for i in range(Kd)) for j in range(Vd)]
        u = [b * (_F(V[t][j]) - v_old[j]) for j in range(Vd)]
        S = [[S[i][j] + k[i] * u[j] for j in range(Vd)] for i in range(Kd)]
        outs.append([sum(q[i] * S[i][j] for i in range(Kd)) for j in range(Vd)])
    return outs, S

"""Chunked (WY-form) scan of the gated delta rule: an independent cross-check.

The modelopt config page (LinearAttentionConfig) runs GDN/KDA in chunks of
64 tokens and names the steps of that form: gate_prefix, gate_exp,
key_interaction, wy_value, wy_key, state_read, value_residual,
output_state, output_score, output_value, output_add, state_decay,
state_update, state_add; LinearAttentionSolveConfig fixes an exact solve.
The Circuit.LLM.Mixer page ("Chunked additive linear") states the principle
that the chunked form matches the sequential one.  The pages give no
formulas for it, so this form is derived here from the recurrence and
written with those step names:

Within a chunk of C tokens with initial state S0 [K, V], per-token log
gates g_t ([K] vectors; a scalar gate is the same value on every channel):
  gate_prefix     G_t = sum_{s<=t} g_s
  gate_exp        Gamma_t = diag(exp G_t)
  key_interaction A[t, s] = beta_t k_t^T Gamma_t Gamma_s^-1 k_s for s < t
  exact solve     Tm = (I + A)^-1 by forward substitution
  wy_value        U~ = Tm diag(beta) V
  wy_key          W  = Tm diag(beta) (Gamma K)
  state_read / value_residual   U = U~ - W S0
  output_state    O1 = (Gamma Q) S0
  output_score    P[t, s] = q_t^T Gamma_t Gamma_s^-1 k_s for s <= t, else 0
  output_value / output_add     O = O1 + P U
  state_decay     Gamma_C S0
  state_update / state_add      S_C = Gamma_C S0 + sum_s (Gamma_C Gamma_s^-1 k_s) u_s^T
Each Gamma_t Gamma_s^-1 with s <= t is formed as exp(G_t - G_s) (a
non-positive exponent), never as a quotient.

This module imports nothing from ``recurrence``; it works on preactivated
inputs (q_hat, k_hat, v, g, beta) of one head.
"""
import numpy as np


def _forward_substitution_inverse(A):
    """(I + A)^-1 for strictly lower-triangular A, column by column."""
    C = A.shape[0]
    Tm = np.zeros((C, C))
    for col in range(C):
        e = np.zeros(C)
        e[col] = 1.0
        x = np.zeros(C)
        for t in range(C):
            x[t] = e[t] - A[t, :t] @ x[:t]
        Tm[:, col] = x
    return Tm


def chunk_step(S0, Q, Kh, V, g, beta):
    """One chunk: S0 [K, V]; Q, Kh [C, K]; V [C, Vd]; g [C, K]; beta [C] -> (O [C, Vd], S_C)."""
    C = Q.shape[0]
    G = np.cumsum(g, axis=0)                          # gate_prefix [C, K]
    GK = np.exp(G) * Kh                               # gate_exp applied to keys
    GQ = np.exp(G) * Q
    # pairwise decay exp(G_t - G_s) [C, C, K], only used where s <= t
    D = G[:, None, :] - G[None, :, :]
    mask_le = np.tril(np.ones((C, C), dtype=bool))
    Dexp = np.where(mask_le[:, :, None], np.exp(np.where(mask_le[:, :, None], D, 0.0)), 0.0)
    KK = np.einsum("tc,tsc,sc->ts", Kh, Dexp, Kh)      # k_t^T Gamma_t Gamma_s^-1 k_s
    A = np.tril(beta[:, None] * KK, k=-1)             # key_interaction (strict)
    Tm = _forward_substitution_inverse(A)             # exact solve
    U_t = Tm @ (beta[:, None] * V)                    # wy_value
    W = Tm @ (beta[:, None] * GK)                     # wy_key
    U = U_t - W @ S0                                  # state_read, value_residual
    P = np.einsum("tc,tsc,sc->ts", Q, Dexp, Kh)       # output_score (s <= t)
    O = GQ @ S0 + P @ U                               # output_state, output_value, output_add
    dC = np.exp(G[-1][None, :] - G)                   # Gamma_C Gamma_s^-1  [C, K]
    S_C = np.exp(G[-1])[:, None] * S0 + (dC * Kh).T @ U   # state_decay, state_update, state_add
    return O, S_C


def chunked_scan(S0, Q, Kh, V, g, beta, chunk_size=64):
    """Whole suffix in chunks of ``chunk_size`` (the last chunk may be shorter).

    S0 [K, V]; Q, Kh [T, K]; V [T, Vd]; g [T] (scalar gate) or [T, K]; beta [T].
    Returns (O [T, Vd], S_T).
    """
    T, K = Kh.shape
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 1:
        g = np.repeat(g[:, None], K, axis=1)
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((T, V.shape[1]))
    for c0 in range(0, T, chunk_size):
        c1 = min(T, c0 + chunk_size)
        O[c0:c1], S = chunk_step(S, Q[c0:c1], Kh[c0:c1], V[c0:c1], g[c0:c1], beta[c0:c1])
    return O, S

"""Explicit transition-product form of the gated delta rule: an independent cross-check.

Substituting the delta write into the decayed state gives, per token,
  S_t = M_t S_{t-1} + beta_t k_t v_t^T,   M_t = (I - beta_t k_t k_t^T) D_t,
with D_t = diag(alpha_t) (alpha_t a scalar for GDN, a vector over key
channels for KDA; Circuit.LLM.Mixer, "Delta rule" and "Gated memory").
Unrolling,
  S_T = (M_T ... M_1) S_0 + sum_s (M_T ... M_{s+1}) beta_s k_s v_s^T,
and the readout after token t is o_t = q_t S_t.  This module forms those
K x K products explicitly, one prefix at a time, and imports nothing from
``recurrence``.  Used only on small T.
"""
import numpy as np


def transition(k, alpha, beta):
    """M = (I - beta k k^T) diag(alpha) for one token (alpha scalar or [K])."""
    K = k.shape[0]
    alpha = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (K,))
    return (np.eye(K) - beta * np.outer(k, k)) @ np.diag(alpha)


def unrolled_scan(S0, Q, Kh, V, alpha, beta):
    """S0 [K, V]; Q, Kh [T, K]; V [T, Vd]; alpha [T] or [T, K]; beta [T] -> (O [T, Vd], S_T).

    Each S_t is rebuilt from S_0 through the full products, not carried.
    """
    T, K = Kh.shape
    Ms = [transition(Kh[t], alpha[t], beta[t]) for t in range(T)]
    O = np.zeros((T, V.shape[1]))
    S_t = np.array(S0, dtype=np.float64)
    for t in range(T):
        prod = np.eye(K)
        for i in range(t, -1, -1):
            prod = prod @ Ms[i]                     # M_t ... M_i
        S_t = prod @ S0
        for s in range(t + 1):
            tail = np.eye(K)
            for i in range(t, s, -1):
                tail = tail @ Ms[i]                 # M_t ... M_{s+1}
            S_t = S_t + beta[s] * tail @ np.outer(Kh[s], V[s])
        O[t] = Q[t] @ S_t
    return O, S_t

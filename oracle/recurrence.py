"""Sequential gated delta-rule recurrence, float64, one step at a time.

Pages followed:
* Circuit.LLM.Mixer, "Delta rule" (deltaAttnStep): with S a [K, V] matrix
  acting on row vectors, what the key already retrieves is k S; the write is
  u = beta (v - k S), S' = S + k^T u, and the readout is o = q S' (the
  updated state).
* Circuit.LLM.Mixer, "Gated memory" (gatedDeltaStep, kdaLiteStep): decay
  the previous state first, then do the delta write.  alpha = 1 is the pure
  delta rule, alpha = 0 forgets everything before writing.  KDA-lite decays
  with a vector alpha over key channels.
* modelopt ... linear_attention.decode, recurrent_decode_reference: the
  reference takes one sequence whose activations are already applied, log
  gates that are either one number per head (GDN) or a vector over the key
  rows (KDA), and keys already mapped onto the value heads; called with no
  tokens it neither writes nor quantises the initial state.

Reading of the KDA decay axis (the Haddock text says "column" while its
own o = q S convention makes rows the key index, and the kda_decode gate is
laid out over key_head_dim): alpha[c] scales ROW c of S[K, V], i.e. the key
channel.

The step runs on a stack of heads: S [H, K, V], q_hat/k_hat [H, K],
v [H, V], alpha [H] (scalar gate) or [H, K] (per key channel), beta [H].

Pins (tests/test_oracle_recurrence.py): beta = 0 and g = 0 leave S
unchanged; beta = 0 is pure decay; alpha = 0 gives S' = beta k^T v and
o = beta (q.k) v; alpha = beta = 1 with orthonormal keys recovers every
stored value; scalar gate == KDA gate with equal channels; hand-worked
examples under tests/golden/; and agreement with the independent chunked,
unrolled and exact-rational forms.
"""
import numpy as np


def decay(S, alpha):
    """S <- alpha * S; alpha [H] scales whole heads, alpha [H, K] scales key rows."""
    alpha = np.asarray(alpha, dtype=np.float64)
    if alpha.ndim == 1:
        return alpha[:, None, None] * S
    return alpha[:, :, None] * S


def delta_write(S, k_hat, v, beta):
    """u = beta (v - k S);  S' = S + k^T u.  Returns S'."""
    v_old = np.einsum("hk,hkv->hv", k_hat, S)
    u = np.asarray(beta, dtype=np.float64)[:, None] * (v - v_old)
    return S + np.einsum("hk,hv->hkv", k_hat, u)


def readout(S, q_hat):
    """o = q S over the key axis: [H, V]."""
    return np.einsum("hk,hkv->hv", q_hat, S)


def gated_delta_step(S, q_hat, k_hat, v, alpha, beta, state_qdq=None, readout_mode="working"):
    """One token: decay, delta write, readout; optional state quantise/dequantise.

    ``state_qdq`` (callable S -> S) is applied after the update.  With
    ``readout_mode='working'`` the output reads the updated state before that
    rounding; with ``'stored'`` it reads the rounded state.
    Returns (o [H, V], S_next [H, K, V]).
    """
    S = decay(S, alpha)
    S = delta_write(S, k_hat, v, beta)
    if state_qdq is None:
        return readout(S, q_hat), S
    if readout_mode == "working":
        o = readout(S, q_hat)
        return o, state_qdq(S)
    if readout_mode == "stored":
        S = state_qdq(S)
        return readout(S, q_hat), S
    raise ValueError(f"unknown readout mode {readout_mode!r}")


def run_suffix(S0, q_hat, k_hat, v, alpha, beta, state_qdq=None, quantize_initial=False,
               readout_mode="working", trace=None):
    """Left fold of the step over the T tokens of one suffix (scanMixer shape).

    S0 [H, K, V]; q_hat/k_hat [T, H, K]; v [T, H, V]; alpha [T, H] or
    [T, H, K]; beta [T, H].  Returns (o [T, H, V], S_T).  With T = 0 the
    state is returned untouched and no initial quantisation happens.
    If ``trace`` is a list, one dict per token is appended with the state
    entering the token and the token's q_hat, k_hat, alpha, beta and the
    state leaving it (instrumentation for tests; no effect on the result).
    """
    T = q_hat.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    outs = np.zeros((T,) + (S.shape[0], S.shape[2]), dtype=np.float64)
    if T == 0:
        return outs, S
    if state_qdq is not None and quantize_initial:
        S = state_qdq(S)
    for t in range(T):
        S_in = S
        outs[t], S = gated_delta_step(S, q_hat[t], k_hat[t], v[t], alpha[t], beta[t],
                                      state_qdq=state_qdq, readout_mode=readout_mode)
        if trace is not None:
            trace.append(dict(S_in=S_in, q_hat=q_hat[t], k_hat=k_hat[t], alpha=alpha[t], beta=beta[t], S_out=S))
    return outs, S

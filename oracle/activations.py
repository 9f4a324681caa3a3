"""Fused input activations of the decode step, in float64.

Pages followed:
* max.nn.state_space.kda_decode -- description: the op takes q and k
  unnormalised, normalises both to unit L2 length itself and multiplies q by
  1/sqrt(key_head_dim); it also applies the gate and beta nonlinearities
  (``gate_mode``, ``beta_mode``).  Parameters: ``raw_gate`` is the gate
  input to which ``dt_bias`` has not yet been added, ``a_log`` has one value
  per value head, and ``beta_mode`` says whether a sigmoid is taken.
* flashinfer.gdn_paged.gated_delta_rule_decode_paged -- signature: ``A_log``,
  ``a``, ``dt_bias``, ``b``, ``scale=None``, ``use_qk_l2norm=True``.

Readings where the pages are silent:
* L2 norm epsilon: x / sqrt(sum(x^2) + 1e-6).
* gate: g = -exp(A_log) * softplus(a + dt_bias), the log of the decay
  factor alpha = exp(g); for KDA the same per key channel.
* softplus(x) = max(x, 0) + log1p(exp(-|x|)) (the overflow-free identity;
  no large-x threshold).
* beta = sigmoid(b) in ``logits`` mode, b itself in ``probability`` mode.

Pins: tests/test_oracle_activations.py checks these against scalar
``math`` library evaluations and closed-form special values
(softplus(0) = ln 2, sigmoid(0) = 1/2, unit norm of the normalised vector).
"""
import numpy as np

L2NORM_EPS = 1e-6


def l2_normalize(x, eps=L2NORM_EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis (head dim)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x):
    """log(1 + exp(x)) written as max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + exp(-x)), evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gdn_log_gate(A_log, a, dt_bias):
    """Scalar-per-head log decay g = -exp(A_log[h]) * softplus(a[..., h] + dt_bias[h]).

    A_log, dt_bias: [HV]; a: [..., HV].  Returns g with the shape of ``a``.
    """
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    return -np.exp(A_log) * softplus(np.asarray(a, dtype=np.float64) + dt_bias)


def kda_log_gate(a_log, raw_gate, dt_bias):
    """Per-key-channel log decay g[..., h, c] = -exp(a_log[h]) * softplus(raw_gate[..., h, c] + dt_bias[h, c]).

    a_log: [HV]; dt_bias: [HV, K]; raw_gate: [..., HV, K].
    """
    a_log = np.asarray(a_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    x = np.asarray(raw_gate, dtype=np.float64) + dt_bias
    return -np.exp(a_log)[:, None] * softplus(x)


def beta_from(b, beta_mode="logits"):
    """Write strength: sigmoid(b) for ``logits``, b unchanged for ``probability``."""
    if beta_mode == "logits":
        return sigmoid(b)
    if beta_mode == "probability":
        return np.asarray(b, dtype=np.float64)
    raise ValueError(f"unknown beta_mode {beta_mode!r}")


def prepare_qk(q, k, scale=None, use_qk_l2norm=True):
    """Normalised query and key of one token: q_hat = l2n(q) * scale, k_hat = l2n(k).

    ``scale`` None means 1/sqrt(K), K being the last axis length.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    if use_qk_l2norm:
        q = l2_normalize(q)
        k = l2_normalize(k)
    return q * scale, k

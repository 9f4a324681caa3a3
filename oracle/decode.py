"""The three decode front-ends: pooled GDN, CSR-paged GDN, pooled KDA.

Each one resolves the rows a sequence reads and writes (``paging``), turns
raw inputs into q_hat, k_hat, alpha = exp(g), beta (``activations``), and
folds the step over the sequence's suffix tokens (``recurrence``), with the
optional state quantise/dequantise (``e4m3`` tiles or the ``hadamard``
int8_hadamard32 codec).  Everything is float64.

Pages followed:
* max.nn.state_space.kda_decode (signature, Parameters, Returns);
* flashinfer.gdn_paged.gated_delta_rule_decode_paged (signature,
  description, Parameters, Returns: [B, 1, HV, V]);
* modelopt ... linear_attention.decode, recurrent_decode_reference, and
  modelopt ... linear_attention.config, LinearAttentionDecodeConfig
  (``quantize_initial``, ``readout``).

Reading of the key-head to value-head map (the decode reference only says
keys must already be aligned with value heads): value head h uses key head
h // (HV / HK), i.e. consecutive value heads share a key head.

``pool`` is anything indexable by a slot or page id that returns that row's
[HV, ...] tile in pool layout (a NumPy array, or a dict holding only the
rows the call reads).  Each function returns ``(out, written)``:
``out`` [T, HV, V] float64 (rows of sequences not in ``seqs`` are NaN) and
``written`` a dict {row id: new tile in pool layout, float64}.  Rows not in
``written`` are not modified by the call.  ``qdq_precision`` is the
precision in which the state rounding decides its codes (oracle.e4m3,
oracle.hadamard): float64 by default.  ``trace`` (a dict, optional)
receives per sequence the per-token record of ``recurrence.run_suffix``.
"""
import numpy as np

from . import activations as act
from . import e4m3
from . import hadamard
from . import paging
from .recurrence import run_suffix


def _qdq_fn(qdq, block_v, precision="float64"):
    if qdq is None or qdq == "none":
        return None
    if qdq == "fp8_e4m3_tile":
        return lambda S: e4m3.tile_qdq(S, block_v, precision)
    if qdq == "int8_hadamard32":
        # block_v is only the execution tile width for this codec
        return lambda S: hadamard.int8_hadamard32_qdq(S, precision)
    raise ValueError(f"unknown qdq {qdq!r}")


def _key_head_map(HK, HV):
    if HV % HK != 0:
        raise ValueError("HV must be a multiple of HK")
    return np.arange(HV) // (HV // HK)


def _run_one(tile, state_layout, q, k, v, alpha, beta, hk_of_h, scale, use_qk_l2norm,
             qdq_fn, quantize_initial, readout, trace=None):
    """Run one sequence's suffix.  q, k [T, HK, K]; v [T, HV, V]; alpha [T, HV] or [T, HV, K]."""
    S0 = paging.to_logical(tile, state_layout)
    q_hat, k_hat = act.prepare_qk(q, k, scale=scale, use_qk_l2norm=use_qk_l2norm)
    q_hat = q_hat[:, hk_of_h, :]
    k_hat = k_hat[:, hk_of_h, :]
    o, S = run_suffix(S0, q_hat, k_hat, np.asarray(v, dtype=np.float64), alpha, beta,
                      state_qdq=qdq_fn, quantize_initial=quantize_initial, readout_mode=readout,
                      trace=trace)
    return o, paging.from_logical(S, state_layout)


def gdn_decode_pooled(q, k, v, a, b, A_log, dt_bias, cu_seqlens, state_indices, pool, *,
                      scale=None, use_qk_l2norm=True, beta_mode="logits", state_layout="K_FIRST",
                      qdq=None, block_v=64, quantize_initial=False, readout="working", seqs=None,
                      trace=None, qdq_precision="float64"):
    """GDN (scalar gate per value head) decode on a slot pool, varlen suffixes.

    q, k [T, HK, K]; v [T, HV, V]; a, b [T, HV]; A_log, dt_bias [HV];
    cu_seqlens [B+1] or None (one token per sequence, B = T);
    state_indices [B].
    """
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    B = len(state_indices)
    hk_of_h = _key_head_map(HK, HV)
    qdq_fn = _qdq_fn(qdq, block_v, qdq_precision)
    out = np.full((T, HV, V), np.nan)
    written = {}
    for bi in (range(B) if seqs is None else seqs):
        t0, t1 = paging.pooled_token_range(cu_seqlens, bi)
        if t1 <= t0:
            continue
        r, w = paging.pooled_rows(state_indices, bi)
        alpha = np.exp(act.gdn_log_gate(A_log, a[t0:t1], dt_bias))
        beta = act.beta_from(b[t0:t1], beta_mode)
        o, tile = _run_one(pool[r], state_layout, q[t0:t1], k[t0:t1], v[t0:t1], alpha, beta,
                           hk_of_h, scale, use_qk_l2norm, qdq_fn, quantize_initial, readout,
                           None if trace is None else trace.setdefault(bi, []))
        out[t0:t1] = o
        written[w] = tile
    return out, written


def kda_decode_pooled(q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_indices,
                      pool, *, scale=None, use_qk_l2norm=True, beta_mode="logits",
                      state_layout="K_FIRST", qdq=None, block_v=64, quantize_initial=False,
                      readout="working", seqs=None, trace=None, qdq_precision="float64"):
    """KDA (per-key-channel gate) decode on a slot pool, varlen suffixes.

    q, k [T, HK, K]; v [T, HV, V]; raw_gate [T, HV, K]; beta_logits [T, HV];
    a_log [HV]; dt_bias [HV, K]; cu_seqlens [B+1]; state_indices [B].
    """
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    B = len(state_indices)
    hk_of_h = _key_head_map(HK, HV)
    qdq_fn = _qdq_fn(qdq, block_v, qdq_precision)
    out = np.full((T, HV, V), np.nan)
    written = {}
    for bi in (range(B) if seqs is None else seqs):
        t0, t1 = paging.pooled_token_range(cu_seqlens, bi)
        if t1 <= t0:
            continue
        r, w = paging.pooled_rows(state_indices, bi)
        alpha = np.exp(act.kda_log_gate(a_log, raw_gate[t0:t1], dt_bias))
        beta = act.beta_from(beta_logits[t0:t1], beta_mode)
        o, tile = _run_one(pool[r], state_layout, q[t0:t1], k[t0:t1], v[t0:t1], alpha, beta,
                           hk_of_h, scale, use_qk_l2norm, qdq_fn, quantize_initial, readout,
                           None if trace is None else trace.setdefault(bi, []))
        out[t0:t1] = o
        written[w] = tile
    return out, written


def _paged_varlen(kind, q, k, v, gate, beta_in, A_log, dt_bias, cu_seqlens, page_indices, page_indptr,
                  last_page_len, page_size, pool, scale, use_qk_l2norm, beta_mode, state_layout, qdq, block_v,
                  quantize_initial, readout, seqs, trace, qdq_precision):
    """Several decoded tokens per sequence on a CSR-paged pool (see paging.paged_suffix_rows).

    Each page that a suffix token fills receives the state after that token;
    the last page receives the final state.  Rows are written in token order.
    """
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    B = len(cu_seqlens) - 1
    hk_of_h = _key_head_map(HK, HV)
    qdq_fn = _qdq_fn(qdq, block_v, qdq_precision)
    out = np.full((T, HV, V), np.nan)
    written = {}
    for bi in (range(B) if seqs is None else seqs):
        t0, t1 = paging.pooled_token_range(cu_seqlens, bi)
        if t1 <= t0:
            continue
        r, writes = paging.paged_suffix_rows(page_indices, page_indptr, last_page_len, page_size, t1 - t0, bi)
        if kind == "kda":
            alpha = np.exp(act.kda_log_gate(A_log, gate[t0:t1], dt_bias))
        else:
            alpha = np.exp(act.gdn_log_gate(A_log, gate[t0:t1], dt_bias))
        beta = act.beta_from(beta_in[t0:t1], beta_mode)
        S = pool[r]
        done = 0
        for i, row in writes:
            # tokens done..i: the state carries over between pieces of the suffix
            o, S = _run_one(S, state_layout, q[t0 + done:t0 + i + 1], k[t0 + done:t0 + i + 1],
                            v[t0 + done:t0 + i + 1], alpha[done:i + 1], beta[done:i + 1], hk_of_h, scale,
                            use_qk_l2norm, qdq_fn, quantize_initial and done == 0, readout,
                            None if trace is None else trace.setdefault(bi, []))
            out[t0 + done:t0 + i + 1] = o
            written[row] = S
            done = i + 1
    return out, written


def gdn_decode_paged_varlen(q, k, v, a, b, A_log, dt_bias, cu_seqlens, page_indices, page_indptr,
                            last_page_len, page_size, pool, *, scale=None, use_qk_l2norm=True,
                            beta_mode="logits", state_layout="V_FIRST", qdq=None, block_v=64,
                            quantize_initial=False, readout="working", seqs=None, trace=None,
                            qdq_precision="float64"):
    """GDN decode of varlen suffixes on a CSR-paged pool; cu_seqlens [B+1] as in kda_decode."""
    return _paged_varlen("gdn", q, k, v, a, b, A_log, dt_bias, cu_seqlens, page_indices, page_indptr,
                         last_page_len, page_size, pool, scale, use_qk_l2norm, beta_mode, state_layout, qdq,
                         block_v, quantize_initial, readout, seqs, trace, qdq_precision)


def kda_decode_paged_varlen(q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, page_indices, page_indptr,
                            last_page_len, page_size, pool, *, scale=None, use_qk_l2norm=True,
                            beta_mode="logits", state_layout="V_FIRST", qdq=None, block_v=64,
                            quantize_initial=False, readout="working", seqs=None, trace=None,
                            qdq_precision="float64"):
    """KDA decode of varlen suffixes on a CSR-paged pool (per-key-channel gate)."""
    return _paged_varlen("kda", q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, page_indices,
                         page_indptr, last_page_len, page_size, pool, scale, use_qk_l2norm, beta_mode,
                         state_layout, qdq, block_v, quantize_initial, readout, seqs, trace, qdq_precision)


def kda_decode_paged(q, k, v, raw_gate, beta_logits, a_log, dt_bias, page_indices, page_indptr, last_page_len,
                     pool, *, scale=None, use_qk_l2norm=True, beta_mode="logits", state_layout="V_FIRST",
                     qdq=None, block_v=64, quantize_initial=False, readout="working", seqs=None, trace=None,
                     qdq_precision="float64"):
    """Single-token KDA decode on a CSR-paged pool: the paging of gated_delta_rule_decode_paged
    (flashinfer.gdn_paged) with the gate of kda_decode (max.nn.state_space)."""
    B, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    hk_of_h = _key_head_map(HK, HV)
    qdq_fn = _qdq_fn(qdq, block_v, qdq_precision)
    out = np.full((B, HV, V), np.nan)
    written = {}
    for bi in (range(B) if seqs is None else seqs):
        r, w = paging.paged_rows(page_indices, page_indptr, last_page_len, bi)
        sl = slice(bi, bi + 1)
        alpha = np.exp(act.kda_log_gate(a_log, raw_gate[sl], dt_bias))
        beta = act.beta_from(beta_logits[sl], beta_mode)
        o, tile = _run_one(pool[r], state_layout, q[sl], k[sl], v[sl], alpha, beta, hk_of_h,
                           scale, use_qk_l2norm, qdq_fn, quantize_initial, readout,
                           None if trace is None else trace.setdefault(bi, []))
        out[bi] = o[0]
        written[w] = tile
    return out, written


def gdn_decode_paged(q, k, v, a, b, A_log, dt_bias, page_indices, page_indptr, last_page_len,
                     pool, *, scale=None, use_qk_l2norm=True, beta_mode="logits",
                     state_layout="V_FIRST", qdq=None, block_v=64, quantize_initial=False,
                     readout="working", seqs=None, trace=None, qdq_precision="float64"):
    """GDN decode of one token per sequence on a CSR-paged pool (token b belongs to sequence b).

    q, k [B, HK, K]; v [B, HV, V]; a, b [B, HV]; returns out [B, HV, V]
    (the [B, 1, HV, V] output without its unit axis).
    """
    B, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    hk_of_h = _key_head_map(HK, HV)
    qdq_fn = _qdq_fn(qdq, block_v, qdq_precision)
    out = np.full((B, HV, V), np.nan)
    written = {}
    for bi in (range(B) if seqs is None else seqs):
        r, w = paging.paged_rows(page_indices, page_indptr, last_page_len, bi)
        sl = slice(bi, bi + 1)
        alpha = np.exp(act.gdn_log_gate(A_log, a[sl], dt_bias))
        beta = act.beta_from(b[sl], beta_mode)
        o, tile = _run_one(pool[r], state_layout, q[sl], k[sl], v[sl], alpha, beta, hk_of_h,
                           scale, use_qk_l2norm, qdq_fn, quantize_initial, readout,
                           None if trace is None else trace.setdefault(bi, []))
        out[bi] = o[0]
        written[w] = tile
    return out, written

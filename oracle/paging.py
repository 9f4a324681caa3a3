"""Which pool rows a decode call reads and writes.

Pages followed:
* max.nn.state_space.kda_decode, Parameters: ``cu_seqlens`` [B+1] holds
  exclusive prefix offsets of each sequence's suffix tokens;
  ``state_indices`` [B] names the pool slot of each sequence; the pool is
  mutated in place.
* flashinfer.gdn_paged.gated_delta_rule_decode_paged, description: sequence
  b ends with its decoded token, which occupies slot ``last_page_len[b]``
  of the final page in its table row.  A decoded token in slot 1 starts
  that page, so the pre-token state comes from the page before it, the
  post-token state goes to the final page, and the page before (which
  other sequences may share) keeps its contents; in any other slot the
  final page is both the source and the destination.  Parameters: a CSR
  table, ``page_indptr`` [B+1] and ``page_indices`` [nnz].  Notes: the
  decoded token is never a sequence's first token.
* modelopt ... linear_attention.decode, recurrent_decode_reference: a call
  with no tokens writes nothing.

Pins (tests/test_oracle_paging.py): brute force over small CSR tables
against a token-position model (the state after token n lives on the page
holding token n), and a multi-call simulation of a growing sequence on a
paged pool against one sequential run over all its tokens.
"""
import numpy as np


def pooled_token_range(cu_seqlens, b):
    """[start, end) token rows of sequence b; ``cu_seqlens`` None means one token each."""
    if cu_seqlens is None:
        return b, b + 1
    return int(cu_seqlens[b]), int(cu_seqlens[b + 1])


def pooled_rows(state_indices, b):
    """(read slot, write slot) of sequence b in a slot pool: both are state_indices[b]."""
    s = int(state_indices[b])
    return s, s


def paged_rows(page_indices, page_indptr, last_page_len, b):
    """(read page, write page) of sequence b for one decoded token on a CSR-paged pool."""
    end = int(page_indptr[b + 1])
    last = int(page_indices[end - 1])
    if int(last_page_len[b]) == 1:
        return int(page_indices[end - 2]), last
    return last, last


def paged_suffix_rows(page_indices, page_indptr, last_page_len, page_size, n_suffix, b):
    """Rows touched by a suffix of ``n_suffix`` tokens of sequence b on a CSR-paged pool.

    Extends the single-token rule of gated_delta_rule_decode_paged
    (flashinfer.gdn_paged, description) to several appended tokens, with the
    same model that rule follows: the state after token m lives on the page
    that holds token m.  The sequence holds n = (pages - 1) * page_size +
    last_page_len tokens after the suffix, the suffix is tokens
    n - n_suffix + 1 .. n (1-based), and at least one token precedes it
    (flashinfer.gdn_paged, Notes).

    Returns (read row, [(i, row), ...]): the page holding token
    n - n_suffix supplies the starting state; suffix token i (0-based)
    stores its state to ``row`` when it completes a page or ends the
    suffix.
    """
    start = int(page_indptr[b])
    n = (int(page_indptr[b + 1]) - start - 1) * page_size + int(last_page_len[b])
    m0 = n - n_suffix + 1
    if m0 < 2:
        raise ValueError("a paged suffix needs at least one token before it")
    page_of = lambda m: int(page_indices[start + (m - 1) // page_size])
    writes = []
    for i in range(n_suffix):
        m = m0 + i
        if m % page_size == 0 or m == n:
            writes.append((i, page_of(m)))
    return page_of(m0 - 1), writes


def to_logical(tile, state_layout):
    """Pool tile -> logical S[..., K, V].  K_FIRST stores (K, V); V_FIRST stores (V, K)."""
    if state_layout == "K_FIRST":
        return np.asarray(tile, dtype=np.float64)
    if state_layout == "V_FIRST":
        return np.swapaxes(np.asarray(tile, dtype=np.float64), -1, -2)
    raise ValueError(f"unknown state_layout {state_layout!r}")


def from_logical(S, state_layout):
    """Logical S[..., K, V] -> pool tile in the given layout."""
    if state_layout == "K_FIRST":
        return S
    if state_layout == "V_FIRST":
        return np.swapaxes(S, -1, -2)
    raise ValueError(f"unknown state_layout {state_layout!r}")

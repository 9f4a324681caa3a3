"""Which pool rows a decode call reads and writes.

Pages followed:
* max.nn.state_space.kda_decode, Parameters: ``cu_seqlens`` [B+1] holds
  exclusive prefix offsets of each sequence's suffix tokens;
  ``state_indices`` [B] names the pool slot of each sequence; the pool is
  mutated in place.
* flashinfer.gdn_paged.gated_delta_rule_decode_paged, description: the
  decoded token is the last token of its sequence, at position
  ``last_page_len[b]`` of the sequence's last page.  If it opens a new page
  (``last_page_len[b] == 1``) the state is read from the previous page and
  written to the new one, leaving the previous (possibly shared) page
  untouched; otherwise the last page is read and updated in place.
  Parameters: CSR ``page_indptr`` [B+1] / ``page_indices`` [nnz].  Notes:
  every sequence holds at least one token before the decoded one.
* modelopt ... linear_attention.decode, recurrent_decode_reference: an empty
  call performs no write.

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

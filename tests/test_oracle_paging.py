"""Pins of the slot/page resolution against a token-position model and a growing-sequence simulation.

flashinfer.gdn_paged.gated_delta_rule_decode_paged (description, Parameters,
Notes) fixes where the decoded token sits (position last_page_len[b] of the
last page) and what a token that opens a new page reads and writes.  The
model used here is independent of that rule's wording: the state after
token m of a sequence lives on the page that holds token m, so decoding
token n reads the page of token n-1 and writes the page of token n.
"""
import numpy as np
import pytest

from oracle import decode as odec
from oracle import paging
from oracle.recurrence import run_suffix
from oracle import activations as act


def _table(lengths, page_size, rng):
    """CSR table for sequences of ``lengths`` tokens (decoded token included), random page ids."""
    pages = [-(-n // page_size) for n in lengths]
    ids = rng.permutation(sum(pages) + 7)[:sum(pages)]
    indptr = np.concatenate([[0], np.cumsum(pages)])
    last_len = np.array([n - page_size * (p - 1) for n, p in zip(lengths, pages)])
    return ids, indptr, last_len


@pytest.mark.parametrize("page_size", [1, 2, 3, 4, 16])
def test_paged_rows_match_token_position_model(page_size):
    rng = np.random.default_rng(page_size)
    lengths = list(range(2, 3 * page_size + 4)) + list(rng.integers(2, 200, 30))
    ids, indptr, last_len = _table(lengths, page_size, rng)
    for b, n in enumerate(lengths):
        page_of = lambda m: int(ids[indptr[b] + (m - 1) // page_size])     # token m is 1-based
        r, w = paging.paged_rows(ids, indptr, last_len, b)
        assert (r, w) == (page_of(n - 1), page_of(n))
        assert 1 <= last_len[b] <= page_size


def _gdn_tokens(rng, T, HK, HV, K, V):
    return dict(q=rng.standard_normal((T, HK, K)), k=rng.standard_normal((T, HK, K)),
                v=rng.standard_normal((T, HV, V)), a=rng.standard_normal((T, HV)),
                b=rng.standard_normal((T, HV)))


@pytest.mark.parametrize("page_size", [1, 3, 4])
def test_growing_sequence_on_paged_pool_equals_one_sequential_run(page_size):
    rng = np.random.default_rng(40 + page_size)
    HK, HV, K, V = 1, 2, 4, 3
    A_log = rng.uniform(0, np.log(16), HV)
    dt = rng.uniform(-1, 1, HV)
    n0, n_end = 5, 17                          # prefix of 5 tokens, then decode tokens 6..17
    toks = _gdn_tokens(rng, n_end, HK, HV, K, V)
    S_prefix = rng.standard_normal((HV, K, V)) * 0.1   # state after token n0 (V_FIRST pool)
    n_pages = -(-n_end // page_size)
    page_ids = list(rng.permutation(n_pages + 5)[:n_pages])
    pool = {}
    pool[page_ids[(n0 - 1) // page_size]] = np.swapaxes(S_prefix, -1, -2)
    snapshots = {}
    for n in range(n0 + 1, n_end + 1):
        pages = -(-n // page_size)
        ids = np.array(page_ids[:pages])
        indptr = np.array([0, pages])
        last_len = np.array([n - page_size * (pages - 1)])
        t = n - 1
        out, written = odec.gdn_decode_paged(toks["q"][t:t + 1], toks["k"][t:t + 1], toks["v"][t:t + 1],
                                             toks["a"][t:t + 1], toks["b"][t:t + 1], A_log, dt,
                                             ids, indptr, last_len, pool)
        (w, tile), = written.items()
        assert w == page_ids[(n - 1) // page_size]
        before = {p: v.copy() for p, v in pool.items() if p != w}
        pool[w] = tile
        for p, v in before.items():
            assert np.array_equal(pool[p], v)       # nothing but the write page changes
        snapshots[n] = (out[0], tile.copy())
    # one sequential run over tokens n0+1..n_end from the prefix state
    q_hat, k_hat = act.prepare_qk(toks["q"][n0:], toks["k"][n0:])
    alpha = np.exp(act.gdn_log_gate(A_log, toks["a"][n0:], dt))
    beta = act.beta_from(toks["b"][n0:])
    hk = np.arange(HV) // (HV // HK)
    o_seq, S_end = run_suffix(S_prefix, q_hat[:, hk], k_hat[:, hk], toks["v"][n0:], alpha, beta)
    for i, n in enumerate(range(n0 + 1, n_end + 1)):
        np.testing.assert_allclose(snapshots[n][0], o_seq[i], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(np.swapaxes(pool[page_ids[(n_end - 1) // page_size]], -1, -2), S_end,
                               rtol=1e-13, atol=1e-14)
    # every full page still holds the state after its last token
    for p in range((n0 - 1) // page_size + 1, (n_end - 1) // page_size):
        last_tok = (p + 1) * page_size
        if last_tok > n0:
            np.testing.assert_allclose(pool[page_ids[p]], snapshots[last_tok][1], rtol=0, atol=0)


def test_shared_previous_page_is_read_by_two_sequences_and_written_by_neither():
    rng = np.random.default_rng(50)
    HK, HV, K, V = 1, 1, 4, 4
    A_log, dt = rng.uniform(0, 1, HV), rng.uniform(-1, 1, HV)
    toks = _gdn_tokens(rng, 2, HK, HV, K, V)
    pool = {7: rng.standard_normal((HV, V, K)), 3: np.zeros((HV, V, K)), 9: np.zeros((HV, V, K))}
    # both sequences: page 7 full (shared prefix), decoded token opens pages 3 and 9
    ids = np.array([7, 3, 7, 9])
    indptr = np.array([0, 2, 4])
    last_len = np.array([1, 1])
    keep = pool[7].copy()
    out, written = odec.gdn_decode_paged(toks["q"], toks["k"], toks["v"], toks["a"], toks["b"], A_log, dt,
                                         ids, indptr, last_len, pool)
    assert set(written) == {3, 9}
    assert np.array_equal(pool[7], keep)
    # identical inputs from the same read page give identical results
    toks2 = {kk: np.repeat(vv[:1], 2, axis=0) for kk, vv in toks.items()}
    out2, written2 = odec.gdn_decode_paged(toks2["q"], toks2["k"], toks2["v"], toks2["a"], toks2["b"], A_log, dt,
                                           ids, indptr, last_len, pool)
    assert np.array_equal(written2[3], written2[9])


def test_pooled_rows_and_token_ranges():
    cu = np.array([0, 3, 3, 7])
    assert paging.pooled_token_range(cu, 0) == (0, 3)
    assert paging.pooled_token_range(cu, 1) == (3, 3)
    assert paging.pooled_token_range(None, 5) == (5, 6)
    assert paging.pooled_rows([9, 4], 1) == (4, 4)


@pytest.mark.parametrize("page_size", [1, 2, 4, 16])
def test_single_token_suffix_rows_equal_the_new_page_rule(page_size):
    """paged_suffix_rows (page of token m) with one token == paged_rows (last_page_len == 1 rule)."""
    rng = np.random.default_rng(60 + page_size)
    lengths = list(range(2, 3 * page_size + 4)) + list(rng.integers(2, 300, 40))
    ids, indptr, last_len = _table(lengths, page_size, rng)
    for b in range(len(lengths)):
        r, writes = paging.paged_suffix_rows(ids, indptr, last_len, page_size, 1, b)
        assert (r, writes[0][1]) == paging.paged_rows(ids, indptr, last_len, b) and len(writes) == 1


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("page_size", [1, 3, 4])
def test_paged_suffix_equals_chain_of_single_token_calls(kind, page_size):
    """One call decoding several tokens per sequence == one single-token paged call per token,
    with the table grown by one token each time; every page written along the way matches."""
    rng = np.random.default_rng(70 + page_size)
    HK, HV, K, V = 1, 2, 4, 3
    prefix = [3, 1, 7, 4]                     # tokens before the suffix
    suffix = [5, 1, 6, 0]                     # tokens decoded by the call
    B = len(prefix)
    T = sum(suffix)
    cu = np.concatenate([[0], np.cumsum(suffix)])
    q, k = rng.standard_normal((T, HK, K)), rng.standard_normal((T, HK, K))
    v = rng.standard_normal((T, HV, V))
    gate = rng.standard_normal((T, HV, K)) if kind == "kda" else rng.standard_normal((T, HV))
    bl = rng.standard_normal((T, HV))
    A_log = rng.uniform(0, np.log(16), HV)
    dt = rng.uniform(-1, 1, (HV, K)) if kind == "kda" else rng.uniform(-1, 1, HV)
    # page ids for the final lengths; every page a sequence will ever use is distinct
    lengths = [p + s for p, s in zip(prefix, suffix)]
    ids, indptr, last_len = _table(lengths, page_size, rng)
    pool = {int(i): rng.standard_normal((HV, V, K)) * 0.1 for i in ids}
    start_pool = {r: x.copy() for r, x in pool.items()}
    multi = odec.kda_decode_paged_varlen if kind == "kda" else odec.gdn_decode_paged_varlen
    out_m, wr_m = multi(q, k, v, gate, bl, A_log, dt, cu, ids, indptr, last_len, page_size, start_pool)
    # chain: grow each sequence one token at a time with the single-token rule
    single = odec.kda_decode_paged if kind == "kda" else odec.gdn_decode_paged
    chain = {r: x.copy() for r, x in pool.items()}
    out_c = np.full_like(out_m, np.nan)
    for b in range(B):
        for i in range(suffix[b]):
            t = cu[b] + i
            n = prefix[b] + i + 1
            pages = -(-n // page_size)
            sub_ids = ids[indptr[b]:indptr[b] + pages]
            o, w = single(q[t:t + 1], k[t:t + 1], v[t:t + 1], gate[t:t + 1], bl[t:t + 1], A_log, dt, sub_ids,
                          np.array([0, pages]), np.array([n - page_size * (pages - 1)]), chain)
            out_c[t] = o[0]
            (row, tile), = w.items()
            chain[row] = tile
    np.testing.assert_allclose(out_m, out_c, rtol=1e-13, atol=1e-14)
    for row, tile in wr_m.items():
        np.testing.assert_allclose(tile, chain[row], rtol=1e-13, atol=1e-14)
    # rows the chain changed are exactly the rows the multi-token call wrote
    changed = {r for r in chain if not np.array_equal(chain[r], pool[r])}
    assert changed == set(wr_m)

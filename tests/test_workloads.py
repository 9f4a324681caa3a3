"""CPU checks of the seeded generators: the preconditions the decode call relies on hold."""
import numpy as np
import pytest
import torch

from recurrent_state_decode_amd import workloads as wl


def test_pooled_slots_distinct_and_in_range():
    for w in (wl.pooled_gdn_b64(), wl.pooled_kda_varlen_b128(), wl.fp8_qdq_gdn_b512(), wl.tiny_gdn()):
        si = w.inputs["state_indices"].numpy()
        assert len(set(si.tolist())) == len(si) == w.B
        assert si.min() >= 0 and si.max() < w.num_rows


def test_kda_lengths_and_cu_seqlens():
    w = wl.pooled_kda_varlen_b128()
    cu = w.inputs["cu_seqlens"].numpy()
    lens = np.diff(cu)
    assert cu[0] == 0 and cu[-1] == w.T and lens.min() >= 1 and lens.max() <= 8
    assert w.inputs["raw_gate"].shape == (w.T, 32, 128) and w.inputs["dt_bias"].shape == (32, 128)


def test_seeded_draws_are_reproducible():
    a, b = wl.pooled_gdn_b64(), wl.pooled_gdn_b64()
    for kk in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "state_indices"):
        assert torch.equal(a.inputs[kk], b.inputs[kk])
    assert torch.equal(wl.make_pool(wl.tiny_gdn(), "cpu"), torch.zeros(1, 1, 16, 16))


def _check_paged_invariants(w, page_size):
    ind = w.inputs["page_indices"].numpy()
    ptr = w.inputs["page_indptr"].numpy()
    lpl = w.inputs["last_page_len"].numpy()
    L = w.inputs["prefix_lengths"].numpy()
    B = w.B
    n = L + 1
    P = np.diff(ptr)
    assert np.array_equal(P, -(-n // page_size))
    assert np.array_equal(lpl, n - page_size * (P - 1))
    assert ind.min() >= 0 and ind.max() < w.num_rows
    assert len(np.unique(ind)) == w.num_rows                  # compact ids
    last = ind[ptr[1:] - 1]
    assert len(np.unique(last)) == B                          # unique write pages
    reads = np.where(lpl == 1, ind[np.maximum(ptr[1:] - 2, 0)], last)
    assert np.all(P[lpl == 1] >= 2)                           # a new page has a previous page
    nonlast = set(np.concatenate([ind[ptr[b]:ptr[b + 1] - 1] for b in range(B)]).tolist())
    assert not (set(last.tolist()) & nonlast)                 # shared pages are never last pages
    for b in range(B):                                        # no write page is read by another sequence
        others = np.delete(reads, b)
        assert last[b] not in set(others.tolist())
    return ind, ptr, lpl, reads


def test_paged_table_invariants_small():
    for seed in range(5):
        w = wl.gdn_paged(40, 2, 4, 16, 16, max_prefix=100, page_size=4, share_frac=0.2, seed=seed)
        _check_paged_invariants(w, 4)


def test_paged_b256_table_shape_and_sharing():
    w = wl.paged_gdn_b256()
    ind, ptr, lpl, reads = _check_paged_invariants(w, 16)
    full_slots = int(np.sum(np.diff(ptr) - 1))
    assert 14000 < w.num_rows < 17500
    # about 10% of the full-page slots alias another sequence's page
    shared = full_slots + w.B - w.num_rows
    assert 0.08 * full_slots <= shared <= 0.12 * full_slots
    # about 1/16 of the decoded tokens open a new page; some of those read a shared page
    frac = np.mean(lpl == 1)
    assert 0.01 < frac < 0.15
    counts = np.bincount(ind, minlength=w.num_rows)
    assert np.sum((lpl == 1) & (counts[reads] > 1)) >= 1
    assert w.pool_shape() == (w.num_rows, 32, 128, 128)


def test_paged_varlen_tables_never_share_pages_that_a_suffix_writes():
    from oracle import paging as opaging
    for seed in range(4):
        suffix = np.random.default_rng(seed).integers(0, 10, 30)
        w = wl.paged("gdn", 30, 2, 4, 16, 16, max_prefix=60, page_size=4, share_frac=0.3,
                     suffix_lengths=suffix, seed=seed)
        ind, ptr, lpl = (w.inputs[k].numpy() for k in ("page_indices", "page_indptr", "last_page_len"))
        cu = w.inputs["cu_seqlens"].numpy()
        counts = np.bincount(ind, minlength=w.num_rows)
        writes, reads = [], []
        for b in range(w.B):
            nb = int(cu[b + 1] - cu[b])
            if nb == 0:
                continue
            r, wr = opaging.paged_suffix_rows(ind, ptr, lpl, 4, nb, b)
            reads.append(r)
            writes.extend(row for _, row in wr)
        assert len(writes) == len(set(writes))              # each written page once
        assert all(counts[r] == 1 for r in writes)           # written pages are never shared
        assert not (set(writes) & set(reads)) or all(      # a sequence may update its own read page
            reads.count(r) == 1 for r in set(writes) & set(reads))
        assert w.T == int(suffix.sum()) and w.inputs["q"].shape[0] == w.T


def test_paged_kda_workload_shapes():
    w = wl.paged_kda_b256()
    assert w.kind == "kda_paged" and w.inputs["raw_gate"].shape == (256, 32, 128)
    assert w.inputs["dt_bias"].shape == (32, 128) and w.inputs["a_log"].shape == (32,)
    _check_paged_invariants(w, 16)

"""The host-side precondition checks of the C ABI (gdn_check_pooled / _paged / _paged_varlen).

The kernels trust their index arrays (flashinfer.gdn_paged,
gated_delta_rule_decode_paged, slots; max.nn.state_space.kda_decode, Raises);
these calls, and every call of the GDN_DEVICE_CHECKS build, refuse a call
whose indices break a precondition.  Pinned three ways, all on the CPU:
every seeded workload passes; each precondition, broken on its own, is
refused with a message naming it; and on randomly corrupted small tables the
verdict equals a brute-force predicate built on the oracle's row resolution
(oracle/paging.py).
"""
import numpy as np
import pytest
import torch

import recurrent_state_decode_amd as rsd
from oracle import paging as opaging
from recurrent_state_decode_amd import workloads as wl


def _refused(fn, *args, match, **kw):
    with pytest.raises(rsd.GdnError) as e:
        fn(*args, **kw)
    assert e.value.name == "GDN_ERR_PRECONDITION", e.value
    assert match in e.value.message, e.value.message


def _table(w):
    i = w.inputs
    return i["page_indices"].clone(), i["page_indptr"].clone(), i["last_page_len"].clone()


# ---------------------------------------------------------------- seeded workloads pass

def test_named_workloads_pass():
    for w in (wl.tiny_gdn(), wl.pooled_gdn_b64(), wl.pooled_kda_varlen_b128(), wl.fp8_qdq_gdn_b512(),
              wl.int8h32_gdn_b512()):
        rsd.check_pooled(w.inputs["state_indices"], w.num_rows, w.inputs.get("cu_seqlens"), T=w.T)
    for w in (wl.paged_gdn_b256(), wl.paged_gdn_b256(index_dtype=torch.int32), wl.paged_kda_b256()):
        rsd.check_paged(*_table(w), w.num_rows, page_size=16)
    for w in (wl.paged_gdn_varlen_b256_t4(), wl.paged_gdn_prefill_b16_t1024(), wl.paged_kda_prefill_b16_t1024()):
        rsd.check_paged_varlen(w.inputs["cu_seqlens"], *_table(w), w.options["page_size"], w.num_rows, T=w.T)


# ---------------------------------------------------------------- each precondition on its own

def test_pooled_violations():
    si = torch.tensor([4, 0, 2, 7], dtype=torch.int32)
    cu = torch.tensor([0, 1, 3, 3, 5], dtype=torch.int32)
    rsd.check_pooled(si, 8, cu)
    _refused(rsd.check_pooled, torch.tensor([4, 0, 2, 4], dtype=torch.int32), 8, cu, match="share slot 4")
    _refused(rsd.check_pooled, torch.tensor([4, 0, 2, 8], dtype=torch.int32), 8, cu, match="outside [0, 8)")
    _refused(rsd.check_pooled, torch.tensor([-1, 0, 2, 7], dtype=torch.int32), 8, cu, match="state_indices[0]")
    # an empty suffix reads and writes nothing: its slot is never used
    rsd.check_pooled(torch.tensor([4, 0, 0, 7], dtype=torch.int32), 8, cu)
    rsd.check_pooled(torch.tensor([4, 0, 99, 7], dtype=torch.int32), 8, cu)
    _refused(rsd.check_pooled, si, 8, torch.tensor([0, 1, 3, 2, 5], dtype=torch.int32), match="decreases at sequence 2")
    _refused(rsd.check_pooled, si, 8, torch.tensor([1, 1, 3, 3, 5], dtype=torch.int32), match="cu_seqlens[0]")
    _refused(rsd.check_pooled, si, 8, cu, T=6, match="not T = 6")
    _refused(rsd.check_pooled, si, 8, None, T=5, match="must equal B")


def _small_paged(seed=3, B=12, page_size=4, **kw):
    return wl.gdn_paged(B, 1, 2, 16, 16, max_prefix=30, page_size=page_size, share_frac=0.3, seed=seed, **kw)


def _seq_with(lpl, pred):
    return next(b for b in range(len(lpl)) if pred(b))


def test_paged_violations():
    w = _small_paged()
    pi, ptr, lpl = _table(w)
    rows = w.num_rows
    rsd.check_paged(pi, ptr, lpl, rows, page_size=4)
    B = w.B
    # two sequences write one page
    x = pi.clone()
    x[ptr[2] - 1] = x[ptr[1] - 1]
    _refused(rsd.check_paged, x, ptr, lpl, rows, match="write page")
    # a sequence writes the page another reads: point b's last page at the page a new-page sequence reads from
    b_new = _seq_with(lpl, lambda b: int(lpl[b]) == 1)
    read_page = int(pi[ptr[b_new + 1] - 2])
    b_other = _seq_with(lpl, lambda b: b != b_new and int(pi[ptr[b + 1] - 1]) != read_page
                        and read_page not in pi[ptr[b]:ptr[b + 1]].tolist())
    x = pi.clone()
    x[ptr[b_other + 1] - 1] = read_page
    _refused(rsd.check_paged, x, ptr, lpl, rows, match=f"which sequence {b_new} reads")
    # a new page without a previous page
    b1 = _seq_with(lpl, lambda b: int(ptr[b + 1] - ptr[b]) == 1)
    y = lpl.clone()
    y[b1] = 1
    _refused(rsd.check_paged, pi, ptr, y, rows, match="no previous page")
    y = lpl.clone()
    y[0] = 0
    _refused(rsd.check_paged, pi, ptr, y, rows, match="below 1")
    y = lpl.clone()
    y[0] = 5
    _refused(rsd.check_paged, pi, ptr, y, rows, page_size=4, match="exceeds page_size 4")
    rsd.check_paged(pi, ptr, y, rows, page_size=0)        # page size unknown: only >= 1
    # a page id outside the pool
    x = pi.clone()
    x[ptr[1] - 1] = rows
    _refused(rsd.check_paged, x, ptr, lpl, rows, match=f"page {rows} is outside [0, {rows})")
    x = pi.clone()
    x[ptr[b_new + 1] - 2] = -3
    _refused(rsd.check_paged, x, ptr, lpl, rows, match="read page -3")
    # CSR structure
    p = ptr.clone()
    p[3] = p[2]
    _refused(rsd.check_paged, pi, p, lpl, rows, match="sequence 2 has no page")
    p = ptr.clone()
    p[B] = pi.numel() + 1
    _refused(rsd.check_paged, pi, p, lpl, rows, match="exceeds nnz")
    # slots must agree with the table
    slots = torch.tensor([opaging.paged_rows(pi, ptr, lpl, b) for b in range(B)], dtype=torch.int64)
    rsd.check_paged(pi, ptr, lpl, rows, slots=slots)
    bad = slots.clone()
    bad[b_new] = bad[b_new].flip(0)
    _refused(rsd.check_paged, pi, ptr, lpl, rows, slots=bad, match=f"slots of sequence {b_new}")


def test_paged_varlen_violations():
    suffix = np.array([3, 0, 9, 1, 6, 2])
    # sequence 4's prefix (8 tokens) ends on a page boundary: its suffix reads a page it never writes
    w = wl.paged("gdn", len(suffix), 1, 2, 16, 16, prefix_lengths=[5, 7, 12, 3, 8, 6], page_size=4, share_frac=0.3,
                 suffix_lengths=suffix, seed=5)
    pi, ptr, lpl = _table(w)
    cu = w.inputs["cu_seqlens"]
    rows = w.num_rows
    rsd.check_paged_varlen(cu, pi, ptr, lpl, 4, rows)
    # a suffix with no earlier token: the whole sequence is the suffix
    n2 = int((ptr[3] - ptr[2] - 1) * 4 + lpl[2])
    c = cu.clone()
    c[3:] += n2 - 9
    _refused(rsd.check_paged_varlen, c, pi, ptr, lpl, 4, rows, match="sequence 2: its")
    # a page that sequence 2 fills mid-suffix also belongs to sequence 0
    _, wr = opaging.paged_suffix_rows(pi, ptr, lpl, 4, 9, 2)
    first_written = wr[0][1]
    x = pi.clone()
    x[ptr[1] - 1] = first_written
    _refused(rsd.check_paged_varlen, cu, x, ptr, lpl, 4, rows, match="write page")
    # a sequence reads a page that sequence 2 writes (one whose read page is not also its own write page)
    def read_only(b):
        r, wr_b = opaging.paged_suffix_rows(pi, ptr, lpl, 4, int(suffix[b]), b)
        return r not in {row for _, row in wr_b}
    b_r = 4
    assert read_only(b_r)
    pos_last = int((ptr[b_r + 1] - ptr[b_r] - 1) * 4 + lpl[b_r])
    x = pi.clone()
    x[ptr[b_r] + (pos_last - int(suffix[b_r]) - 1) // 4] = first_written
    _refused(rsd.check_paged_varlen, cu, x, ptr, lpl, 4, rows, match=f"which sequence {b_r} reads")
    y = lpl.clone()
    y[0] = 5
    _refused(rsd.check_paged_varlen, cu, pi, ptr, y, 4, rows, match="exceeds page_size 4")
    # the empty suffix (sequence 1) touches nothing, so its pages may be anything in the table
    x = pi.clone()
    x[ptr[1]:ptr[2]] = rows + 5
    rsd.check_paged_varlen(cu, x, ptr, lpl, 4, rows)


# ---------------------------------------------------------------- random corruption vs brute force

def _brute_table_ok(pi, ptr, lpl, page_size):
    B = len(lpl)
    if ptr[0] < 0 or ptr[B] > len(pi):
        return False
    for b in range(B):
        if ptr[b + 1] <= ptr[b] or lpl[b] < 1 or (page_size > 0 and lpl[b] > page_size):
            return False
    return True


def _brute_paged_ok(pi, ptr, lpl, rows, page_size):
    if not _brute_table_ok(pi, ptr, lpl, page_size):
        return False
    B = len(lpl)
    rw = []
    for b in range(B):
        if lpl[b] == 1 and ptr[b + 1] - ptr[b] < 2:
            return False
        r, w = opaging.paged_rows(pi, ptr, lpl, b)
        if not (0 <= r < rows and 0 <= w < rows):
            return False
        rw.append((r, w))
    for b in range(B):
        for c in range(B):
            if b != c and (rw[b][1] == rw[c][1] or rw[b][1] == rw[c][0]):
                return False
    return True


def _brute_varlen_ok(cu, pi, ptr, lpl, rows, page_size):
    if not _brute_table_ok(pi, ptr, lpl, page_size):
        return False
    B = len(lpl)
    touched = {}
    for b in range(B):
        n = cu[b + 1] - cu[b]
        if n == 0:
            continue
        try:
            r, wr = opaging.paged_suffix_rows(pi, ptr, lpl, page_size, n, b)
        except ValueError:
            return False
        ws = {row for _, row in wr}
        if not all(0 <= x < rows for x in ws | {r}):
            return False
        touched[b] = (r, ws)
    for b, (_, ws) in touched.items():
        for c, (rc, wc) in touched.items():
            if b != c and ws & (wc | {rc}):
                return False
    return True


def _verdict(fn, *args, **kw):
    try:
        fn(*args, **kw)
        return True
    except rsd.GdnError as e:
        assert e.name == "GDN_ERR_PRECONDITION", e
        return False


def _corrupt(rng, pi, ptr, lpl, rows, page_size):
    pi, ptr, lpl = pi.copy(), ptr.copy(), lpl.copy()
    kind = rng.integers(0, 4)
    if kind == 0:
        pi[rng.integers(0, len(pi))] = rng.integers(-1, rows + 1)
    elif kind == 1:
        pi[rng.integers(0, len(pi))] = pi[rng.integers(0, len(pi))]
    elif kind == 2:
        lpl[rng.integers(0, len(lpl))] = rng.integers(0, page_size + 2)
    else:
        b = rng.integers(1, len(ptr))
        ptr[b] = max(ptr[b] + rng.choice([-1, 1]), 0)
    return pi, ptr, lpl


def test_random_corruption_matches_brute_force_paged():
    rng = np.random.default_rng(11)
    outcomes = set()
    for trial in range(300):
        w = _small_paged(seed=int(rng.integers(0, 1 << 30)), B=int(rng.integers(2, 9)))
        pi, ptr, lpl = (t.numpy() for t in _table(w))
        if trial % 4:
            pi, ptr, lpl = _corrupt(rng, pi, ptr, lpl, w.num_rows, 4)
        want = _brute_paged_ok(pi, ptr, lpl, w.num_rows, 4)
        got = _verdict(rsd.check_paged, torch.from_numpy(pi), torch.from_numpy(ptr), torch.from_numpy(lpl),
                       w.num_rows, page_size=4)
        assert got == want, (trial, pi, ptr, lpl)
        outcomes.add(got)
    assert outcomes == {True, False}


def test_random_corruption_matches_brute_force_varlen():
    rng = np.random.default_rng(12)
    outcomes = set()
    for trial in range(300):
        B = int(rng.integers(2, 7))
        suffix = rng.integers(0, 10, B)
        w = wl.paged("gdn", B, 1, 2, 16, 16, max_prefix=20, page_size=4, share_frac=0.3, suffix_lengths=suffix,
                     seed=int(rng.integers(0, 1 << 30)))
        pi, ptr, lpl = (t.numpy() for t in _table(w))
        cu = w.inputs["cu_seqlens"].numpy()
        if trial % 4:
            pi, ptr, lpl = _corrupt(rng, pi, ptr, lpl, w.num_rows, 4)
        want = _brute_varlen_ok(cu, pi, ptr, lpl, w.num_rows, 4)
        got = _verdict(rsd.check_paged_varlen, torch.from_numpy(cu), torch.from_numpy(pi), torch.from_numpy(ptr),
                       torch.from_numpy(lpl), 4, w.num_rows)
        assert got == want, (trial, cu, pi, ptr, lpl)
        outcomes.add(got)
    assert outcomes == {True, False}


def test_random_pooled_matches_brute_force():
    rng = np.random.default_rng(13)
    for trial in range(300):
        B = int(rng.integers(1, 8))
        rows = int(rng.integers(1, 10))
        si = rng.integers(-1, rows + 1, B).astype(np.int32)
        lens = rng.integers(0, 3, B)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        used = [int(si[b]) for b in range(B) if lens[b] > 0]
        want = all(0 <= s < rows for s in used) and len(set(used)) == len(used)
        got = _verdict(rsd.check_pooled, torch.from_numpy(si), rows, torch.from_numpy(cu))
        assert got == want, (si, cu, rows)


def test_check_argument_errors():
    with pytest.raises(rsd.GdnError) as e:
        rsd.check_pooled(torch.zeros(0, dtype=torch.int32), 4)
    assert e.value.name == "GDN_ERR_INVALID"
    w = _small_paged()
    with pytest.raises(rsd.GdnError) as e:
        rsd.check_paged(*_table(w), 0)
    assert e.value.name == "GDN_ERR_INVALID"
    with pytest.raises(TypeError):
        rsd.check_pooled(torch.zeros(3, dtype=torch.int64), 4)

"""The GDN_DEVICE_CHECKS build (libgdn_decode_checked.so) on the GPU.

On valid calls it gives bit for bit the release library's outputs and pool;
a call whose index arrays break a precondition is refused with
GDN_ERR_PRECONDITION before anything is launched, so the pool and ``out``
keep every byte.  The refused calls below break only preconditions whose
indices all stay inside their arrays (shared slots and pages, a page one
sequence writes and another reads, slots that disagree with the table), so
that no access could leave its buffer even if a check were missing;
out-of-range indices are pinned on the CPU (test_preconditions.py).
"""
import numpy as np
import pytest
import torch

import recurrent_state_decode_amd as rsd
from oracle import paging as opaging
from recurrent_state_decode_amd import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu


def _cases():
    return [
        wl.gdn_pooled(6, 2, 4, 128, 128, lengths=[1, 3, 0, 9, 2, 1], num_slots=8, seed=61),
        wl.kda_pooled(4, 2, 2, 128, 128, lengths=[2, 1, 0, 4], num_slots=5, state_layout="V_FIRST", seed=62),
        wl.gdn_paged(24, 2, 4, 128, 128, max_prefix=40, page_size=4, share_frac=0.3, seed=63),
        wl.paged("kda", 16, 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3, seed=64,
                 suffix_lengths=np.array([0, 1, 2, 3, 4, 5, 8, 9, 7, 1, 4, 0, 6, 2, 9, 3])),
        wl.paged("gdn", 3, 2, 4, 128, 128, max_prefix=40, page_size=16, suffix_lengths=[20, 1, 37], seed=65,
                 chunked=True),
    ]


@pytest.mark.parametrize("case", range(5))
def test_checked_build_matches_release(case):
    w = _cases()[case]
    d = P.device_inputs(w)
    pool_a = wl.make_pool(w, "cuda")
    pool_b = pool_a.clone()
    out_a = P.gpu_call(w, pool_a, d)
    with rsd.checked_library() as lib:
        assert lib.gdn_checked_build() == 1
        out_b = P.gpu_call(w, pool_b, d)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(pool_a, pool_b)


def _refused_untouched(w, d, match, **over):
    pool = wl.make_pool(w, "cuda")
    before = pool.clone()
    out = torch.full((w.T, w.HV, w.V), float("nan"), dtype=w.out_dtype, device="cuda")
    with rsd.checked_library() as lib:
        assert lib.gdn_checked_build() == 1
        with pytest.raises(rsd.GdnError) as e:
            P.gpu_call(w, pool, d, out=out, **over)
    torch.cuda.synchronize()
    assert e.value.name == "GDN_ERR_PRECONDITION" and match in e.value.message, e.value
    assert torch.equal(pool, before) and bool(torch.isnan(out.float()).all())


def test_checked_build_refuses_shared_slot():
    w = _cases()[0]
    d = P.device_inputs(w)
    d["state_indices"][3] = d["state_indices"][1]          # both suffixes are non-empty
    _refused_untouched(w, d, "share slot")


def test_checked_build_refuses_shared_write_page():
    w = _cases()[2]
    d = P.device_inputs(w)
    ptr = w.inputs["page_indptr"]
    d["page_indices"][int(ptr[2]) - 1] = d["page_indices"][int(ptr[1]) - 1]
    _refused_untouched(w, d, "write page")


def test_checked_build_refuses_slots_that_disagree_with_the_table():
    w = _cases()[2]
    d = P.device_inputs(w)
    pi, ptr, lpl = (w.inputs[k] for k in ("page_indices", "page_indptr", "last_page_len"))
    slots = torch.tensor([opaging.paged_rows(pi, ptr, lpl, b) for b in range(w.B)], dtype=torch.int64)
    b_new = int(np.flatnonzero(lpl.numpy() == 1)[0])
    slots[b_new] = slots[b_new].flip(0)                      # in range, but read and write swapped
    _refused_untouched(w, d, f"slots of sequence {b_new}", slots=slots.cuda())


@pytest.mark.parametrize("case", [3, 4])
def test_checked_build_refuses_a_page_written_by_two_suffixes(case):
    w = _cases()[case]
    d = P.device_inputs(w)
    cu = w.inputs["cu_seqlens"].numpy()
    ptr = w.inputs["page_indptr"].numpy()
    b1, b2 = [b for b in range(w.B) if cu[b + 1] > cu[b]][:2]
    d["page_indices"][int(ptr[b2 + 1]) - 1] = d["page_indices"][int(ptr[b1 + 1]) - 1]
    _refused_untouched(w, d, "write page")


@pytest.mark.parametrize("qdq", ["fp8_e4m3_tile", "int8_hadamard32"])
def test_checked_build_matches_release_on_packed_pools(qdq):
    layout = "V_FIRST" if qdq == "fp8_e4m3_tile" else "K_FIRST"
    suffix = np.array([0, 1, 2, 3, 4, 5, 8, 9, 7, 1, 4, 0])
    w = wl.paged("gdn", len(suffix), 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3, seed=66,
                 suffix_lengths=suffix, state_layout=layout, qdq=qdq, block_v=64)
    d = P.device_inputs(w)
    pool_a = P.make_packed_pool(w, "cuda")
    pool_b = pool_a.clone()
    out_a = P.gpu_call(w, pool_a, d)
    with rsd.checked_library() as lib:
        assert lib.gdn_checked_build() == 1
        out_b = P.gpu_call(w, pool_b, d)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(pool_a, pool_b)

"""GPU check of the measurement helper gdn_stream_rows (the decode step's state traffic without its
arithmetic): each pair's write row receives its read row bit for bit, and no other row changes."""
import pytest
import torch

import recurrent_state_decode_amd as rsd
from recurrent_state_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("in_place", [True, False])
def test_stream_rows_copies_read_rows_to_write_rows(in_place):
    g = torch.Generator(device="cuda").manual_seed(5)
    src = torch.randn((40, 4, 16, 128), generator=g, device="cuda")
    dst = src if in_place else torch.randn((40, 4, 16, 128), generator=g, device="cuda")
    # rows 0..9 read; writes go to 10..19 (copy to a new row) or back to the read row
    pairs = [(r, r if r % 3 == 0 else 10 + r) for r in range(10)]
    slots = torch.tensor(pairs, dtype=torch.int64, device="cuda")
    src_before, dst_before = src.clone(), dst.clone()
    rsd.stream_rows(src, dst, slots)
    torch.cuda.synchronize()
    expect = dst_before.clone()
    for r, w in pairs:
        expect[w] = src_before[r]
    assert torch.equal(dst.view(torch.int32), expect.view(torch.int32))
    if not in_place:
        assert torch.equal(src.view(torch.int32), src_before.view(torch.int32))


def test_stream_rows_on_the_paged_table():
    w = wl.gdn_paged(48, 2, 4, 128, 128, max_prefix=40, page_size=4, share_frac=0.3, seed=35)
    d = wl.device_inputs(w)
    pool = wl.make_pool(w, "cuda")
    slots = rsd.gdn_paged_decode_slots(d["page_indices"], d["page_indptr"], d["last_page_len"])
    before = pool.clone()
    rsd.stream_rows(pool, pool, slots)
    torch.cuda.synchronize()
    s = slots.cpu().tolist()
    written = {wr for _, wr in s}
    for r, wr in s:
        assert torch.equal(pool[wr].view(torch.int32), before[r].view(torch.int32))
    for row in range(pool.shape[0]):
        if row not in written:
            assert torch.equal(pool[row].view(torch.int32), before[row].view(torch.int32))

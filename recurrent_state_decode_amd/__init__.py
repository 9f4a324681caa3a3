"""MI355X-native gated delta-rule (GDN / KDA) recurrent-state decode.

The compute lives in ``libgdn_decode.so`` (hand-written HIP kernels for
gfx950 behind the C ABI of ``include/gdn_decode.h``); this package is its
thin Python binding plus the seeded workload generators used by the tests
and the bench.  PyTorch only provides device memory and streams.
"""
from ._binding import (  # noqa: F401
    CHECKED_LIB_PATH,
    GdnError,
    LIB_PATH,
    check_paged,
    check_paged_varlen,
    check_pooled,
    checked_library,
    fp8_tile_bytes,
    gdn_decode_paged,
    gdn_decode_paged_varlen,
    gdn_decode_pooled,
    gdn_paged_decode_slots,
    gdn_prefill_paged,
    kda_decode_paged,
    kda_decode_paged_varlen,
    kda_decode_pooled,
    kda_prefill_paged,
    load_library,
    packed_tile_bytes,
    stream_rows,
    supported_head_dims,
    workgroup_order,
)

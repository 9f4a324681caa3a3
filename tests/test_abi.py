"""CPU checks of the C ABI: the library loads, exports every declared symbol, and refuses bad
arguments on the host with the documented status codes.  Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest
import torch

import recurrent_state_decode_amd as rsd
from recurrent_state_decode_amd import _binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]

# The error-path calls below pass fake (never dereferenced) pointers.  They are
# refused on the host before any launch; still, keep them off a machine with a GPU.
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer ABI checks run only without a GPU")


def declared_functions():
    names = []
    for path in HEADERS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?(?:int64_t|int|void|char)\s*\*?\s*(\w+)\s*\(", text, flags=re.M):
            names.append(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"gdn_decode_pooled", "gdn_decode_paged", "kda_decode_pooled", "gdn_status_string",
            "gdn_check_paged", "gdn_checked_build", "gdn_packed_tile_bytes", "gdn_fp8_tile_bytes"} <= set(names)
    for path, checked in ((rsd.LIB_PATH, 0), (rsd.CHECKED_LIB_PATH, 1)):
        lib = bnd.load_library(path)
        for n in names:
            assert hasattr(lib, n), (path, n)
        assert lib.gdn_checked_build() == checked, path


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        bnd.load_library(str(tmp_path / "absent.so"))


def test_options_defaults_and_status_strings():
    o = bnd._options()
    assert (o.scale, o.use_qk_l2norm, o.io_dtype, o.out_dtype, o.state_layout) == (0.0, 1, 1, 1, 0)
    assert (o.beta_mode, o.gate_mode, o.index_dtype, o.qdq, o.block_v, o.quantize_initial, o.readout) == \
        (0, 0, bnd.GDN_I32, 0, 64, 0, 0)
    lib = rsd.load_library()
    assert [lib.gdn_status_string(i).decode() for i in range(6)] == \
        ["GDN_OK", "GDN_ERR_INVALID", "GDN_ERR_SHAPE", "GDN_ERR_UNSUPPORTED", "GDN_ERR_HIP", "GDN_ERR_PRECONDITION"]
    assert lib.gdn_status_string(99).decode() == "unknown status"
    assert (128, 64) in rsd.supported_head_dims() and (16, 16) in rsd.supported_head_dims()


FAKE = ctypes.c_void_p(0x1000)


def _pooled(lib, B=2, T=2, HK=1, HV=2, K=128, V=128, cu=FAKE, nulls=(), **opt):
    o = bnd._options(**opt)
    ptrs = [None if i in nulls else FAKE for i in range(11)]
    ptrs[7] = cu
    return lib.gdn_decode_pooled(*ptrs, B, T, HK, HV, K, V, 4, ctypes.byref(o), None)


@no_gpu
def test_pooled_argument_errors():
    lib = rsd.load_library()
    assert _pooled(lib, nulls=(0,)) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, nulls=(9,)) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, HK=3, HV=4) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, B=0) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, K=96) == bnd.GDN_ERR_UNSUPPORTED
    assert _pooled(lib, V=96) == bnd.GDN_ERR_UNSUPPORTED
    assert _pooled(lib, cu=None, B=3, T=2) == bnd.GDN_ERR_SHAPE
    assert _pooled(lib, gate_mode=1) == bnd.GDN_ERR_UNSUPPORTED
    assert "SAFE" in lib.gdn_last_error().decode()
    assert _pooled(lib, io_dtype=7) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, state_layout=2) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, qdq=1, block_v=48) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, qdq=1, block_v=128) == bnd.GDN_ERR_UNSUPPORTED
    assert _pooled(lib, qdq=3) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, qdq=2, block_v=48) == bnd.GDN_ERR_INVALID       # not a multiple of 32
    assert _pooled(lib, qdq=2, block_v=96) == bnd.GDN_ERR_INVALID       # does not divide V
    assert _pooled(lib, qdq=2, K=16, V=32, block_v=32) == bnd.GDN_ERR_UNSUPPORTED
    assert "K=128" in lib.gdn_last_error().decode()
    assert _pooled(lib, qdq=2, block_v=128, T=0) == bnd.GDN_OK          # any multiple of 32 dividing V
    assert _pooled(lib, scale=float("inf")) == bnd.GDN_ERR_INVALID
    # an empty call (T = 0 with cu_seqlens) launches nothing and succeeds
    assert _pooled(lib, T=0) == bnd.GDN_OK
    # a grid beyond 2^31 - 1 workgroups is refused before any launch (B HV V / VB units)
    big = 1 << 26
    assert _pooled(lib, cu=None, B=big, T=big, HK=16, HV=32, state_layout=1) == bnd.GDN_ERR_UNSUPPORTED
    assert "too large" in lib.gdn_last_error().decode()


@no_gpu
def test_packed_storage_argument_errors():
    lib = rsd.load_library()
    assert bnd._options().state_storage == bnd.GDN_STORAGE_F32
    assert rsd.packed_tile_bytes(128, 128) == 128 * 128 + 4 * 128 * 4 == 18432
    assert lib.gdn_packed_tile_bytes(128, 48) == -1
    with pytest.raises(ValueError):
        rsd.packed_tile_bytes(128, 48)
    assert _pooled(lib, state_storage=1) == bnd.GDN_ERR_INVALID                 # packed needs the codec
    assert "INT8_HADAMARD32" in lib.gdn_last_error().decode()
    assert _pooled(lib, state_storage=1, qdq=1) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, state_storage=1, qdq=2, state_layout=1) == bnd.GDN_ERR_UNSUPPORTED
    assert _pooled(lib, state_storage=2, qdq=2) == bnd.GDN_ERR_INVALID           # fp8 storage needs fp8 tiles
    assert "FP8_E4M3_TILE" in lib.gdn_last_error().decode()
    assert _pooled(lib, state_storage=3, qdq=1) == bnd.GDN_ERR_INVALID
    assert _pooled(lib, state_storage=1, qdq=2, T=0) == bnd.GDN_OK               # accepted (nothing to launch)
    assert _pooled(lib, state_storage=2, qdq=1, T=0) == bnd.GDN_OK
    assert _pooled(lib, state_storage=2, qdq=1, state_layout=1, T=0) == bnd.GDN_OK   # either layout


@no_gpu
def test_fp8_tile_bytes():
    from oracle import e4m3
    lib = rsd.load_library()
    assert rsd.fp8_tile_bytes(128, 128) == 128 * 128 + 128 == 16512              # two scales, padded to a line
    for K, V, bv in ((128, 128, 64), (128, 256, 64), (16, 48, 16), (128, 64, 64), (16, 320, 16)):
        assert lib.gdn_fp8_tile_bytes(K, V, bv) == e4m3.fp8_tile_bytes(K, V, bv)
        assert lib.gdn_fp8_tile_bytes(K, V, bv) % 128 == 0
    assert lib.gdn_fp8_tile_bytes(128, 100, 64) == -1
    assert lib.gdn_fp8_tile_bytes(128, 128, 0) == -1
    with pytest.raises(ValueError):
        rsd.fp8_tile_bytes(128, 96)


@no_gpu
def test_paged_and_kda_argument_errors():
    lib = rsd.load_library()
    o = bnd._options(index_dtype=5)
    assert lib.gdn_decode_paged(*([FAKE] * 12), 2, 1, 2, 128, 128, 10, 4, ctypes.byref(o), None) == bnd.GDN_ERR_INVALID
    o = bnd._options(index_dtype=bnd.GDN_I64)
    assert lib.gdn_decode_paged(*([FAKE] * 12), 4, 1, 2, 128, 128, 10, 3, ctypes.byref(o), None) == bnd.GDN_ERR_SHAPE
    ptrs = [FAKE] * 11
    ptrs[7] = None                     # cu_seqlens is required for KDA
    o = bnd._options()
    assert lib.kda_decode_pooled(*ptrs, 2, 4, 1, 2, 128, 128, 4, ctypes.byref(o), None) == bnd.GDN_ERR_INVALID
    assert "cu_seqlens" in lib.gdn_last_error().decode()


@no_gpu
def test_new_paged_entry_points_argument_errors():
    lib = rsd.load_library()
    o = bnd._options(index_dtype=bnd.GDN_I64)
    # varlen paged: page_size must be positive, cu_seqlens is required
    args = [FAKE] * 11
    assert lib.gdn_decode_paged_varlen(*args, 0, FAKE, FAKE, 2, 4, 1, 2, 128, 128, 10, 4, ctypes.byref(o), None) \
        == bnd.GDN_ERR_INVALID
    args[7] = None
    assert lib.kda_decode_paged_varlen(*args, 16, FAKE, FAKE, 2, 4, 1, 2, 128, 128, 10, 4, ctypes.byref(o), None) \
        == bnd.GDN_ERR_INVALID
    # slots belong to single-token paged calls
    o2 = bnd._options(index_dtype=bnd.GDN_I64, slots=0x2000)
    assert lib.gdn_decode_paged_varlen(*([FAKE] * 11), 16, FAKE, FAKE, 2, 4, 1, 2, 128, 128, 10, 4,
                                       ctypes.byref(o2), None) == bnd.GDN_ERR_INVALID
    ptrs = [FAKE] * 11
    assert lib.gdn_decode_pooled(*ptrs, 2, 2, 1, 2, 128, 128, 4, ctypes.byref(o2), None) == bnd.GDN_ERR_INVALID
    assert "slots" in lib.gdn_last_error().decode()
    # the slot pass checks its index type and pointers
    assert lib.gdn_paged_decode_slots(FAKE, FAKE, FAKE, 4, 9, FAKE, None) == bnd.GDN_ERR_INVALID
    assert lib.gdn_paged_decode_slots(FAKE, FAKE, None, 4, bnd.GDN_I32, FAKE, None) == bnd.GDN_ERR_INVALID
    assert lib.kda_decode_paged(*([FAKE] * 12), 2, 2, 3, 128, 128, 10, 4, ctypes.byref(o), None) \
        == bnd.GDN_ERR_INVALID   # HV % HK != 0


@no_gpu
def test_prefill_argument_errors():
    lib = rsd.load_library()
    o = bnd._options(index_dtype=bnd.GDN_I64)
    args = [FAKE] * 11

    def call(page_size=16, B=2, T=4, HK=1, HV=2, K=128, V=128, opt=o, a=args):
        return lib.gdn_prefill_paged(*a, page_size, FAKE, FAKE, B, T, HK, HV, K, V, 10, 4, ctypes.byref(opt), None)

    assert call(T=0) == bnd.GDN_OK                        # nothing to do: no launch
    assert call(page_size=0) == bnd.GDN_ERR_INVALID
    assert call(page_size=8) == bnd.GDN_ERR_UNSUPPORTED   # chunks of 16 must end on page ends
    assert "multiple of 16" in lib.gdn_last_error().decode()
    assert call(K=16, V=16) == bnd.GDN_ERR_UNSUPPORTED
    assert call(V=64) == bnd.GDN_ERR_UNSUPPORTED
    assert call(opt=bnd._options(index_dtype=bnd.GDN_I64, qdq=1)) == bnd.GDN_ERR_UNSUPPORTED
    assert call(opt=bnd._options(index_dtype=bnd.GDN_I64, slots=0x2000)) == bnd.GDN_ERR_INVALID
    nul = list(args)
    nul[7] = None                                          # cu_seqlens is required
    assert call(a=nul) == bnd.GDN_ERR_INVALID
    assert call(HK=3, HV=4) == bnd.GDN_ERR_INVALID
    kcall = lambda **kw: lib.kda_prefill_paged(*args, kw.get("page_size", 16), FAKE, FAKE, 2, 4, 1, 2, 128,
                                               kw.get("V", 128), 10, 4, ctypes.byref(kw.get("opt", o)), None)
    assert kcall(page_size=24) == bnd.GDN_ERR_UNSUPPORTED
    assert kcall(V=64) == bnd.GDN_ERR_UNSUPPORTED
    assert kcall(opt=bnd._options(index_dtype=bnd.GDN_I64, gate_mode=1)) == bnd.GDN_ERR_UNSUPPORTED


@no_gpu
def test_stream_rows_argument_errors():
    lib = rsd.load_library()
    assert lib.gdn_stream_rows(None, FAKE, FAKE, 1, 512, None) == bnd.GDN_ERR_INVALID
    assert lib.gdn_stream_rows(FAKE, None, FAKE, 1, 512, None) == bnd.GDN_ERR_INVALID
    assert lib.gdn_stream_rows(FAKE, FAKE, None, 1, 512, None) == bnd.GDN_ERR_INVALID
    assert lib.gdn_stream_rows(FAKE, FAKE, FAKE, -1, 512, None) == bnd.GDN_ERR_INVALID
    assert lib.gdn_stream_rows(FAKE, FAKE, FAKE, 1, 0, None) == bnd.GDN_ERR_INVALID
    assert lib.gdn_stream_rows(FAKE, FAKE, FAKE, 1, 768, None) == bnd.GDN_ERR_INVALID
    assert "multiple of 512" in lib.gdn_last_error().decode()
    # no pairs: nothing to launch, no slots needed
    assert lib.gdn_stream_rows(FAKE, FAKE, None, 0, 512, None) == bnd.GDN_OK
    # more than 2^31 - 1 workgroups (one per 512 floats of every pair) is refused before any launch
    assert lib.gdn_stream_rows(FAKE, FAKE, FAKE, 1 << 30, 512 * 4, None) == bnd.GDN_ERR_UNSUPPORTED
    assert "too large" in lib.gdn_last_error().decode()

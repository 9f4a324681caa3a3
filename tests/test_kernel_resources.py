"""Resource use of the compiled kernels (CPU only: hipcc cross-compiles for gfx950).

No decode kernel may use scratch (private) memory: a per-token stack round trip is a memory
wait on every token (it cost 4-11 % when a select chain was compiled that way).  The four-wave
chunked prefill may spill a few registers outside its chunk loop but no more than 64 bytes; the
producer / consumer prefill at most 8 bytes, before its chunk loops.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from recurrent_state_decode_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kernel_sets():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "recurrent_state_decode_amd", "csrc", "gdn_decode.hip")
    with tempfile.TemporaryDirectory() as d:
        asm = os.path.join(d, "k.s")
        flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
        cmd = [hipcc, *flags, "-I", os.path.join(ROOT, "include"), "-I", os.path.dirname(src),
               "--cuda-device-only", "-S", "-o", asm, src]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=1200)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(asm).read()
    scratch = {m.group(1): int(m.group(2)) for m in
               re.finditer(r"\.set (_ZN3gdn\d+\w+?_kernel\w*?)\.private_seg_size, (\d+)", text)}
    return scratch


def test_decode_kernels_use_no_scratch(kernel_sets):
    dec = {k: v for k, v in kernel_sets.items() if "decode_kernel" in k}
    assert len(dec) > 100, "decode kernel instantiations not found"
    bad = {k: v for k, v in dec.items() if v}
    assert not bad, f"{len(bad)} decode kernels use scratch: {list(bad.items())[:3]}"


def test_prefill_spills_stay_small(kernel_sets):
    # the four-wave kernel: KDA (both I/O types and layouts) and GDN with 32-bit inputs
    pre = {k: v for k, v in kernel_sets.items() if "prefill_kernel" in k}
    assert len(pre) == 6, sorted(pre)
    assert max(pre.values()) <= 64, pre


def test_split_prefill_spills_at_most_a_register_pair(kernel_sets):
    """The producer / consumer GDN prefill (16-bit inputs, both layouts) spills at most a register or two, once,
    before its chunk loops (the K_FIRST build: one value of a producer's prologue).  More would put reloads in
    the loop, where each one waits for the later chunks' input loads in flight (the counter retires loads in
    order)."""
    ws = {k: v for k, v in kernel_sets.items() if "prefill_ws_kernel" in k}
    assert len(ws) == 2, sorted(ws)
    assert max(ws.values()) <= 8, ws

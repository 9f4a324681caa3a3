"""Resource use of the compiled kernels (CPU only: hipcc cross-compiles for gfx950).

No decode kernel may use scratch (private) memory: a per-token stack round trip is a memory
wait on every token (it cost 4-11 % when a select chain was compiled that way).  The four-wave
chunked prefill may spill a few registers outside its chunk loop but no more than 64 bytes; the
producer / consumer prefill at most 16 bytes, and no scratch access inside any of its loops.
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
    return scratch, text


def kernel_body(text, symbol):
    """The assembly lines of one kernel, from its label to its end marker."""
    start = text.index(f"\n{symbol}:")
    end = text.index(f".Lfunc_end", start)
    return text[start:end].split("\n")


def scratch_in_loops(lines):
    """Scratch (private memory) instructions inside a loop: between a block the compiler marks as a loop
    header and the last branch back to it."""
    found = []
    for i, line in enumerate(lines):
        m = re.match(r"^\.(LBB\d+_\d+):.*Loop Header", line)
        if not m:
            continue
        backs = [j for j, ln in enumerate(lines) if re.search(rf"s_(c)?branch\w* \.{m.group(1)}$", ln)]
        if backs and max(backs) > i:
            found += [ln.strip() for ln in lines[i:max(backs)] if "scratch_" in ln]
    return found


def test_decode_kernels_use_no_scratch(kernel_sets):
    kernel_sets = kernel_sets[0]
    dec = {k: v for k, v in kernel_sets.items() if "decode_kernel" in k}
    assert len(dec) > 100, "decode kernel instantiations not found"
    bad = {k: v for k, v in dec.items() if v}
    assert not bad, f"{len(bad)} decode kernels use scratch: {list(bad.items())[:3]}"


def test_prefill_spills_stay_small(kernel_sets):
    kernel_sets = kernel_sets[0]
    # the four-wave kernel: KDA (both I/O types and layouts) and GDN with 32-bit inputs
    pre = {k: v for k, v in kernel_sets.items() if "prefill_kernel" in k}
    assert len(pre) == 6, sorted(pre)
    assert max(pre.values()) <= 64, pre


def test_split_prefill_spills_stay_out_of_its_loops(kernel_sets):
    """The producer / consumer GDN prefill (16-bit inputs, both layouts) spills at most a few registers, and
    never inside a loop: those are values set before the chunk loops and read after them (the V_FIRST build's
    whole-line page stores take the extra registers).  A reload inside a chunk loop would wait for the later
    chunks' input loads in flight (the counter retires loads in order)."""
    sizes, text = kernel_sets
    ws = {k: v for k, v in sizes.items() if "prefill_ws_kernel" in k}
    assert len(ws) == 2, sorted(ws)
    assert max(ws.values()) <= 16, ws
    for sym in ws:
        bad = scratch_in_loops(kernel_body(text, sym))
        assert not bad, f"{sym}: scratch access inside a loop: {bad[:3]}"


def test_scratch_in_loops_finds_a_reload_in_a_loop():
    """The loop scan on a hand-made listing: a reload between a loop header and its back branch is found, one
    after the loop is not."""
    lines = [".LBB0_1:  ; =>This Loop Header: Depth=1", "  v_add_f32 v0, v1, v2",
             "  scratch_load_dword v3, off, off offset:4", "  s_cbranch_scc1 .LBB0_1",
             "  scratch_load_dword v4, off, off", "  s_endpgm"]
    assert scratch_in_loops(lines) == ["scratch_load_dword v3, off, off offset:4"]
    assert scratch_in_loops(lines[:2] + lines[3:]) == []

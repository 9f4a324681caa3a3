"""bench.py host logic (no GPU): byte counts, the profile source hash, the one-GPU contract, and that the
timed leg stays clear of the oracle."""
import os
import subprocess
import sys

import bench
from recurrent_state_decode_amd import workloads as wl
from tests import parity as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_algorithmic_bytes():
    state, io = bench.algorithmic_bytes(wl.paged_gdn_b256())
    assert state == 256 * 32 * 2 * 128 * 128 * 4
    assert state + io == 1_080_066_048


def test_packed_algorithmic_bytes():
    w = wl.paged_gdn_b256()
    w.options.update(qdq="fp8_e4m3_tile", block_v=64)
    assert bench.algorithmic_bytes(w, "fp8")[0] == 2 * 256 * 32 * (128 * 128 + 128)
    w.options.update(qdq="int8_hadamard32")
    assert bench.algorithmic_bytes(w, "i8h32")[0] == 2 * 256 * 32 * (128 * 128 + 4 * 128 * 4)


def test_paged_varlen_write_count_matches_the_page_rule():
    """bench.py counts written pages with its own arithmetic; the oracle's row resolution must agree."""
    for w in (wl.paged_gdn_varlen_b256_t4(), wl.paged_gdn_prefill_b16_t1024(),
              wl.paged("kda", 16, 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3, seed=64,
                       suffix_lengths=[0, 1, 2, 3, 4, 5, 8, 9, 7, 1, 4, 0, 6, 2, 9, 3])):
        reads, writes = P.rows_for(w)
        state, _ = bench.algorithmic_bytes(w)
        assert state == (len(reads) + len(writes)) * w.HV * w.K * w.V * 4


def test_source_hash_ignores_comments():
    code = "int f(int a) { return a + 1; }"
    assert bench._code_only(code) == bench._code_only("/* doc\n */ int f(int a) {  // note\n return a + 1; }")
    assert bench._code_only(code) != bench._code_only("int f(int a) { return a + 2; }")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stdout + r.stderr


def test_timed_leg_does_not_import_the_oracle():
    code = ("import sys, bench; from recurrent_state_decode_amd import workloads as wl; "
            "bench.algorithmic_bytes(wl.paged_gdn_varlen_b256_t4()); wl.run; wl.random_packed_pool; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.') or m.startswith('tests')]; "
            "assert not bad, bad")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]


def test_cpu_baseline_runs_on_every_core_of_the_share():
    """The oracle leg forks one worker per host core of this process's share and reports that count;
    the parent process itself never imports the oracle."""
    code = ("import sys, json, bench; from recurrent_state_decode_amd import workloads as wl; "
            "r = bench.cpu_baseline(wl.pooled_gdn_b64(), 1.0, 0.5); "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.') or m.startswith('tests')]; "
            "assert not bad, bad; print(json.dumps(r))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    import json
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["cores"] == bench.cpu_cores() and res["kind"] == "oracle" and res["value"] > 0
    assert res["single_core"]["cores"] == 1 and res["single_core"]["value"] > 0


def test_clock_sampler_reads_the_marked_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2103Mhz *\n2: 2400Mhz\n")
    c = bench.ClockSampler(period_s=0.001)
    c.paths = {"sclk": str(f)}
    c.samples = {"sclk": []}
    import time
    with c:
        time.sleep(0.02)
    s = c.summary()["sclk_mhz"]
    assert s["min"] == s["max"] == 2103 and s["samples"] >= 2

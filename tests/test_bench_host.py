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


def _counter_run(tmp_path, counters, workload="paged_gdn_prefill_b16_t1024_hv32_k128_ps16"):
    """A fake rocprofv3 counter run directory: two dispatches of the timed kernel and one of another."""
    import json
    d = tmp_path / "run"
    d.mkdir()
    kern = "gdn::prefill_kernel<2, 4, false, true, gdn::bf16_t>(gdn::PrefillParams)"
    with open(str(d) + ".json", "w") as f:
        f.write(json.dumps({"config": {"workload": workload},
                            "roofline": {"kernel": "gdn::prefill_kernel", "source_hash": "abc"}}) + "\n")
    with open(d / "c_kernel_trace.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        f.write(f'1,"{kern}",1000,901000\n2,"{kern}",2000000,2900000\n3,"other",0,10\n')
    with open(d / "c_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for did in (1, 2):
            for name, val in counters.items():
                f.write(f'{did},"{kern}",{name},{val}\n')
        f.write('3,"other",SQ_WAVES,5\n')
    return str(d)


def test_counter_summaries(tmp_path, monkeypatch):
    """The matrix-core summary: busy cycles per MFMA instruction and the busy fraction per SIMD from the
    clock counter (GRBM_GUI_ACTIVE sums the 8 XCDs); the activity summary keeps its own file name."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    cycles = 2_000_000                                   # per XCD
    run = _counter_run(tmp_path, {"SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cycles * bench.SIMDS, "SQ_INSTS_MFMA": 32000,
                                  "SQ_INSTS_VALU_MFMA_MOPS_F32": 1, "SQ_WAVES": 2048,
                                  "GRBM_GUI_ACTIVE": cycles * bench.XCDS})
    bench.summarize_counters(run, " --workload paged_gdn_prefill_b16_t1024")
    text = (tmp_path / "profiles" / "counters_mfma_paged_gdn_prefill_b16_t1024_hv32_k128_ps16.txt").read_text()
    assert "MFMA instructions per wave: 15.6" in text
    assert f"MFMA pipe busy cycles per MFMA instruction: {0.5 * cycles * bench.SIMDS / 32000:.2f}" in text
    assert "MFMA pipe busy fraction per SIMD: 0.500" in text
    assert "dispatches: 2; kernel duration median 900.0 us" in text
    assert "--pmc " + " ".join(bench.COUNTERS_MFMA) in text

    import shutil
    shutil.rmtree(run)
    run = _counter_run(tmp_path, {"VALUBusy": 40, "SQ_INSTS_VALU": 4096, "SQ_WAVES": 2048,
                                  "GRBM_GUI_ACTIVE": cycles * bench.XCDS})
    bench.summarize_counters(run, "")
    text = (tmp_path / "profiles" / "counters_paged_gdn_prefill_b16_t1024_hv32_k128_ps16.txt").read_text()
    assert "VALU instructions per wave: 2.0" in text and "--pmc " + " ".join(bench.COUNTERS) in text

"""Throughput of the gated delta-rule decode on one MI355X.

A step is one decode call over one batch of the workload (default: paged
GDN decode, B=256 sequences, HV=32, HK=16, K=V=128, page_size 16, prefixes
U{1..2048}, 10% shared full pages, V_FIRST fp32 pool of ~15k pages, bf16
I/O).  Inputs are resident in HBM before timing starts.  Before every step a
2 GiB buffer is written so that neither L2 nor the 256 MB MALL holds the
state rows the step touches (a decode step of one layer follows the steps of
all other layers in a model); each decode launch is bracketed by HIP events
on the stream it runs on, so the flush is not counted.

Prints one JSON line:
  value        decoded tokens per second (tokens per call / mean kernel time)
  roofline     the decode kernel against MI355X peak HBM bandwidth (8 TB/s):
               achieved = algorithmic bytes per launch / mean launch time;
               traffic = HBM bytes per launch measured with rocprofv3
               FETCH_SIZE/WRITE_SIZE (from profiles/, only if taken on the
               same kernel sources), else null
  cpu_baseline the CPU oracle timed on this host's cores (worker processes
               forked before any GPU call) on a bounded sample of the same
               workload, with a one-core figure beside it
  state_stream_reference
               the step's state bytes moved with no arithmetic over the same
               rows (gdn_stream_rows), timed like the decode
  gpu_clocks_during_timed_steps
               shader / memory clocks sampled while the timed steps run
"""
import argparse
import hashlib
import inspect
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "tokens/s & state-pool HBM GB/s (% peak), GDN decode B=256,HV=32,K=V=128"


def _code_only(text):
    """C/C++ source without its comments and blank space, so that a comment edit keeps the hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(chunked=False):
    """Hash of the code a kernel is built from (ties a profile to a kernel version): the decode
    kernel's header, the host launch code and the C header, comments left out; the chunked prefill
    adds its own header."""
    h = hashlib.sha256()
    files = ["recurrent_state_decode_amd/csrc/decode_kernel.hpp"]
    if chunked:
        files.append("recurrent_state_decode_amd/csrc/prefill_kernel.hpp")
    files += ["recurrent_state_decode_amd/csrc/gdn_decode.hip", "include/gdn_decode.h"]
    for rel in files:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, storage="f32"):
    """State read+write for every (sequence, head) with a non-empty suffix, plus per-token I/O.

    A packed int8_hadamard32 pool moves K V code bytes and K V / 32 float32 scales per tile, a packed
    fp8 pool K V code bytes and V / block_v float32 scales (the tile padded to whole 128-byte lines), instead of K V float32
    states."""
    import numpy as np
    import torch
    esz = 2 if w.io_dtype == torch.bfloat16 else 4
    osz = 2 if w.out_dtype == torch.bfloat16 else 4
    if w.kind in ("gdn_paged", "kda_paged") or w.inputs.get("cu_seqlens") is None:
        active = w.B
    else:
        active = int(np.sum(np.diff(w.inputs["cu_seqlens"].numpy()) > 0))
    if storage == "i8h32":
        tile = w.K * w.V + 4 * w.K * (w.V // 32)
    elif storage == "fp8":
        tile = 128 * ((w.K * w.V + 4 * (w.V // w.options.get("block_v", 64)) + 127) // 128)
    else:
        tile = w.K * w.V * 4
    state = 2 * active * w.HV * tile
    if w.kind.endswith("paged_varlen"):
        # one tile read per sequence; every page a suffix fills or ends on is written: sequence b
        # holds n = (pages - 1) page_size + last_page_len tokens and decodes its last T_b, so it writes
        # a page for each multiple of page_size in (n - T_b, n], plus the last page unless n is one
        ps = w.options["page_size"]
        cu = w.inputs["cu_seqlens"].numpy().astype(np.int64)
        ptr = w.inputs["page_indptr"].numpy().astype(np.int64)
        lpl = w.inputs["last_page_len"].numpy().astype(np.int64)
        t_b = np.diff(cu)
        n = (np.diff(ptr) - 1) * ps + lpl
        n_writes = int(np.sum(np.where(t_b > 0, n // ps - (n - t_b) // ps + (n % ps != 0), 0)))
        state = (active + n_writes) * w.HV * tile
    T = w.T
    per_tok = 2 * w.HK * w.K * esz + w.HV * w.V * esz + w.HV * w.V * osz
    if w.kind.startswith("kda"):
        per_tok += w.HV * w.K * esz + w.HV * esz
    else:
        per_tok += 2 * w.HV * esz
    return state, T * per_tok


PEAK_FP32_MFMA_TFLOPS = 157.3


def chunked_flops(w):
    """Algorithmic FLOPs of the chunked prefill's WY form: per chunk of 16 aligned positions, value head
    and 128 value columns, 2 x (k.k^T and q.k^T: 2 x 16 x 16 x K; K S0, Q S0 and the state update:
    3 x 16 x K x 128; T (V - ...) and P U: 2 x 16 x 16 x 128) multiply-adds; the 16 x 16 solve is
    negligible."""
    import numpy as np
    cu = w.inputs["cu_seqlens"].numpy()
    lpl = w.inputs["last_page_len"].numpy()
    ptr = w.inputs["page_indptr"].numpy()
    ps = w.options["page_size"]
    chunks = 0
    for b in range(w.B):
        n = int(cu[b + 1] - cu[b])
        if n <= 0:
            continue
        pos_last = int(ptr[b + 1] - ptr[b] - 1) * ps + int(lpl[b])
        pos0 = pos_last - n + 1
        chunks += (pos_last - 1) // 16 - (pos0 - 1) // 16 + 1
    per = 2 * (2 * 16 * 16 * w.K + 3 * 16 * w.K * 128 + 2 * 16 * 16 * 128)
    return chunks * w.HV * (w.V // 128) * per


class ClockSampler:
    """Samples the GPU's current shader and memory clocks from a thread while the timed steps run: the
    amdgpu sysfs files pp_dpm_sclk / pp_dpm_mclk list the clock levels, and the one marked '*' carries the
    current frequency.  summary() gives min / median / max per clock over the samples."""

    def __init__(self, period_s=0.0005):
        import glob
        import threading
        self.period = period_s
        self.paths = {}
        for key in ("sclk", "mclk"):
            found = sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{key}"))
            if found:
                self.paths[key] = found[0]
        self.samples = {k: [] for k in self.paths}
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self, path):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for k, path in self.paths.items():
                v = self._read(path)
                if v is not None:
                    self.samples[k].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        import statistics
        out = {}
        for k, v in self.samples.items():
            if v:
                out[k + "_mhz"] = {"min": min(v), "median": statistics.median(v), "max": max(v), "samples": len(v)}
        return out or None


def copy_bandwidth(torch, dev, flush):
    """Best of three plain 1 GiB -> 1 GiB device copies, in GB/s (read + write bytes)."""
    n = 256 * 1024 * 1024
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    best = None
    for _ in range(3):
        if flush is not None:
            flush.fill_(0.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * n * 4 / (best * 1e-3) / 1e9


def stream_reference(torch, rsd, w, pool, d, flush, steps, warmup, stream, state_bytes):
    """The step's state traffic without its arithmetic: gdn_stream_rows over the same (read row, write row)
    pairs as the decode (paged: from gdn_paged_decode_slots; pooled: (slot, slot) of every non-empty
    suffix), timed the same way (cache flush before each launch, HIP events around it).  Its rate is what
    this access pattern reaches on this machine, a reference for the decode kernel's.  None for packed pools
    and multi-token paged workloads (their row pattern is not one read and one write per sequence)."""
    import numpy as np
    if pool.dtype != torch.float32:
        return None
    if w.kind in ("gdn_paged", "kda_paged"):
        slots = rsd.gdn_paged_decode_slots(d["page_indices"], d["page_indptr"], d["last_page_len"])
    elif w.kind in ("gdn_pooled", "kda_pooled"):
        si = w.inputs["state_indices"].to(torch.int64)
        cu = w.inputs.get("cu_seqlens")
        if cu is not None:
            si = si[torch.from_numpy(np.diff(cu.numpy()) > 0)]
        slots = torch.stack([si, si], dim=1).contiguous().to(pool.device)
    else:
        return None
    if pool[0].numel() % 512:
        return None
    for i in range(warmup):
        if flush is not None:
            flush.fill_(float(i & 7))
        rsd.stream_rows(pool, pool, slots)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i & 7))
        starts[i].record(stream)
        rsd.stream_rows(pool, pool, slots)
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / steps
    return {"kernel": "gdn::stream_rows_kernel", "ms_per_step": round(ms, 5),
            "state_gbps": round(state_bytes / (ms * 1e-3) / 1e9, 1), "rows": int(slots.shape[0])}


def kernel_name(w):
    """The kernel a workload's step launches (as rocprofv3 names it, without template arguments): GDN chunked
    prefill with 16-bit inputs runs the producer / consumer kernel, other chunked prefills the four-wave one."""
    if not w.chunked:
        return "gdn::decode_kernel"
    if w.kind.startswith("gdn") and w.io_dtype.itemsize == 2:
        return "gdn::prefill_ws_kernel"
    return "gdn::prefill_kernel"


def is_kernel(name, kern):
    """Whether a rocprofv3 kernel name is `kern` itself (template arguments or parameters follow), not a longer
    name that begins with it."""
    return re.search(re.escape(kern) + r"[<(]", name) is not None


def traffic_path(workload_name):
    return os.path.join(ROOT, "profiles", f"traffic_{workload_name}.txt")


def load_traffic(workload_name, chunked=False):
    """Per-launch HBM bytes from a committed rocprofv3 counter summary, if it matches these sources."""
    path = traffic_path(workload_name)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_hash") != source_hash(chunked):
        return None
    return int(rec["bytes_per_launch"])


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def summarize_profiles(kt_dir, fetch_dir, write_dir, commands):
    """Turn rocprofv3 outputs into the short summaries kept under profiles/.

    kt_dir: a --kernel-trace --stats run of bench.py; fetch_dir / write_dir:
    --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of bench.py --copy-calibration.
    The plain 1 GiB copy in those runs gives the scale of each counter.
    """
    import csv
    import statistics

    def load_json(d):
        with open(d.rstrip("/") + ".json") as f:
            return json.loads(f.read().strip().splitlines()[-1])

    bench_kt = load_json(kt_dir)
    name = bench_kt["config"]["workload"]
    kern = bench_kt["roofline"]["kernel"]
    # kernel trace: per-dispatch durations of the decode kernel, warm-up dispatches dropped
    trace = [r for f in _csvs(kt_dir, "kernel_trace.csv") for r in csv.DictReader(open(f))]
    dec = sorted((r for r in trace if is_kernel(r["Kernel_Name"], kern)), key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in dec]
    timed = durs[bench_kt["warmup"]:]
    stats = [r for f in _csvs(kt_dir, "kernel_stats.csv") for r in csv.DictReader(open(f))]
    lines = [f"# rocprofv3 kernel trace: {name}", "", "Command (from the repository root):", "",
             "    " + commands["kt"], "",
             f"bench.py line of this run: ms_per_step={bench_kt['ms_per_step']} "
             f"(HIP events around each launch, after the cache-flush kernel), value={bench_kt['value']} tokens/s", "",
             f"{kern}, timed dispatches ({len(timed)}): mean {statistics.mean(timed):.1f} us, "
             f"median {statistics.median(timed):.1f} us, min {min(timed):.1f} us, max {max(timed):.1f} us", "",
             "| kernel | calls | average ns | min ns | max ns | % time |", "|---|---|---|---|---|---|"]
    for r in stats:
        kname = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
        lines.append(f"| {kname} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.1f} |")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def counter(d, cname):
        rows = [r for f in _csvs(d, "counter_collection.csv") for r in csv.DictReader(open(f))]
        dec_v = [float(r["Counter_Value"]) for r in rows if is_kernel(r["Kernel_Name"], kern) and r["Counter_Name"] == cname]
        big = [r for r in rows if r["Counter_Name"] == cname and "copyBuffer" in r["Kernel_Name"]]
        big = [float(r["Counter_Value"]) for r in big if int(r["Grid_Size"]) >= 65536]
        return statistics.median(dec_v), statistics.median(big), len(dec_v)

    bench_f = load_json(fetch_dir)
    copy_kib = bench_f["copy_calibration_bytes"] / 1024
    f_dec, f_copy, nf = counter(fetch_dir, "FETCH_SIZE")
    w_dec, w_copy, nw = counter(write_dir, "WRITE_SIZE")
    f_scale, w_scale = f_copy / copy_kib, w_copy / copy_kib
    read_b = f_dec / f_scale * 1024
    write_b = w_dec / w_scale * 1024
    alg = bench_kt["roofline"]["algorithmic_bytes_per_launch"]
    tl = [f"# rocprofv3 HBM traffic counters: {name}", "",
          "Commands (from the repository root, one counter per run):", "",
          "    " + commands["fetch"], "    " + commands["write"], "",
          "Each run also copies 1 GiB -> 1 GiB once per call with a plain device copy (bench.py",
          "--copy-calibration); what the counter reads for that copy scales the decode kernel's reading.", "",
          f"workload: {name}",
          f"kernel: {kern}",
          f"source_hash: {bench_kt['roofline']['source_hash']}",
          f"decode FETCH_SIZE KiB per dispatch (median of {nf}): {f_dec:.1f}",
          f"decode WRITE_SIZE KiB per dispatch (median of {nw}): {w_dec:.1f}",
          f"copy FETCH_SIZE KiB for {copy_kib:.0f} KiB read: {f_copy:.1f} (scale {f_scale:.4f})",
          f"copy WRITE_SIZE KiB for {copy_kib:.0f} KiB written: {w_copy:.1f} (scale {w_scale:.4f})",
          f"read_bytes_per_launch: {read_b:.0f}",
          f"write_bytes_per_launch: {write_b:.0f}",
          f"bytes_per_launch: {read_b + write_b:.0f}",
          f"algorithmic_bytes_per_launch: {alg}",
          f"traffic_over_algorithmic: {(read_b + write_b) / alg:.4f}"]
    with open(traffic_path(name), "w") as f:
        f.write("\n".join(tl) + "\n")
    print("\n".join(tl))


# ---------------------------------------------------------------- the oracle on the host cores (cpu_baseline)
#
# The oracle runs in worker processes forked before this process makes any GPU call (a process that
# holds the GPU must not fork or exec).  Each worker takes every n-th sequence of the workload, draws
# the pool rows those sequences read (N(0, 0.05), the workload's state distribution: the timing does
# not depend on the values), waits for the others at a barrier, and runs the oracle over its sequences
# in batches of 8, round after round, until the time budget is spent.  Only the oracle's arithmetic is
# timed; the whole-host rate is the tokens all workers finished divided by the budget's wall time.

_CPU = {}


COUNTERS = ("VALUBusy", "VALUUtilization", "OccupancyPercent", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
            "SQ_WAVES")
# the matrix-core set, for the kernels that run MFMA (the chunked prefill): cycles the MFMA pipe of each
# SIMD is busy, MFMA instructions issued, and the same clock and wave counts
COUNTERS_MFMA = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_WAVES",
                 "GRBM_GUI_ACTIVE")
SIMDS = 1024        # 256 CUs x 4 SIMDs
XCDS = 8


def summarize_counters(run_dir, sel):
    """profiles/counters_<workload>.txt from one rocprofv3 run with --pmc COUNTERS and --kernel-trace.

    Per dispatch of the kernel the bench times (medians over its dispatches): VALUBusy (percent of the
    active time some VALU instruction issues), VALUUtilization (active lanes), OccupancyPercent (resident
    waves against 32 per CU), VALU and LDS instructions per wave, and the shader clock the kernel ran at,
    GRBM_GUI_ACTIVE cycles over the dispatch's duration.  A run with --pmc COUNTERS_MFMA instead writes
    profiles/counters_mfma_<workload>.txt: MFMA instructions per wave, the cycles the matrix pipe is
    busy per instruction, and the fraction of the kernel's cycles each SIMD's pipe is busy
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / XCDS cycles x SIMDS)."""
    import csv
    import statistics

    with open(run_dir.rstrip("/") + ".json") as f:
        bench_line = json.loads(f.read().strip().splitlines()[-1])
    name = bench_line["config"]["workload"]
    kern = bench_line["roofline"]["kernel"]
    rows = [r for f in _csvs(run_dir, "counter_collection.csv") for r in csv.DictReader(open(f))]
    trace = [r for f in _csvs(run_dir, "kernel_trace.csv") for r in csv.DictReader(open(f))]
    dur = {r["Dispatch_Id"]: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
           for r in trace if is_kernel(r["Kernel_Name"], kern)}
    per = {}
    meta = {}
    for r in rows:
        if not is_kernel(r["Kernel_Name"], kern):
            continue
        per.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
        meta = {k: r.get(k) for k in ("VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size",
                                      "Scratch_Size", "Workgroup_Size", "Grid_Size")}
    med = {k: statistics.median(v.values()) for k, v in per.items()}
    waves = med.get("SQ_WAVES", 0) or 1
    clocks = [per["GRBM_GUI_ACTIVE"][d] / dur[d] for d in per.get("GRBM_GUI_ACTIVE", {}) if d in dur and dur[d] > 0]
    mfma = "SQ_VALU_MFMA_BUSY_CYCLES" in med
    command = (f"rocprofv3 --pmc {' '.join(COUNTERS_MFMA if mfma else COUNTERS)} --kernel-trace -d {run_dir} -o c "
               f"--output-format csv -- python3 bench.py{sel} --steps 10 --warmup 1 --no-cpu-baseline > {run_dir}.json")
    head = [f"# rocprofv3 {'matrix-core' if mfma else 'activity'} counters: {name}", "",
            "Command (from the repository root):", "", "    " + command, "",
            f"kernel: {kern}", f"source_hash: {bench_line['roofline']['source_hash']}",
            f"dispatches: {len(dur)}; kernel duration median {statistics.median(dur.values()):.1f} us" if dur else
            "dispatches: 0",
            *(f"{k}: {v}" for k, v in meta.items()),
            *(f"{k} (median per dispatch): {med[k]:.4g}" for k in (COUNTERS_MFMA if mfma else COUNTERS) if k in med)]
    clock_line = (f"GRBM_GUI_ACTIVE per us of the dispatch (median): {statistics.median(clocks):.0f}" if clocks else
                  "GRBM_GUI_ACTIVE per us: n/a")
    if mfma:
        n_mfma = med.get("SQ_INSTS_MFMA", 0)
        busy = med["SQ_VALU_MFMA_BUSY_CYCLES"]
        cycles = med.get("GRBM_GUI_ACTIVE", 0) / XCDS
        lines = head + [f"MFMA instructions per wave: {n_mfma / waves:.1f}",
                        f"MFMA pipe busy cycles per MFMA instruction: {busy / n_mfma:.2f}" if n_mfma else
                        "MFMA pipe busy cycles per MFMA instruction: n/a",
                        f"MFMA pipe busy fraction per SIMD: {busy / (cycles * SIMDS):.3f}" if cycles else
                        "MFMA pipe busy fraction per SIMD: n/a", clock_line]
    else:
        lines = head + [f"VALU instructions per wave: {med.get('SQ_INSTS_VALU', 0) / waves:.1f}",
                        f"LDS instructions per wave: {med.get('SQ_INSTS_LDS', 0) / waves:.1f}", clock_line]
    path = os.path.join(ROOT, "profiles", f"counters_{'mfma_' if mfma else ''}{name}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_cores():
    """Host cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS when that is set (the
    share of the host that belongs to one GPU)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _cpu_oracle_worker(idx):
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from tests import parity as P

    torch.set_num_threads(1)         # a forked child runs torch's CPU ops inline
    w, n, budget, barrier = _CPU["w"], _CPU["n"], _CPU["budget"], _CPU["barrier"]
    seqs = list(range(idx, w.B, n)) or [idx % w.B]
    rng = np.random.default_rng(7000 + idx)
    shape = w.pool_shape()[1:]
    reads, _ = P.rows_for(w, seqs)
    rows = {r: rng.standard_normal(shape) * 0.05 for r in set(reads)}
    with threadpool_limits(limits=1):
        barrier.wait(timeout=300)
        t0 = time.perf_counter()
        toks, nseq, i = 0, 0, 0
        while time.perf_counter() - t0 < budget:
            batch = [seqs[(i + j) % len(seqs)] for j in range(min(8, len(seqs)))]
            P.oracle_call(w, rows, seqs=batch)
            toks += len(P.token_rows(w, batch))
            nseq += len(batch)
            i += len(batch)
        return toks, nseq, time.perf_counter() - t0


def cpu_baseline(w, budget_s, single_budget_s):
    """Time the oracle on the host cores (and, beside it, on one core); call before any GPU work."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")

    def leg(n, budget):
        _CPU.update(w=w, n=n, budget=budget, barrier=ctx.Barrier(n))
        with ctx.Pool(n) as pool:
            res = pool.map(_cpu_oracle_worker, range(n), chunksize=1)
        toks = sum(r[0] for r in res)
        nseq = sum(r[1] for r in res)
        wall = max(r[2] for r in res)
        return toks, nseq, wall

    n = cpu_cores()
    toks, nseq, wall = leg(n, budget_s)
    toks1, nseq1, wall1 = leg(1, single_budget_s)
    return {"value": round(toks / wall, 1), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{nseq} sequences ({toks} tokens) of {w.name}: each of {n} worker processes takes every "
                      f"{n}-th sequence, batches of 8, repeated for {budget_s:.0f} s of wall time; float64 NumPy, "
                      f"one thread per worker",
            "seconds": round(wall, 3), "host_cpus": len(os.sched_getaffinity(0)),
            "single_core": {"value": round(toks1 / wall1, 1), "cores": 1, "seconds": round(wall1, 3),
                            "sample": f"{nseq1} sequences ({toks1} tokens), one worker"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="paged_gdn_b256",
                    choices=["paged_gdn_b256", "pooled_gdn_b64", "pooled_kda_varlen_b128", "fp8_qdq_gdn_b512",
                             "tiny_gdn", "paged_kda_b256", "paged_gdn_varlen_b256_t4", "int8h32_gdn_b512",
                             "paged_gdn_prefill_b16_t1024", "paged_kda_prefill_b16_t1024"])
    ap.add_argument("--layout", default=None, help="override the pool layout (K_FIRST / V_FIRST); a layout other than the workload's own gets a +LAYOUT suffix on its name")
    ap.add_argument("--qdq", default=None, choices=["none", "fp8_e4m3_tile", "int8_hadamard32"],
                    help="override the workload's state quantisation (the workload name gets a +qdq suffix)")
    ap.add_argument("--storage", default="f32", choices=["f32", "i8h32", "fp8"],
                    help="i8h32: a packed int8_hadamard32 pool (codes + scales; implies --qdq int8_hadamard32 and a "
                         "K_FIRST layout); fp8: a packed fp8 tile pool (E4M3 bytes + tile scales; implies --qdq "
                         "fp8_e4m3_tile, any layout); the workload name gets a +i8h32 / +fp8 suffix")
    ap.add_argument("--token-path", action="store_true",
                    help="run a chunked-prefill workload through the token-by-token paged call instead")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="wall seconds of the oracle on all host cores for cpu_baseline (one core: a third of it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 output directories (no GPU needed)")
    ap.add_argument("--summarize-counters", metavar="RUN_DIR",
                    help="write profiles/counters_<workload>.txt (or counters_mfma_<workload>.txt) from a "
                         "rocprofv3 --pmc run of COUNTERS (or COUNTERS_MFMA) with --kernel-trace (no GPU needed)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 1 GiB -> 1 GiB copy 3 times (a kernel of known traffic for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.summarize_profiles:
        kt, fe, wr = args.summarize_profiles
        sel = "" if args.workload == "paged_gdn_b256" else f" --workload {args.workload}"
        sel += f" --layout {args.layout}" if args.layout else ""
        sel += f" --qdq {args.qdq}" if args.qdq else ""
        sel += " --token-path" if args.token_path else ""
        sel += f" --storage {args.storage}" if args.storage != "f32" else ""
        cmds = {"kt": f"rocprofv3 --kernel-trace --stats -d {kt} -o kt --output-format csv -- "
                      f"python3 bench.py{sel} --steps 20 --warmup 2 --no-cpu-baseline",
                "fetch": f"rocprofv3 --pmc FETCH_SIZE -d {fe} -o f --output-format csv -- "
                         f"python3 bench.py{sel} --steps 10 --warmup 1 --no-cpu-baseline --copy-calibration",
                "write": f"rocprofv3 --pmc WRITE_SIZE -d {wr} -o w --output-format csv -- "
                         f"python3 bench.py{sel} --steps 10 --warmup 1 --no-cpu-baseline --copy-calibration"}
        summarize_profiles(kt, fe, wr, cmds)
        return

    if args.summarize_counters:
        sel = "" if args.workload == "paged_gdn_b256" else f" --workload {args.workload}"
        sel += f" --layout {args.layout}" if args.layout else ""
        sel += f" --qdq {args.qdq}" if args.qdq else ""
        sel += " --token-path" if args.token_path else ""
        sel += f" --storage {args.storage}" if args.storage != "f32" else ""
        summarize_counters(args.summarize_counters, sel)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Every (sequence, value head) state is independent, so the pool would shard by value heads or by "
              "sequences with this same kernel on each GPU's share.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_state_decode_amd import workloads as wl

    dev = torch.device("cuda", 0)
    maker = wl.NAMED[args.workload]
    paged_makers = ("paged_gdn_b256", "paged_kda_b256", "paged_gdn_varlen_b256_t4", "paged_gdn_prefill_b16_t1024",
                    "paged_kda_prefill_b16_t1024")
    packed = args.storage != "f32"
    if args.storage == "i8h32":
        if args.qdq not in (None, "int8_hadamard32") or args.layout not in (None, "K_FIRST"):
            raise SystemExit("--storage i8h32 holds int8_hadamard32 codes in a K_FIRST layout")
        args.qdq, args.layout = "int8_hadamard32", "K_FIRST"
    elif args.storage == "fp8":
        if args.qdq not in (None, "fp8_e4m3_tile"):
            raise SystemExit("--storage fp8 holds fp8_e4m3_tile codes")
        args.qdq = "fp8_e4m3_tile"
    if args.workload in paged_makers:
        default_layout = inspect.signature(maker).parameters["state_layout"].default
        w = maker(state_layout=args.layout) if args.layout else maker()
    else:
        w = maker()
        default_layout = w.state_layout
        if args.layout:
            w.state_layout = args.layout
    if args.layout and args.layout != default_layout:
        w.name = f"{w.name}+{args.layout}"     # its own profiles and traffic figure
    if args.token_path and w.chunked:
        w.chunked = False
        w.name = f"{w.name}+token_path"
    if args.qdq is not None and args.qdq != w.options.get("qdq", "none"):
        if args.qdq == "none":
            w.options.pop("qdq", None)
        else:
            w.options["qdq"] = args.qdq
            w.options.setdefault("block_v", 64)
        w.name = f"{w.name}+{args.qdq}"
    if packed:
        w.name = f"{w.name}+{args.storage}"
    # the oracle on the host cores first: its worker processes are forked before this process touches the GPU
    cpu_res = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget, args.cpu_budget / 3)
    torch.cuda.set_device(dev)
    d = wl.device_inputs(w, dev)
    # (a packed pool for timing: seeded random codes and scales)
    pool = wl.random_packed_pool(w, dev) if packed else wl.make_pool(w, dev)
    out = torch.empty((w.T, w.HV, w.V), dtype=w.out_dtype, device=dev)
    flush = None if args.no_flush else torch.empty(512 * 1024 * 1024, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] workload {w.name} layout {w.state_layout} pool {tuple(pool.shape)} "
          f"({pool.numel() * pool.element_size() / 2**30:.1f} GiB)", file=sys.stderr, flush=True)

    def step(i):
        if flush is not None:
            flush.fill_(float(i & 7))
        wl.run(w, pool, d, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            if flush is not None:
                flush.fill_(float(i & 7))
            starts[i].record(stream)
            wl.run(w, pool, d, out=out)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    times_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    mean_ms = sum(times_ms) / len(times_ms)
    med_ms = sorted(times_ms)[len(times_ms) // 2]

    tokens = w.T
    state_b, io_b = algorithmic_bytes(w, args.storage)
    achieved = (state_b + io_b) / (mean_ms * 1e-3) / 1e9
    traffic = load_traffic(w.name, w.chunked)
    res = {
        "metric": METRIC,
        "value": round(tokens / (mean_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "kind": w.kind, "B": w.B, "HK": w.HK, "HV": w.HV, "K": w.K, "V": w.V,
                   "tokens_per_step": tokens, "state_layout": w.state_layout,
                   "io_dtype": str(w.io_dtype).replace("torch.", ""), "pool_rows": w.num_rows,
                   "cache_flush_between_steps": flush is not None, "state_storage": args.storage,
                   **{k: v for k, v in w.options.items()}},
        "state_pool_gbps": round(state_b / (mean_ms * 1e-3) / 1e9, 1),
        "state_pool_pct_peak": round(100 * state_b / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "ms_per_step_median": round(med_ms, 5),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": state_b + io_b,
                     "kernel": kernel_name(w), "source_hash": source_hash(w.chunked)},
    }
    if not args.copy_calibration:
        import recurrent_state_decode_amd as rsd
        ref = stream_reference(torch, rsd, w, pool, d, flush, args.steps, args.warmup, stream, state_b)
        if ref is not None:
            # the decode kernel's state rate as a fraction of the plain stream's over the same rows
            ref["decode_frac_of_stream"] = round(ref["ms_per_step"] / mean_ms, 4)
            res["state_stream_reference"] = ref
    try:
        cbw = copy_bandwidth(torch, dev, flush)
        res["device_copy_gbps"] = round(cbw, 1)        # torch's 1 GiB device-to-device copy, best of 3
        res["frac_of_device_copy"] = round(achieved / cbw, 4)
    except RuntimeError:
        pass
    # clocks sampled while the timed steps ran (the GPU idles before and after them)
    res["gpu_clocks_during_timed_steps"] = clocks.summary()
    if w.chunked:
        fl = chunked_flops(w)
        tf = fl / (mean_ms * 1e-3) / 1e12
        res["roofline_mfma_fp32"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP32_MFMA_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
                                     "algorithmic_flops_per_launch": fl}
    if args.copy_calibration:
        n = 256 * 1024 * 1024
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            flush.fill_(0.0) if flush is not None else None
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n * 4
    if cpu_res is not None:
        res["cpu_baseline"] = cpu_res
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

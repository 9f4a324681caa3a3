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
  cpu_baseline the CPU oracle timed on this host on a bounded sample of the
               same workload (rank 0, one GPU only)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "tokens/s & state-pool HBM GB/s (% peak), GDN decode B=256,HV=32,K=V=128"


def source_hash():
    """Hash of the sources the kernels are built from (ties a profile to a kernel version)."""
    h = hashlib.sha256()
    for rel in ("recurrent_state_decode_amd/csrc/decode_kernel.hpp", "recurrent_state_decode_amd/csrc/gdn_decode.hip",
                "include/gdn_decode.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """State read+write for every (sequence, head) with a non-empty suffix, plus per-token I/O."""
    import numpy as np
    import torch
    esz = 2 if w.io_dtype == torch.bfloat16 else 4
    osz = 2 if w.out_dtype == torch.bfloat16 else 4
    if w.kind == "gdn_paged" or w.inputs.get("cu_seqlens") is None:
        active = w.B
    else:
        active = int(np.sum(np.diff(w.inputs["cu_seqlens"].numpy()) > 0))
    state = 2 * active * w.HV * w.K * w.V * 4
    T = w.T
    per_tok = 2 * w.HK * w.K * esz + w.HV * w.V * esz + w.HV * w.V * osz
    if w.kind == "kda_pooled":
        per_tok += w.HV * w.K * esz + w.HV * esz
    else:
        per_tok += 2 * w.HV * esz
    return state, T * per_tok


def load_traffic(workload_name):
    """Per-launch HBM bytes from a committed rocprofv3 counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, pool, budget_s):
    """Time the oracle on the first sequences of the workload until about ``budget_s`` seconds."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from tests import parity as P

    seqs_all = list(range(w.B))
    reads, _ = P.rows_for(w)
    # pool rows are read back before timing; only the oracle arithmetic is timed
    with threadpool_limits(limits=1):
        done, t_used, toks = 0, 0.0, 0
        batch = 8
        while done < len(seqs_all) and t_used < budget_s:
            seqs = seqs_all[done:done + batch]
            r, _ = P.rows_for(w, seqs)
            rows = P.gather_rows(pool, r)
            t0 = time.perf_counter()
            P.oracle_call(w, rows, seqs=seqs)
            t_used += time.perf_counter() - t0
            toks += len(P.token_rows(w, seqs))
            done += len(seqs)
    return {"value": toks / t_used, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {w.B} sequences ({toks} tokens) of {w.name}, float64 NumPy, one thread",
            "seconds": round(t_used, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="paged_gdn_b256",
                    choices=["paged_gdn_b256", "pooled_gdn_b64", "pooled_kda_varlen_b128", "fp8_qdq_gdn_b512",
                             "tiny_gdn"])
    ap.add_argument("--layout", default=None, help="override the pool layout (K_FIRST / V_FIRST)")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Every (sequence, value head) state is independent; see DESIGN.md for how the pool would shard.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_state_decode_amd import workloads as wl
    from tests import parity as P

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    maker = wl.NAMED[args.workload]
    w = maker(state_layout=args.layout) if (args.layout and args.workload == "paged_gdn_b256") else maker()
    if args.layout and args.workload != "paged_gdn_b256":
        w.state_layout = args.layout
    d = P.device_inputs(w, dev)
    pool = wl.make_pool(w, dev)
    out = torch.empty((w.T, w.HV, w.V), dtype=w.out_dtype, device=dev)
    flush = None if args.no_flush else torch.empty(512 * 1024 * 1024, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] workload {w.name} layout {w.state_layout} pool {tuple(pool.shape)} "
          f"({pool.numel() * 4 / 2**30:.1f} GiB)", file=sys.stderr, flush=True)

    def step(i):
        if flush is not None:
            flush.fill_(float(i & 7))
        P.gpu_call(w, pool, d, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(float(i & 7))
        starts[i].record(stream)
        P.gpu_call(w, pool, d, out=out)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    mean_ms = sum(times_ms) / len(times_ms)
    med_ms = sorted(times_ms)[len(times_ms) // 2]

    tokens = w.T
    state_b, io_b = algorithmic_bytes(w)
    achieved = (state_b + io_b) / (mean_ms * 1e-3) / 1e9
    traffic = load_traffic(w.name)
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
                   "cache_flush_between_steps": flush is not None, **{k: v for k, v in w.options.items()}},
        "state_pool_gbps": round(state_b / (mean_ms * 1e-3) / 1e9, 1),
        "state_pool_pct_peak": round(100 * state_b / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "ms_per_step_median": round(med_ms, 5),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": state_b + io_b,
                     "kernel": "gdn::decode_kernel", "source_hash": source_hash()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, pool, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Helpers shared by the GPU parity tests, the smoke run and the bench's oracle leg.

They move seeded workloads to the device, call the HIP library through its
Python binding, run the CPU oracle on the same values (pool rows read back
from the device before the call), and compare the two under the tolerances
below.  The oracle runs on groups of at most 64 QDQ tokens (1024 otherwise)
so that its per-token trace stays bounded in host memory, on a few threads
side by side; sums over the whole call (the outputs' relative L2 error, the
flip counts) decide the call-wide checks.

Tolerances (readings of the stated contract):
* index work is exact: the rows written are exactly the call's write rows,
  every other pool byte is bit-identical to its value before the call;
* fp32 states: |gpu - ref| <= 2e-3 * (|ref| + rms(ref over the row's tile));
* outputs: the oracle value is rounded to the output dtype (nearest even)
  first; bf16 outputs must then agree to one bf16 ulp at the larger
  magnitude plus 1e-5 * rms(ref) (an absolute floor for values near 0),
  fp32 outputs to 2e-3 * (|ref| + rms(ref)); and the relative L2 error of
  all outputs against the unrounded oracle must be <= 2e-3 (plus, for bf16,
  the 2^-9 relative rounding the output dtype itself adds);
* fp8 tile QDQ ("one quantisation step"): every rounding of the state may
  land one E4M3 step (the grid spacing at that magnitude, in its tile's
  scale) away from the oracle's, and an earlier difference is carried by the
  recurrence's linear update.  So the bound E_t on |gpu - oracle| of the
  state after token t is E_t = A(E_{t-1}) + step_t, with
  A(E) = alpha*E + beta |k_hat| (|k_hat|^T (alpha*E)) the elementwise bound
  of the update's action on a state difference, E_0 = 0 (one step of S_0
  with quantize_initial), plus 1e-5 relative for float32 arithmetic.  A
  working-readout output is bounded by its bf16 ulp + |q_hat|^T(alpha E_{t-1})
  + |q_hat . k_hat| beta |k_hat|^T (alpha E_{t-1}); a stored-readout output by
  its ulp + |q_hat|^T E_t.  Since a bound of this kind would also accept a
  systematically different rounding rule, the fraction of state elements
  rounded the other way (moved by more than half a step) must stay below
  1e-3 over the whole call (exact agreement of the rounding itself is
  tested separately with a scale of exactly 1).  Where a token amplifies an
  error along its key (|1 - beta |k_hat|^2| > 1: unnormalised keys, or a
  probability-mode beta outside [0, 1]) a carried difference can grow, so
  the flip rate is then counted only on states no earlier difference
  reached: a suffix's state after its first token, without quantize_initial.
* the oracle decides every rounding in float64 (the pages fix only the
  amax / 448 tile scale and the codec's per-group scale; float64 is the
  plain reading); a second comparison with the decisions taken in float32,
  as the kernel takes them, shows how often the two precisions decide
  differently and is held to the same bounds.
* int8_hadamard32 codec: per (key row, 32 values) group the two sides'
  rounding errors in the rotated basis are each at most half a step
  amax|y| / 127 (amax taken over the larger of the two states, i.e. the
  oracle's plus the carried difference), so after rotating back an element
  differs by at most sqrt(32) steps more than the carried difference -- a
  bound that holds for any code choice; so the fraction of rotated
  coordinates that differ by more than a quarter step (a different code)
  must stay below 1e-3.
* packed int8_hadamard32 pools: the written tiles, decoded, meet the codec
  bound above; their codes equal the oracle's encoding of its final state
  except for at most 1e-3 of them, each off by one (a rounding decided the
  other way), and their scales agree to 1e-5 relative except in at most 1 %
  of the groups (those an earlier such rounding moved), never by 1 % or more.
"""
import concurrent.futures
import math
import os

import numpy as np
import torch

import recurrent_state_decode_amd as rsd
from recurrent_state_decode_amd import workloads as wl
from oracle import decode as odec
from oracle import e4m3
from oracle import hadamard as ohad
from oracle import paging as opaging

STATE_RTOL = 2e-3
OUT_REL_L2 = 2e-3


device_inputs = wl.device_inputs
gpu_call = wl.run
_opts = wl.call_options


def host64(t):
    return None if t is None else t.detach().to("cpu").to(torch.float64).numpy()


def host_int(t):
    return None if t is None else t.detach().to("cpu").to(torch.int64).numpy()


def written_rows(w, b):
    """[(token index inside the suffix, pool row)] the call writes for sequence b (none if its suffix is empty)."""
    inp = w.inputs
    cu = host_int(inp.get("cu_seqlens"))
    if cu is not None and cu[b + 1] <= cu[b]:
        return []
    nb = 1 if cu is None or w.kind in ("gdn_paged", "kda_paged") else int(cu[b + 1] - cu[b])
    if w.kind.endswith("paged_varlen"):
        return opaging.paged_suffix_rows(host_int(inp["page_indices"]), host_int(inp["page_indptr"]),
                                         host_int(inp["last_page_len"]), w.options["page_size"], nb, b)[1]
    return [(nb - 1, rows_for(w, [b])[1][0])]


def rows_for(w, seqs=None):
    """(read rows, write rows) of the sequences ``seqs`` (all if None), from the host tables."""
    inp = w.inputs
    seqs = range(w.B) if seqs is None else seqs
    reads, writes = [], []
    cu = host_int(inp.get("cu_seqlens"))
    for b in seqs:
        if cu is not None and cu[b + 1] <= cu[b]:
            continue
        if w.kind in ("gdn_paged", "kda_paged"):
            ind, ptr, lpl = host_int(inp["page_indices"]), host_int(inp["page_indptr"]), host_int(inp["last_page_len"])
            last = int(ind[ptr[b + 1] - 1])
            reads.append(int(ind[ptr[b + 1] - 2]) if lpl[b] == 1 else last)
            writes.append(last)
        elif w.kind in ("gdn_paged_varlen", "kda_paged_varlen"):
            r, wr = opaging.paged_suffix_rows(host_int(inp["page_indices"]), host_int(inp["page_indptr"]),
                                              host_int(inp["last_page_len"]), w.options["page_size"],
                                              int(cu[b + 1] - cu[b]), b)
            reads.append(r)
            writes.extend(row for _, row in wr)
        else:
            s = int(inp["state_indices"][b])
            reads.append(s)
            writes.append(s)
    return reads, writes


def oracle_call(w, pool_rows, seqs=None, trace=None, qdq_precision="float64", **over):
    """Run the CPU oracle for workload ``w`` on ``pool_rows`` {row: float64 tile}; ``qdq_precision`` is the
    precision of the oracle's rounding decisions (float64, the pages' plain reading, or float32)."""
    o = _opts(w, over, drop=("out_dtype", "slots"))
    inp = w.inputs
    common = dict(state_layout=w.state_layout, seqs=seqs, trace=trace, qdq_precision=qdq_precision, **o)
    kda = w.kind.startswith("kda")
    gate = host64(inp["raw_gate"] if kda else inp["a"])
    beta = host64(inp["beta_logits"] if kda else inp["b"])
    alog = host64(inp["a_log"] if kda else inp["A_log"])
    qkv = (host64(inp["q"]), host64(inp["k"]), host64(inp["v"]), gate, beta, alog, host64(inp["dt_bias"]))
    cu = host_int(inp.get("cu_seqlens"))
    if w.kind in ("gdn_pooled", "kda_pooled"):
        fn = odec.kda_decode_pooled if kda else odec.gdn_decode_pooled
        return fn(*qkv, cu, host_int(inp["state_indices"]), pool_rows, **common)
    table = (host_int(inp["page_indices"]), host_int(inp["page_indptr"]), host_int(inp["last_page_len"]))
    if w.kind in ("gdn_paged", "kda_paged"):
        fn = odec.kda_decode_paged if kda else odec.gdn_decode_paged
        return fn(*qkv, *table, pool_rows, **common)
    if w.kind in ("gdn_paged_varlen", "kda_paged_varlen"):
        fn = odec.kda_decode_paged_varlen if kda else odec.gdn_decode_paged_varlen
        return fn(*qkv, cu, *table, w.options["page_size"], pool_rows, **common)
    raise ValueError(w.kind)


def gather_rows(pool, rows, dtype=torch.float64):
    """{row: host copy of pool[row]} (as ``dtype``) for the given rows."""
    rows = sorted(set(rows))
    if not rows:
        return {}
    idx = torch.tensor(rows, dtype=torch.int64, device=pool.device)
    vals = pool.index_select(0, idx).to("cpu").to(dtype).numpy()
    return {r: vals[i] for i, r in enumerate(rows)}


def seq_batches(w, seqs, max_tokens):
    """Consecutive groups of the sequences ``seqs`` holding at most ``max_tokens`` suffix tokens each (a longer
    suffix is a group of its own): the oracle runs and is compared one group at a time, so that its
    per-token trace stays bounded in host memory."""
    cu = host_int(w.inputs.get("cu_seqlens"))
    batch, ntok = [], 0
    for b in seqs:
        nb = 1 if (cu is None or w.kind in ("gdn_paged", "kda_paged")) else int(cu[b + 1] - cu[b])
        if batch and ntok + nb > max_tokens:
            yield batch
            batch, ntok = [], 0
        batch.append(b)
        ntok += nb
    if batch:
        yield batch


def bf16_ulp(x):
    _, ex = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(ex - 8, -133))


def token_rows(w, seqs):
    """Token indices (output rows) that belong to sequences ``seqs``."""
    if w.kind in ("gdn_paged", "kda_paged"):
        return np.array(sorted(seqs), dtype=np.int64)
    cu = host_int(w.inputs["cu_seqlens"])
    if cu is None:
        return np.array(sorted(seqs), dtype=np.int64)
    return np.concatenate([np.arange(cu[b], cu[b + 1]) for b in sorted(seqs)] + [np.zeros(0, np.int64)])


def _step_at(S, bv, mag):
    """E4M3 grid spacing at magnitude ``mag`` in the tile scale of S [H, K, V] (0 where the tile is 0)."""
    s = np.repeat(e4m3.tile_scales(S, bv), bv, axis=1)[:, None, :]
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(s > 0, s * e4m3.e4m3_spacing(mag / np.where(s > 0, s, 1)), 0.0)


def _rotate32(S):
    """[H, K, V] -> [H, K, V/32, 32] in the orthonormal Hadamard value basis of each 32-value group."""
    H, K, V = S.shape
    return S.reshape(H, K, V // 32, 32) @ (ohad.hadamard_matrix() / math.sqrt(32))


def _codec_step(S, carried):
    """Per-element bound of the codec's rounding difference on S [H, K, V], given the carried difference."""
    H, K, V = S.shape
    amax = np.max(np.abs(_rotate32(S)), axis=-1, keepdims=True)
    emax = np.max(np.asarray(carried).reshape(H, K, V // 32, 32), axis=-1, keepdims=True)
    step = (amax + math.sqrt(32) * emax) * (1 + 1e-5) / 127
    return np.broadcast_to(math.sqrt(32) * step, (H, K, V // 32, 32)).reshape(H, K, V)


def qdq_bounds(w, trace, seqs):
    """Propagated one-step-per-rounding bounds: ({token: output bound [H, V]},
    {seq: [state bound [H, K, V] after each of its tokens]})."""
    bv = w.options.get("block_v", 64)
    stored = w.options.get("readout", "working") == "stored"
    qinit = bool(w.options.get("quantize_initial", False))
    out_b, state_b = {}, {}
    cu = host_int(w.inputs.get("cu_seqlens"))
    for b in seqs:
        recs = trace.get(b, [])
        if not recs:
            continue
        t0 = b if (w.kind in ("gdn_paged", "kda_paged") or cu is None) else int(cu[b])
        S0 = recs[0]["S_in"]
        codec = w.options.get("qdq") == "int8_hadamard32"

        def rounding(S, carried):
            if codec:
                return _codec_step(S, carried)
            return _step_at(S, bv, (np.abs(S) + carried) * 1.125)

        E = rounding(S0, np.zeros_like(S0)) if qinit else np.zeros_like(S0)
        for i, rec in enumerate(recs):
            al = np.asarray(rec["alpha"], dtype=np.float64)
            al = al[:, None, None] if al.ndim == 1 else al[:, :, None]
            aE = al * E
            kabs = np.abs(rec["k_hat"])
            # |beta|: in probability mode beta is b itself, any real number
            babs = np.abs(rec["beta"])
            carried = aE + babs[:, None, None] * kabs[:, :, None] * np.einsum("hk,hkv->hv", kabs, aE)[:, None, :]
            S = rec["S_out"]
            E_new = carried + rounding(S, carried) + 1e-5 * np.abs(S)
            if stored:
                bound = np.einsum("hk,hkv->hv", np.abs(rec["q_hat"]), E_new)
            else:
                qk = np.abs(np.sum(rec["q_hat"] * rec["k_hat"], axis=-1))
                bound = (np.einsum("hk,hkv->hv", np.abs(rec["q_hat"]), aE)
                         + (qk * babs)[:, None] * np.einsum("hk,hkv->hv", kabs, aE))
            out_b[t0 + i] = bound
            E = E_new
            state_b.setdefault(b, []).append(E)
    return out_b, state_b


def non_expanding(trace):
    """True when no traced token amplifies an error along its key: |1 - beta |k_hat|^2| <= 1.  The
    delta write maps an error E to (I - beta k k^T) E along k, so with unnormalised keys or beta
    outside [0, 1] one rounding difference grows every token."""
    for recs in trace.values():
        for rec in recs:
            kk = np.sum(np.asarray(rec["k_hat"], dtype=np.float64) ** 2, axis=-1)
            if np.any(np.abs(1.0 - np.asarray(rec["beta"], dtype=np.float64) * kk) > 1.0 + 1e-9):
                return False
    return True


def flip_rows(w, trace, seqs):
    """Written rows whose elements count towards the flip-rate check, or None for all of them.

    The flip rate catches a wrong rounding rule: it is the fraction of elements that the two sides
    rounded to different codes.  Where no token amplifies an error (non_expanding) every written
    state counts.  Where one does, a rounding difference carried from an earlier token can grow and
    move later decisions, so only states that no earlier difference reached count: the state after a
    suffix's first token, without quantize_initial (both sides round the same state once)."""
    if non_expanding(trace):
        return None
    if w.options.get("quantize_initial"):
        return set()
    return {row for b in seqs for i, row in written_rows(w, b) if i == 0}


class Report:
    """Collects worst normalised errors for printing next to the pass/fail assertions."""

    def __init__(self):
        self.items = {}

    def add(self, k, v):
        self.items[k] = max(self.items.get(k, 0.0), float(v))

    def merge(self, other):
        for k, v in other.items.items():
            self.add(k, v)

    def __str__(self):
        return " ".join(f"{k}={v:.3g}" for k, v in self.items.items())


class Totals:
    """Whole-call sums that single batches of sequences cannot decide: the relative L2 error of the
    outputs and the counts behind the flip-rate checks."""

    SUMS = ("d2", "r2", "flips", "total", "code_flips", "codes", "off_scales", "groups")

    def __init__(self):
        self.d2 = 0.0          # sum (gpu - ref)^2 over compared outputs
        self.r2 = 0.0          # sum ref^2
        self.flips = 0         # state elements (or rotated coordinates) rounded the other way
        self.total = 0
        self.code_flips = 0    # packed pools: stored codes that differ from the oracle's encoding
        self.codes = 0
        self.off_scales = 0    # packed codec: group scales off by more than 1e-5
        self.groups = 0
        self.worst_scale = 0.0

    def merge(self, other):
        for k in self.SUMS:
            setattr(self, k, getattr(self, k) + getattr(other, k))
        self.worst_scale = max(self.worst_scale, other.worst_scale)


def compare_outputs(host_out, ref, w, rows, report, totals, qdq_bound=None):
    """Element-wise output check of the token rows ``rows`` (host_out: the GPU's outputs as float64 NumPy)."""
    g = host_out[rows]
    r = ref[rows]
    assert np.all(np.isfinite(r)), "oracle produced non-finite outputs"
    assert np.all(np.isfinite(g)), "GPU produced non-finite outputs"
    r_round = torch.from_numpy(r).to(w.out_dtype).to(torch.float64).numpy()
    rms = math.sqrt(float(np.mean(r * r))) if r.size else 0.0
    diff = np.abs(g - r_round)
    if w.out_dtype == torch.bfloat16:
        tol = bf16_ulp(np.maximum(np.abs(g), np.abs(r_round))) + 1e-5 * rms
    else:
        tol = STATE_RTOL * (np.abs(r) + rms)
    if qdq_bound is not None:
        tol = tol + qdq_bound
    ratio = diff / tol
    report.add("out_max_tol_ratio", ratio.max() if ratio.size else 0)
    bad = np.argwhere(diff > tol)
    assert bad.size == 0, f"{len(bad)} outputs out of tolerance; first {bad[:5].tolist()} gpu={g[tuple(bad[0])]} ref={r[tuple(bad[0])]}"
    totals.d2 += float(np.sum((g - r) ** 2))
    totals.r2 += float(np.sum(r * r))


def check_output_l2(w, report, totals):
    """Relative L2 error of all compared outputs against the unrounded oracle."""
    l2_tol = OUT_REL_L2 + (2.0 ** -9 if w.out_dtype == torch.bfloat16 else 0.0)
    rel = math.sqrt(totals.d2) / max(math.sqrt(totals.r2), 1e-30)
    report.add("out_rel_l2", rel)
    assert rel <= l2_tol, f"output relative L2 error {rel} > {l2_tol}"


def compare_states(gpu_rows, ref_rows, report, totals, qdq_bound=None, layout="K_FIRST", codec=None, block_v=64,
                   flip_rows=None):
    """fp32 states within the relative tolerance, or (QDQ) within the propagated bounds {row: [H, K, V]}.

    With QDQ, an element counts as rounded the other way (a flip) when it moves by more than half a
    quantisation step of its tile (fp8) or group (codec); a scale that moved because an earlier flip
    changed the tile's amax shifts every element by much less than that and is not counted.  Flips are
    counted in the rows ``flip_rows`` (None: all)."""
    assert set(gpu_rows) == set(ref_rows)
    for row, ref in ref_rows.items():
        g = gpu_rows[row]
        assert np.all(np.isfinite(g)), f"non-finite GPU state in row {row}"
        counted = flip_rows is None or row in flip_rows
        if qdq_bound is not None:
            logical = ref if layout == "K_FIRST" else np.swapaxes(ref, -1, -2)
            gl = g if layout == "K_FIRST" else np.swapaxes(g, -1, -2)
            tol = qdq_bound[row]
            diff = np.abs(gl - logical)
            if codec == "int8_hadamard32":
                yr = _rotate32(logical)
                dy = np.abs(_rotate32(gl) - yr)
                if counted:
                    totals.flips += int(np.sum(dy > 0.25 * np.max(np.abs(yr), axis=-1, keepdims=True) / 127))
                    totals.total += dy.size
            else:
                # the oracle's state is on its tiles' grids: scale = amax / 448 per [K, block_v] tile
                H, K, V = logical.shape
                amax = np.abs(logical).reshape(H, K, V // block_v, block_v).max(axis=(1, 3))
                sc = np.repeat(amax / 448.0, block_v, axis=-1)[:, None, :]
                step = e4m3.e4m3_spacing(np.abs(logical) / np.where(sc > 0, sc, 1.0)) * sc
                if counted:
                    totals.flips += int(np.sum(diff > 0.5 * step + 1e-30))
                    totals.total += diff.size
            report.add("qdq_state_bound_ratio", (diff / np.maximum(tol, 1e-300)).max())
        else:
            rms = np.sqrt(np.mean(ref * ref, axis=(-1, -2), keepdims=True))
            tol = STATE_RTOL * (np.abs(ref) + rms)
            diff = np.abs(g - ref)
            report.add("state_max_tol_ratio", (diff / tol).max())
            report.add("state_max_rel", (diff / (np.abs(ref) + rms)).max())
        bad = np.argwhere(diff > tol)
        assert bad.size == 0, f"row {row}: {len(bad)} state elements out of tolerance, first {bad[:3].tolist()}"


FLIP_RATE = 1e-3


def check_flip_rate(report, totals, what="QDQ state elements"):
    """The fraction of elements rounded the other way, over every counted row of the call."""
    if totals.total:
        frac = totals.flips / totals.total
        report.add("qdq_state_diff_frac", frac)
        report.add("qdq_flip_counted_elems", totals.total)
        assert frac < FLIP_RATE, f"{totals.flips} of {totals.total} {what} differ: rounding rule mismatch?"


def check_untouched(pool_before, pool_after, write_rows, chunk_rows=256):
    """Every row not in ``write_rows`` is bit-identical to its value before the call."""
    n = pool_before.shape[0]
    written = torch.zeros(n, dtype=torch.bool, device=pool_before.device)
    if write_rows:
        written[torch.tensor(sorted(set(write_rows)), device=pool_before.device)] = True
    changed = torch.zeros(n, dtype=torch.bool, device=pool_before.device)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        a = pool_before[r0:r1].view(torch.int32).flatten(1)
        b = pool_after[r0:r1].view(torch.int32).flatten(1)
        changed[r0:r1] = (a != b).any(dim=1)
    stray = torch.nonzero(changed & ~written).flatten().tolist()
    assert not stray, f"rows modified that the call does not write: {stray[:10]}"


def _host_out(out):
    return out.detach().to("cpu").to(torch.float64).numpy()


def _batch_bounds(w, trace, batch, ref_shape):
    """(output bound for the batch's token rows, {written row: state bound}) from one batch's trace."""
    out_b, seq_b = qdq_bounds(w, trace, batch)
    full = np.zeros(ref_shape)
    for t, bnd in out_b.items():
        full[t] = bnd
    state_bound = {row: seq_b[b][i] for b in batch if b in seq_b for i, row in written_rows(w, b)}
    return full, state_bound


# threads that run the oracle on batches of sequences side by side (NumPy releases the interpreter lock
# inside its large element-wise operations); every batch is checked on its own and the results are merged
# in batch order
CHECK_THREADS = max(1, min(8, len(os.sched_getaffinity(0))))


def _check_batches(w, seq_list, before, got_state, host_out, report, totals, qdq_precision, over, per_row=None):
    """Run the oracle one batch of sequences at a time on the pre-call rows ``before`` {row: array} and
    compare the GPU's outputs and written states (``got_state(rows)`` -> {row: float64 state}).
    ``per_row(row, ref_state, stable, totals)`` adds checks of a written row (packed pools).  Returns the
    written rows."""
    qdq = bool(w.options.get("qdq"))

    def check(batch):
        rep, tot = Report(), Totals()
        reads_b, _ = rows_for(w, batch)
        before_b = {r: np.asarray(before[r], dtype=np.float64) for r in reads_b}
        trace = {} if qdq else None
        ref_out, ref_written = oracle_call(w, before_b, seqs=batch, trace=trace, qdq_precision=qdq_precision, **over)
        trows = token_rows(w, batch)
        bound, state_bound, frows, stable = None, None, None, True
        if qdq:
            full, state_bound = _batch_bounds(w, trace, batch, ref_out.shape)
            bound = full[trows]
            frows = flip_rows(w, trace, batch)
            stable = frows is None
        del trace
        if len(trows):
            compare_outputs(host_out, ref_out, w, trows, rep, tot, qdq_bound=bound)
        got = got_state(list(ref_written))
        compare_states(got, ref_written, rep, tot, qdq_bound=state_bound, layout=w.state_layout,
                       codec=w.options.get("qdq"), block_v=w.options.get("block_v", 64), flip_rows=frows)
        if per_row is not None:
            for row, ref in ref_written.items():
                per_row(row, ref, stable, tot)
        return rep, tot, set(ref_written)

    batches = list(seq_batches(w, seq_list, 64 if qdq else 1024))
    written = set()
    if CHECK_THREADS == 1 or len(batches) == 1:
        results = map(check, batches)
    else:
        pool = concurrent.futures.ThreadPoolExecutor(CHECK_THREADS)
        results = pool.map(check, batches)
    try:
        for rep, tot, wr in results:
            report.merge(rep)
            totals.merge(tot)
            written.update(wr)
    finally:
        if not (CHECK_THREADS == 1 or len(batches) == 1):
            pool.shutdown(cancel_futures=True)
    return written


def run_and_check(w, seqs=None, report=None, pool=None, snapshot=True, qdq_precision="float64", **over):
    """Full parity check of workload ``w``: GPU call vs oracle on the sequences ``seqs`` (all if None).

    The oracle decides the state rounding in ``qdq_precision`` (float64 by default; float32 compares the
    code decisions taken in the kernel's own precision)."""
    report = report if report is not None else Report()
    totals = Totals()
    d = device_inputs(w)
    if pool is None:
        pool = wl.make_pool(w, "cuda")
    all_reads, all_writes = rows_for(w)
    seq_list = list(range(w.B)) if seqs is None else list(seqs)
    reads, writes = rows_for(w, seq_list)
    before = gather_rows(pool, reads, torch.float32)
    snap = pool.clone() if snapshot else None
    out = gpu_call(w, pool, d, **over)
    torch.cuda.synchronize()
    host_out = _host_out(out)
    after = gather_rows(pool, writes, torch.float32)
    written = _check_batches(w, seq_list, before, lambda rows: {r: after[r].astype(np.float64) for r in rows},
                             host_out, report, totals, qdq_precision, over)
    check_output_l2(w, report, totals)
    check_flip_rate(report, totals)
    assert sorted(written) == sorted(set(writes))
    if snap is not None:
        check_untouched(snap, pool, all_writes)
    return report, out, pool


# ---------------------------------------------------------------- packed int8_hadamard32 pools

def _is_fp8(w):
    return w.options.get("qdq") == "fp8_e4m3_tile"


def _to_layout(x, w):
    """Logical [..., K, V] -> the pool layout's order (V_FIRST: [..., V, K]); its own inverse."""
    return x if w.state_layout == "K_FIRST" else np.swapaxes(x, -1, -2)


def packed_bytes(w):
    """Bytes per (row, head) of a packed pool for workload ``w`` (codec or fp8 tiles)."""
    if _is_fp8(w):
        return e4m3.fp8_tile_bytes(w.K, w.V, w.options.get("block_v", 64))
    return ohad.packed_tile_bytes(w.K, w.V)


def make_packed_pool(w, device="cuda", rows=None):
    """Packed pool [rows, HV, tile bytes] for workload ``w`` (codec: K_FIRST; fp8 tiles: either layout): the
    oracle's encoding of make_pool's fp32 states for ``rows`` (all if None); the other rows hold random codes
    with positive scales."""
    K, V, HV, n = w.K, w.V, w.HV, w.num_rows
    fp8 = _is_fp8(w)
    bv = w.options.get("block_v", 64)
    assert packed_bytes(w) == (rsd.fp8_tile_bytes(K, V, bv) if fp8 else rsd.packed_tile_bytes(K, V))
    packed = wl.random_packed_pool(w, device)
    rows = list(range(n)) if rows is None else sorted(set(rows))
    if rows:
        fp32 = wl.make_pool(w, device)
        for r0 in range(0, len(rows), 64):
            part = rows[r0:r0 + 64]
            idx = torch.tensor(part, dtype=torch.int64, device=device)
            tiles = fp32.index_select(0, idx).cpu().numpy().astype(np.float64)
            if fp8:
                code, scale = e4m3.tile_encode(_to_layout(tiles, w).reshape(-1, K, V), bv, "float32")
                t = e4m3.pack_fp8_tiles(code.reshape(len(part), HV, K, V), scale.reshape(len(part), HV, V // bv),
                                        w.state_layout, bv)
            else:
                code, scale = ohad.int8_hadamard32_encode(tiles.reshape(-1, K, V), "float32")
                t = ohad.pack_tiles(code.reshape(len(part), HV, K, V), scale.reshape(len(part), HV, K, V // 32))
            packed[idx] = torch.from_numpy(t).to(device)
        del fp32
    return packed


def gather_packed(pool, rows, K, V):
    """{row: (codes int8 [HV, K, V], scales [HV, K, V / 32])} read back from a packed codec pool."""
    rows = sorted(set(rows))
    if not rows:
        return {}
    t = pool.index_select(0, torch.tensor(rows, dtype=torch.int64, device=pool.device)).cpu().numpy()
    return {r: ohad.unpack_tiles(t[i], K, V) for i, r in enumerate(rows)}


def gather_fp8(pool, rows, w):
    """{row: (E4M3 bytes [HV, K, V] in logical order, tile scales [HV, V / block_v])} of a packed fp8 pool."""
    rows = sorted(set(rows))
    if not rows:
        return {}
    bv = w.options.get("block_v", 64)
    t = pool.index_select(0, torch.tensor(rows, dtype=torch.int64, device=pool.device)).cpu().numpy()
    return {r: e4m3.unpack_fp8_tiles(t[i], w.K, w.V, w.state_layout, bv) for i, r in enumerate(rows)}


def decode_fp8(codes, scales, w):
    """The fp64 state, in the pool layout's order, that E4M3 bytes and tile scales stand for."""
    return _to_layout(e4m3.tile_decode(codes, scales, w.options.get("block_v", 64)), w)


class _Lazy(dict):
    """{row: value} computed on first access from fn(row) (decoded packed tiles, one batch at a time)."""

    def __init__(self, fn):
        super().__init__()
        self.fn = fn

    def __missing__(self, row):
        return self.fn(row)


def run_and_check_packed(w, seqs=None, report=None, pool=None, qdq_precision="float64", **over):
    """Parity of a call on a packed pool: outputs as for the codec on fp32 states; the written tiles,
    decoded, as the codec's states; their codes and scales against the oracle's encoding of its final
    states (at the oracle's decision precision); every other byte of the pool unchanged."""
    if _is_fp8(w):
        return _run_and_check_fp8(w, seqs, report, pool, qdq_precision, **over)
    assert w.options.get("qdq") == "int8_hadamard32" and w.state_layout == "K_FIRST"
    report = report if report is not None else Report()
    totals = Totals()
    d = device_inputs(w)
    all_reads, all_writes = rows_for(w)
    seq_list = list(range(w.B)) if seqs is None else list(seqs)
    reads, writes = rows_for(w, seq_list)
    if pool is None:
        pool = make_packed_pool(w, "cuda", rows=all_reads)
    raw_before = gather_packed(pool, reads, w.K, w.V)
    before = _Lazy(lambda r: ohad.int8_hadamard32_decode(*raw_before[r]))
    snap = pool.clone()
    out = gpu_call(w, pool, d, **over)
    torch.cuda.synchronize()
    host_out = _host_out(out)
    got = gather_packed(pool, writes, w.K, w.V)

    def per_row(r, ref, stable, totals):
        code_e, scale_e = ohad.int8_hadamard32_encode(ref, qdq_precision)
        code_g, scale_g = got[r]
        dc = np.abs(code_g.astype(np.int32) - code_e.astype(np.int32))
        # codes of a group whose scale agrees differ by at most two: a code rounded the other way at one
        # token is carried into the next by the decay (alpha ~ 1), and that token's own rounding can land
        # one more step away; a group whose scale moved (an earlier flip changed its amax) is held by the
        # scale checks below, every group by the element-wise bounds above
        same = np.abs(scale_g - scale_e) <= 1e-5 * np.abs(scale_e)
        dcg = dc.reshape(dc.shape[0], dc.shape[1], dc.shape[2] // 32, 32).max(axis=-1)
        assert not stable or dcg[same].max(initial=0) <= 2, f"row {r}: a code differs by {dcg[same].max()}"
        pos = scale_e > 0
        rel = np.abs(scale_g[pos] - scale_e[pos]) / scale_e[pos]
        assert np.all(scale_g[~pos] < 1e-30)
        if stable:
            totals.code_flips += int(np.sum(dc))
            totals.codes += dc.size
            totals.worst_scale = max(totals.worst_scale, float(rel.max()) if rel.size else 0.0)
            totals.off_scales += int(np.sum(rel > 1e-5))
            totals.groups += int(rel.size)

    written = _check_batches(w, seq_list, before,
                             lambda rows: {r: ohad.int8_hadamard32_decode(*got[r]) for r in rows},
                             host_out, report, totals, qdq_precision, over, per_row=per_row)
    check_output_l2(w, report, totals)
    check_flip_rate(report, totals, "rotated coordinates")
    report.add("packed_code_flip_frac", totals.code_flips / max(totals.codes, 1))
    report.add("packed_scale_max_rel", totals.worst_scale)
    if totals.codes:
        assert totals.code_flips / totals.codes < FLIP_RATE, f"{totals.code_flips} of {totals.codes} codes differ"
        # a code rounded the other way at an earlier token moves that group's next amax (so its scale)
        # by up to about a step, 1/127 of it; such groups must stay rare, like the flips themselves
        assert totals.worst_scale < 1e-2, f"scale relative error {totals.worst_scale}"
        assert totals.off_scales <= max(1, totals.groups // 100), \
            f"{totals.off_scales} of {totals.groups} scales differ by more than 1e-5"
    assert sorted(written) == sorted(set(writes))
    check_untouched(snap, pool, all_writes)
    return report, out, pool


def _run_and_check_fp8(w, seqs, report, pool, qdq_precision="float64", **over):
    """run_and_check_packed for fp8 tiles: outputs and decoded states within the fp8 QDQ bounds; the written
    bytes and tile scales against the oracle's encoding of its final states; a non-zero tile's largest code is
    +-448 (its scale is its amax / 448), an all-zero tile's scale is 0; every other byte unchanged."""
    report = report if report is not None else Report()
    totals = Totals()
    d = device_inputs(w)
    all_reads, all_writes = rows_for(w)
    seq_list = list(range(w.B)) if seqs is None else list(seqs)
    reads, writes = rows_for(w, seq_list)
    if pool is None:
        pool = make_packed_pool(w, "cuda", rows=all_reads)
    bv = w.options.get("block_v", 64)
    raw_before = gather_fp8(pool, reads, w)
    before = _Lazy(lambda r: decode_fp8(*raw_before[r], w))
    snap = pool.clone()
    out = gpu_call(w, pool, d, **over)
    torch.cuda.synchronize()
    host_out = _host_out(out)
    got = gather_fp8(pool, writes, w)
    table = e4m3.e4m3_table()

    def per_row(r, ref, stable, totals):
        code_e, scale_e = e4m3.tile_encode(_to_layout(ref, w), bv, qdq_precision)
        code_g, scale_g = got[r]
        vg, ve = table[code_g], table[code_e]
        assert np.all(np.isfinite(vg)), f"row {r}: a NaN code was stored"
        zero = scale_e == 0
        assert np.all(scale_g[zero] == 0), f"row {r}: an all-zero tile stored a non-zero scale"
        peak = np.abs(vg).reshape(vg.shape[0], w.K, w.V // bv, bv).max(axis=(1, 3))
        assert np.all(peak[~zero] == 448.0), f"row {r}: a non-zero tile's largest code is not 448"
        # the decoded values are held to the propagated bounds: a code rounded the other way at one
        # token moves the whole key row's update at the next, which for an element near zero can be many
        # of its own (small) steps; here only how often codes differ is checked
        if stable:
            off = vg != ve
            totals.code_flips += int(np.sum(off))
            totals.codes += off.size
            rel = np.abs(scale_g[~zero] - scale_e[~zero]) / scale_e[~zero]
            totals.worst_scale = max(totals.worst_scale, float(rel.max()) if rel.size else 0.0)

    written = _check_batches(w, seq_list, before,
                             lambda rows: {r: decode_fp8(*got[r], w) for r in rows},
                             host_out, report, totals, qdq_precision, over, per_row=per_row)
    check_output_l2(w, report, totals)
    check_flip_rate(report, totals)
    report.add("fp8_code_flip_frac", totals.code_flips / max(totals.codes, 1))
    report.add("fp8_scale_max_rel", totals.worst_scale)
    if totals.codes:
        assert totals.code_flips / totals.codes < FLIP_RATE, f"{totals.code_flips} of {totals.codes} codes differ"
        # a code rounded the other way at an earlier token moves the tile's later amax by a fraction of
        # a step
        assert totals.worst_scale < 1e-2, f"scale relative error {totals.worst_scale}"
    assert sorted(written) == sorted(set(writes))
    check_untouched(snap, pool, all_writes)
    return report, out, pool

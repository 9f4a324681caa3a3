"""Seeded synthetic inputs for the decode workloads.

This module draws random inputs and builds index tables; it holds none of
the decode arithmetic.  Tests, the bench and the smoke run feed the same
draws to the HIP library and to the CPU oracle.

Recipe (fixed draw order, numpy ``Generator(PCG64(seed))``):
lengths -> page table -> q -> k -> v -> gate input (a or raw_gate) ->
beta input (b or beta_logits) -> dt_bias -> A_log -> slot choice.
Values are drawn in float32 and cast to the I/O dtype with round-to-nearest-
even (torch CPU ``.to(bfloat16)``); the oracle receives the cast values.
The state pool is filled on its own device with ``torch.Generator``
(N(0, 0.05)) from ``seed + 1``; the oracle reads back the rows it needs.

Distributions: q, k, v, a, b, raw_gate, beta_logits ~ N(0, 1);
dt_bias ~ U(-1, 1); A_log (a_log) ~ U(0, ln 16).
"""
import math
from dataclasses import dataclass, field

import numpy as np
import torch

K_FIRST = "K_FIRST"
V_FIRST = "V_FIRST"


@dataclass
class Workload:
    kind: str                         # "gdn_pooled" | "kda_pooled" | "gdn_paged"
    name: str
    B: int
    HK: int
    HV: int
    K: int
    V: int
    io_dtype: torch.dtype
    out_dtype: torch.dtype
    state_layout: str
    num_rows: int                     # slots (pooled) or pages (paged)
    inputs: dict = field(default_factory=dict)   # CPU tensors
    options: dict = field(default_factory=dict)  # beta_mode, qdq, block_v, ...
    pool_seed: int = 0
    pool_zero: bool = False
    chunked: bool = False             # paged suffixes through the chunked prefill entry point

    @property
    def T(self):
        return self.inputs["q"].shape[0]

    def pool_shape(self):
        tail = (self.K, self.V) if self.state_layout == K_FIRST else (self.V, self.K)
        return (self.num_rows, self.HV) + tail

    def read_rows(self):
        """Pool rows read by the call (sorted unique), single-token paged or pooled."""
        if self.kind in ("gdn_paged", "kda_paged"):
            ind = self.inputs["page_indices"].numpy()
            ptr = self.inputs["page_indptr"].numpy()
            lpl = self.inputs["last_page_len"].numpy()
            rows = [int(ind[ptr[b + 1] - 2]) if lpl[b] == 1 else int(ind[ptr[b + 1] - 1])
                    for b in range(self.B)]
        else:
            rows = [int(s) for s in self.inputs["state_indices"].numpy()]
        return sorted(set(rows))

    def tokens(self):
        return self.T


def make_pool(w, device, dtype=torch.float32):
    """The state pool of workload ``w`` on ``device``: N(0, 0.05) or zeros."""
    shape = w.pool_shape()
    if w.pool_zero:
        return torch.zeros(shape, dtype=dtype, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(w.pool_seed)
    pool = torch.empty(shape, dtype=dtype, device=device)
    pool.normal_(0.0, 0.05, generator=g)
    return pool


def device_inputs(w, device="cuda"):
    """The workload's input tensors on ``device`` (index arrays and activations alike)."""
    return {k: (None if v is None else v.to(device)) for k, v in w.inputs.items() if k != "prefix_lengths"}


def random_packed_pool(w, device):
    """A uint8 packed pool [rows, HV, tile bytes] of seeded random codes with positive scales, for the
    workload's state quantisation (qdq 'fp8_e4m3_tile' or 'int8_hadamard32'); fp8 NaN codes (0x7f,
    0xff) are replaced by +-448 (0x7e, 0xfe)."""
    from . import _binding as bnd
    K, V, HV, n = w.K, w.V, w.HV, w.num_rows
    fp8 = w.options.get("qdq") == "fp8_e4m3_tile"
    bv = w.options.get("block_v", 64)
    tb = bnd.fp8_tile_bytes(K, V, bv) if fp8 else bnd.packed_tile_bytes(K, V)
    nsc = V // bv if fp8 else K * V // 32
    g = torch.Generator(device=device)
    g.manual_seed(w.pool_seed + 7)
    packed = torch.randint(0, 256, (n, HV, tb), dtype=torch.uint8, device=device, generator=g)
    if fp8:
        c = packed[:, :, :K * V]
        packed[:, :, :K * V] = torch.where((c & 0x7F) == 0x7F, c ^ 1, c)
    sc = torch.empty((n, HV, nsc), dtype=torch.float32, device=device).uniform_(1e-3, 1e-2, generator=g)
    packed[:, :, K * V:K * V + 4 * nsc] = sc.view(torch.uint8)
    return packed


def call_options(w, over, drop=()):
    """The workload's binding options (``page_size`` removed), updated by ``over``, without ``drop``."""
    o = dict(w.options)
    o.pop("page_size", None)
    o.update(over)
    for k in drop:
        o.pop(k, None)
    return o


def run(w, pool, d, out=None, **over):
    """Run workload ``w`` on the device pool through the binding (inputs ``d`` from device_inputs).
    Returns ``out``."""
    import recurrent_state_decode_amd as rsd
    common = dict(state_layout=w.state_layout, out_dtype=w.out_dtype, **call_options(w, over))
    ps = w.options.get("page_size")
    if w.kind == "gdn_pooled":
        return rsd.gdn_decode_pooled(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                     d["cu_seqlens"], d["state_indices"], pool, out, **common)
    if w.kind == "kda_pooled":
        return rsd.kda_decode_pooled(d["q"], d["k"], d["v"], d["raw_gate"], d["beta_logits"], d["a_log"],
                                     d["dt_bias"], d["cu_seqlens"], d["state_indices"], pool, out, **common)
    table = (d["page_indices"], d["page_indptr"], d["last_page_len"])
    if w.kind == "gdn_paged":
        return rsd.gdn_decode_paged(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], *table,
                                    pool, out, **common)
    if w.kind == "kda_paged":
        return rsd.kda_decode_paged(d["q"], d["k"], d["v"], d["raw_gate"], d["beta_logits"], d["a_log"],
                                    d["dt_bias"], *table, pool, out, **common)
    if w.kind == "gdn_paged_varlen" and w.chunked:
        o = {k2: v2 for k2, v2 in common.items() if k2 in ("scale", "use_qk_l2norm", "beta_mode", "state_layout",
                                                            "out_dtype")}
        return rsd.gdn_prefill_paged(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                     d["cu_seqlens"], *table, ps, pool, out, **o)
    if w.kind == "gdn_paged_varlen":
        return rsd.gdn_decode_paged_varlen(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                           d["cu_seqlens"], *table, ps, pool, out, **common)
    if w.kind == "kda_paged_varlen" and w.chunked:
        o = {k2: v2 for k2, v2 in common.items() if k2 in ("scale", "use_qk_l2norm", "beta_mode", "state_layout",
                                                            "out_dtype", "gate_mode")}
        return rsd.kda_prefill_paged(d["q"], d["k"], d["v"], d["raw_gate"], d["beta_logits"], d["a_log"],
                                     d["dt_bias"], d["cu_seqlens"], *table, ps, pool, out, **o)
    if w.kind == "kda_paged_varlen":
        return rsd.kda_decode_paged_varlen(d["q"], d["k"], d["v"], d["raw_gate"], d["beta_logits"], d["a_log"],
                                           d["dt_bias"], d["cu_seqlens"], *table, ps, pool, out, **common)
    raise ValueError(w.kind)


def _cast(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _uniform(rng, lo, hi, shape):
    return rng.uniform(lo, hi, shape).astype(np.float32)


def lengths_to_cu(lengths):
    return torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)


def gdn_pooled(B, HK, HV, K, V, *, lengths=None, num_slots=None, state_layout=K_FIRST,
               io_dtype=torch.bfloat16, out_dtype=None, seed=0, name="gdn_pooled", zero_state=False,
               **options):
    """Pooled GDN decode; ``lengths`` None means one token per sequence (cu_seqlens = NULL)."""
    rng = np.random.default_rng(seed)
    T = B if lengths is None else int(np.sum(lengths))
    num_slots = num_slots or B
    inp = {}
    inp["q"] = _cast(_normal(rng, (T, HK, K)), io_dtype)
    inp["k"] = _cast(_normal(rng, (T, HK, K)), io_dtype)
    inp["v"] = _cast(_normal(rng, (T, HV, V)), io_dtype)
    inp["a"] = _cast(_normal(rng, (T, HV)), io_dtype)
    inp["b"] = _cast(_normal(rng, (T, HV)), io_dtype)
    inp["dt_bias"] = _cast(_uniform(rng, -1, 1, (HV,)), torch.float32)
    inp["A_log"] = _cast(_uniform(rng, 0, math.log(16), (HV,)), torch.float32)
    inp["state_indices"] = torch.tensor(rng.permutation(num_slots)[:B], dtype=torch.int32)
    inp["cu_seqlens"] = None if lengths is None else lengths_to_cu(lengths)
    return Workload("gdn_pooled", name, B, HK, HV, K, V, io_dtype, out_dtype or io_dtype, state_layout,
                    num_slots, inp, options, pool_seed=seed + 1, pool_zero=zero_state)


def kda_pooled(B, HK, HV, K, V, *, lengths, num_slots=None, state_layout=V_FIRST,
               io_dtype=torch.bfloat16, out_dtype=None, seed=0, name="kda_pooled", zero_state=False,
               **options):
    """Pooled KDA decode over varlen suffixes given by ``lengths``."""
    rng = np.random.default_rng(seed)
    T = int(np.sum(lengths))
    num_slots = num_slots or B
    inp = {}
    inp["q"] = _cast(_normal(rng, (T, HK, K)), io_dtype)
    inp["k"] = _cast(_normal(rng, (T, HK, K)), io_dtype)
    inp["v"] = _cast(_normal(rng, (T, HV, V)), io_dtype)
    inp["raw_gate"] = _cast(_normal(rng, (T, HV, K)), io_dtype)
    inp["beta_logits"] = _cast(_normal(rng, (T, HV)), io_dtype)
    inp["dt_bias"] = _cast(_uniform(rng, -1, 1, (HV, K)), torch.float32)
    inp["a_log"] = _cast(_uniform(rng, 0, math.log(16), (HV,)), torch.float32)
    inp["state_indices"] = torch.tensor(rng.permutation(num_slots)[:B], dtype=torch.int32)
    inp["cu_seqlens"] = lengths_to_cu(lengths)
    return Workload("kda_pooled", name, B, HK, HV, K, V, io_dtype, out_dtype or io_dtype, state_layout,
                    num_slots, inp, options, pool_seed=seed + 1, pool_zero=zero_state)


def build_page_table(prefix_lengths, page_size, share_frac, rng, force_shared_new_page=8, new_tokens=None):
    """CSR page table for sequences that append ``new_tokens`` (default 1) to ``prefix_lengths`` tokens.

    Sequence b holds n_b = L_b + new_b tokens on ceil(n_b / page_size) pages;
    ``last_page_len`` = n_b - page_size * (pages - 1).  A fraction
    ``share_frac`` of the pages that lie entirely inside the prefix is
    aliased to the page with the same position in another sequence whose
    page there also lies inside its prefix, as shared prefixes are; pages
    that hold new tokens are never shared, so no call writes a shared page.
    Some sequences whose state is read from a full page (the prefix ends on a
    page boundary) get a shared page there on purpose.  Page ids are
    compacted to 0..num_pages-1 in a random physical order.
    Returns (page_indices int64 [nnz], page_indptr int64 [B+1],
    last_page_len int64 [B], num_pages).
    """
    L = np.asarray(prefix_lengths, dtype=np.int64)
    new = np.ones_like(L) if new_tokens is None else np.asarray(new_tokens, dtype=np.int64)
    n = L + new
    P = -(-n // page_size)
    last_len = n - page_size * (P - 1)
    full_prefix = L // page_size              # pages 0 .. full_prefix-1 hold prefix tokens only
    B = len(L)
    uid = [list(range(int(s), int(s + p))) for s, p in zip(np.concatenate([[0], np.cumsum(P)[:-1]]), P)]
    full = [(b, j) for b in range(B) for j in range(int(full_prefix[b]))]
    n_share = int(round(share_frac * len(full)))
    chosen = set()
    # sequences whose state is read from a full page: share that page first
    boundary = [b for b in range(B) if L[b] % page_size == 0 and L[b] >= page_size]
    rng.shuffle(boundary)
    for b in boundary[:force_shared_new_page]:
        chosen.add((b, int(full_prefix[b]) - 1))
    order = rng.permutation(len(full))
    for i in order:
        if len(chosen) >= n_share:
            break
        chosen.add(full[i])
    # targets: same page position in another sequence, inside its prefix and not itself aliased
    for (b, j) in sorted(chosen):
        cands = np.nonzero((full_prefix > j) & (np.arange(B) != b))[0]
        cands = [c for c in cands if (int(c), j) not in chosen]
        if not cands:
            continue
        src = int(cands[rng.integers(len(cands))])
        uid[b][j] = uid[src][j]
    used = sorted({p for pages in uid for p in pages})
    phys = rng.permutation(len(used))
    remap = {old: int(phys[i]) for i, old in enumerate(used)}
    indices = np.array([remap[p] for pages in uid for p in pages], dtype=np.int64)
    indptr = np.concatenate([[0], np.cumsum(P)]).astype(np.int64)
    return indices, indptr, last_len.astype(np.int64), len(used)


def paged(kind, B, HK, HV, K, V, *, prefix_lengths=None, max_prefix=2048, page_size=16, share_frac=0.1,
          suffix_lengths=None, state_layout=V_FIRST, io_dtype=torch.bfloat16, out_dtype=None,
          index_dtype=torch.int64, seed=0, name=None, chunked=False, **options):
    """GDN ("gdn") or KDA ("kda") decode on a CSR-paged pool with shared prefix pages.

    ``suffix_lengths`` None: one decoded token per sequence (token b belongs to
    sequence b); otherwise each sequence appends that many tokens and the
    inputs hold them in cu_seqlens order.
    """
    rng = np.random.default_rng(seed)
    if prefix_lengths is None:
        prefix_lengths = rng.integers(1, max_prefix + 1, B)
    ind, ptr, lpl, num_pages = build_page_table(prefix_lengths, page_size, share_frac, rng,
                                                new_tokens=suffix_lengths)
    T = B if suffix_lengths is None else int(np.sum(suffix_lengths))
    inp = {}
    inp["q"] = _cast(_normal(rng, (T, HK, K)), io_dtype)
    inp["k"] = _cast(_normal(rng, (T, HK, K)), io_dtype)
    inp["v"] = _cast(_normal(rng, (T, HV, V)), io_dtype)
    if kind == "kda":
        inp["raw_gate"] = _cast(_normal(rng, (T, HV, K)), io_dtype)
        inp["beta_logits"] = _cast(_normal(rng, (T, HV)), io_dtype)
        inp["dt_bias"] = _cast(_uniform(rng, -1, 1, (HV, K)), torch.float32)
        inp["a_log"] = _cast(_uniform(rng, 0, math.log(16), (HV,)), torch.float32)
    else:
        inp["a"] = _cast(_normal(rng, (T, HV)), io_dtype)
        inp["b"] = _cast(_normal(rng, (T, HV)), io_dtype)
        inp["dt_bias"] = _cast(_uniform(rng, -1, 1, (HV,)), torch.float32)
        inp["A_log"] = _cast(_uniform(rng, 0, math.log(16), (HV,)), torch.float32)
    inp["page_indices"] = torch.from_numpy(ind).to(index_dtype)
    inp["page_indptr"] = torch.from_numpy(ptr).to(index_dtype)
    inp["last_page_len"] = torch.from_numpy(lpl).to(index_dtype)
    inp["prefix_lengths"] = torch.from_numpy(np.asarray(prefix_lengths, dtype=np.int64))
    if suffix_lengths is not None:
        inp["cu_seqlens"] = lengths_to_cu(suffix_lengths)
    opts = dict(page_size=page_size, **options)
    wkind = ("kda" if kind == "kda" else "gdn") + ("_paged" if suffix_lengths is None else "_paged_varlen")
    if chunked and not wkind.endswith("_paged_varlen"):
        raise ValueError("the chunked prefill takes suffixes on a paged pool")
    return Workload(wkind, name or wkind, B, HK, HV, K, V, io_dtype, out_dtype or io_dtype, state_layout,
                    num_pages, inp, opts, pool_seed=seed + 1, chunked=chunked)


def gdn_paged(B, HK, HV, K, V, **kw):
    """One decoded token per sequence, GDN, on a CSR-paged pool with shared prefix pages."""
    kw.setdefault("name", "gdn_paged")
    return paged("gdn", B, HK, HV, K, V, **kw)


# ------------------------------------------------------------------ named workloads

def tiny_gdn(seed=1001):
    """B=1, HK=HV=1, K=V=16, 8 tokens, fp32 everywhere, zero initial state in a 1-slot pool."""
    return gdn_pooled(1, 1, 1, 16, 16, lengths=[8], num_slots=1, state_layout=K_FIRST,
                      io_dtype=torch.float32, seed=seed, name="tiny_gdn_b1_k16_t8_f32", zero_state=True)


def pooled_gdn_b64(seed=1002):
    """B=64 single-token GDN decode, HK=16, HV=32, K=V=128, bf16 I/O, 256-slot K_FIRST pool."""
    return gdn_pooled(64, 16, 32, 128, 128, lengths=None, num_slots=256, state_layout=K_FIRST,
                      seed=seed, name="pooled_gdn_b64_hv32_k128")


def pooled_kda_varlen_b128(seed=1003):
    """B=128 KDA varlen decode, suffixes U{1..8}, HK=HV=32, K=V=128, bf16 I/O, 512-slot V_FIRST pool."""
    rng = np.random.default_rng(seed + 500)
    lengths = rng.integers(1, 9, 128)
    return kda_pooled(128, 32, 32, 128, 128, lengths=lengths, num_slots=512, state_layout=V_FIRST,
                      seed=seed, name="pooled_kda_varlen_b128_hv32_k128")


def paged_gdn_b256(seed=1004, state_layout=V_FIRST, index_dtype=torch.int64):
    """B=256 paged GDN decode, HK=16, HV=32, K=V=128, page_size 16, prefixes U{1..2048}, 10% shared."""
    return gdn_paged(256, 16, 32, 128, 128, max_prefix=2048, page_size=16, share_frac=0.1,
                     state_layout=state_layout, index_dtype=index_dtype, seed=seed,
                     name="paged_gdn_b256_hv32_k128_ps16")


def fp8_qdq_gdn_b512(seed=1005):
    """B=512 GDN decode with 4-token suffixes and fp8 e4m3 tile QDQ (block_v=64), 1024-slot pool."""
    return gdn_pooled(512, 16, 32, 128, 128, lengths=np.full(512, 4), num_slots=1024,
                      state_layout=K_FIRST, seed=seed, name="fp8_qdq_gdn_b512_t4_hv32_k128",
                      qdq="fp8_e4m3_tile", block_v=64)


def paged_gdn_prefill_b16_t1024(seed=1009, state_layout=V_FIRST, index_dtype=torch.int64):
    """Chunked prefill on the paged pool: 16 sequences each append 1024 tokens after a prefix U{1..2048}."""
    return paged("gdn", 16, 16, 32, 128, 128, max_prefix=2048, page_size=16, share_frac=0.1,
                 suffix_lengths=np.full(16, 1024), state_layout=state_layout, index_dtype=index_dtype, seed=seed,
                 name="paged_gdn_prefill_b16_t1024_hv32_k128_ps16", chunked=True)


def paged_kda_prefill_b16_t1024(seed=1010, state_layout=V_FIRST, index_dtype=torch.int64):
    """The chunked-prefill shape with KDA gating: 16 sequences x 1024 tokens, HK=HV=32, K=V=128, page 16."""
    return paged("kda", 16, 32, 32, 128, 128, max_prefix=2048, page_size=16, share_frac=0.1,
                 suffix_lengths=np.full(16, 1024), state_layout=state_layout, index_dtype=index_dtype, seed=seed,
                 name="paged_kda_prefill_b16_t1024_hv32_k128_ps16", chunked=True)


def int8h32_gdn_b512(seed=1008):
    """The B=512, 4-token pooled GDN workload with the int8_hadamard32 state codec instead of fp8 tiles."""
    return gdn_pooled(512, 16, 32, 128, 128, lengths=np.full(512, 4), num_slots=1024,
                      state_layout=K_FIRST, seed=seed, name="int8h32_gdn_b512_t4_hv32_k128",
                      qdq="int8_hadamard32", block_v=64)


def paged_kda_b256(seed=1006, state_layout=V_FIRST, index_dtype=torch.int64):
    """The paged B=256 workload with KDA gating: HK=HV=32, raw_gate [B, 32, 128], dt_bias [32, 128]."""
    return paged("kda", 256, 32, 32, 128, 128, max_prefix=2048, page_size=16, share_frac=0.1,
                 state_layout=state_layout, index_dtype=index_dtype, seed=seed, name="paged_kda_b256_hv32_k128_ps16")


def paged_gdn_varlen_b256_t4(seed=1007, state_layout=V_FIRST, index_dtype=torch.int64):
    """The paged B=256 workload decoding 4 tokens per sequence (pages filled mid-suffix are written)."""
    return paged("gdn", 256, 16, 32, 128, 128, max_prefix=2048, page_size=16, share_frac=0.1,
                 suffix_lengths=np.full(256, 4), state_layout=state_layout, index_dtype=index_dtype, seed=seed,
                 name="paged_gdn_varlen_b256_t4_hv32_k128_ps16")


NAMED = {
    "tiny_gdn": tiny_gdn,
    "pooled_gdn_b64": pooled_gdn_b64,
    "pooled_kda_varlen_b128": pooled_kda_varlen_b128,
    "paged_gdn_b256": paged_gdn_b256,
    "fp8_qdq_gdn_b512": fp8_qdq_gdn_b512,
    "paged_kda_b256": paged_kda_b256,
    "paged_gdn_varlen_b256_t4": paged_gdn_varlen_b256_t4,
    "int8h32_gdn_b512": int8h32_gdn_b512,
    "paged_gdn_prefill_b16_t1024": paged_gdn_prefill_b16_t1024,
    "paged_kda_prefill_b16_t1024": paged_kda_prefill_b16_t1024,
}

"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on seeded inputs.

Every case also checks the index work exactly: the rows written are the
call's write rows and every other pool byte is unchanged.
"""
import numpy as np
import pytest
import torch

from recurrent_state_decode_amd import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu


def _report(name, rep):
    print(f"[parity] {name}: {rep}", flush=True)


# ---------------------------------------------------------------- the five workloads at full size

def test_tiny_gdn_b1_k16_t8_f32():
    w = wl.tiny_gdn()
    rep, _, _ = P.run_and_check(w)
    _report(w.name, rep)


def test_pooled_gdn_b64_hv32_k128():
    w = wl.pooled_gdn_b64()
    rep, _, _ = P.run_and_check(w)
    _report(w.name, rep)


def test_pooled_kda_varlen_b128_hv32_k128():
    w = wl.pooled_kda_varlen_b128()
    rep, _, _ = P.run_and_check(w)
    _report(w.name, rep)


@pytest.mark.parametrize("layout,idx", [("V_FIRST", torch.int64), ("K_FIRST", torch.int32)])
def test_paged_gdn_b256_hv32_k128(layout, idx):
    w = wl.paged_gdn_b256(state_layout=layout, index_dtype=idx)
    rep, _, _ = P.run_and_check(w)
    _report(f"{w.name}/{layout}/{idx}", rep)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_fp8_qdq_gdn_b512_t4(precision):
    """All 512 sequences.  float64: the oracle decides every code in float64 (the plain reading of the
    amax / 448 tile scale) and the kernel must stay within one E4M3 step per rounding; float32: the same
    comparison with the oracle deciding in the kernel's own precision, a diagnostic of how often the two
    sides' code decisions differ."""
    w = wl.fp8_qdq_gdn_b512()
    rep, _, _ = P.run_and_check(w, qdq_precision=precision)
    _report(f"{w.name}/{precision}", rep)


# ---------------------------------------------------------------- smaller cases: layouts, kinds, dtypes

LENS = [0, 1, 3, 0, 8, 9, 17, 2]       # empty suffixes, T = 1, a chunk boundary at 8, several chunks


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("hk", [2, 4])
def test_varlen_small(layout, kind, hk):
    mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
    w = mk(len(LENS), hk, 4, 128, 128, lengths=LENS, num_slots=11, state_layout=layout, seed=31)
    rep, _, _ = P.run_and_check(w)
    _report(f"varlen/{kind}/{layout}/hk{hk}", rep)


@pytest.mark.parametrize("io,out", [(torch.float32, torch.float32), (torch.bfloat16, torch.float32),
                                    (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_dtype_combinations(io, out, layout):
    w = wl.gdn_pooled(5, 1, 2, 128, 256, lengths=[2, 1, 0, 4, 1], num_slots=7, state_layout=layout,
                      io_dtype=io, out_dtype=out, seed=32)
    rep, _, _ = P.run_and_check(w)
    _report(f"dtypes/{io}/{out}/{layout}", rep)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_small_heads_k16_v32(layout):
    w = wl.gdn_pooled(3, 1, 3, 16, 32, lengths=[5, 0, 12], num_slots=4, state_layout=layout,
                      io_dtype=torch.float32, seed=33)
    rep, _, _ = P.run_and_check(w)
    _report(f"k16v32/{layout}", rep)


@pytest.mark.parametrize("opts", [dict(beta_mode="probability"), dict(use_qk_l2norm=False),
                                  dict(scale=0.37), dict(beta_mode="probability", use_qk_l2norm=False)])
def test_activation_options(opts):
    w = wl.gdn_pooled(4, 2, 4, 128, 128, lengths=[1, 3, 2, 1], num_slots=6, seed=34)
    if opts.get("beta_mode") == "probability":
        w.inputs["b"] = torch.rand(w.inputs["b"].shape, generator=torch.Generator().manual_seed(1)).to(w.io_dtype)
    rep, _, _ = P.run_and_check(w, **opts)
    _report(f"opts/{opts}", rep)


@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
@pytest.mark.parametrize("idx", [torch.int32, torch.int64])
def test_paged_small_page_boundaries(layout, idx):
    # page_size 4 puts many decoded tokens on both last_page_len == 1 (new page,
    # often with a shared previous page) and last_page_len == 4 (full page in place)
    w = wl.gdn_paged(48, 2, 4, 128, 128, max_prefix=40, page_size=4, share_frac=0.3, state_layout=layout,
                     index_dtype=idx, seed=35)
    lpl = w.inputs["last_page_len"].numpy()
    assert (lpl == 1).any() and (lpl == 4).any()
    rep, _, _ = P.run_and_check(w)
    _report(f"paged_small/{layout}/{idx}", rep)


# ---------------------------------------------------------------- fp8 tile QDQ variants

@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("extra", [dict(), dict(quantize_initial=True), dict(readout="stored")])
def test_qdq_variants(layout, kind, extra):
    mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
    w = mk(6, 2, 4, 128, 128, lengths=[4, 1, 0, 9, 2, 3], num_slots=8, state_layout=layout, seed=36,
           qdq="fp8_e4m3_tile", block_v=64, **extra)
    rep, _, _ = P.run_and_check(w)
    _report(f"qdq/{kind}/{layout}/{extra}", rep)


@pytest.mark.parametrize("qdq", ["fp8_e4m3_tile", "int8_hadamard32"])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_qdq_with_probability_beta_of_either_sign(qdq, kind):
    """beta_mode='probability' passes b as beta unchanged; with b ~ N(0, 1) beta takes both signs and
    values above 1, and the rounding errors must still stay within the bounds propagated with |beta|."""
    mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
    w = mk(8, 1, 2, 128, 128, lengths=[5, 1, 0, 8, 3, 2, 6, 4], num_slots=10, state_layout="K_FIRST", seed=41,
           qdq=qdq, block_v=64, beta_mode="probability")
    beta = w.inputs["b" if kind == "gdn" else "beta_logits"].float()
    assert bool((beta < 0).any()) and bool((beta > 1).any())
    rep, _, _ = P.run_and_check(w)
    _report(f"qdq_prob_beta/{qdq}/{kind}", rep)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"qdq_prob_beta_packed/{qdq}/{kind}", rep)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_qdq_rounding_matches_e4m3_grid_exactly(layout):
    """alpha = 1 and beta = 0 leave the state unchanged, so the stored state is the tile QDQ of the
    initial pool; each tile holds 448 so that its scale is exactly 1 and every code is
    decided on the value itself: midpoints, their neighbours and random values must round
    exactly as the OCP E4M3 nearest-even grid."""
    from oracle import e4m3
    B, HV, K, V = 4, 4, 128, 128
    w = wl.gdn_pooled(B, 1, HV, K, V, lengths=[1] * B, num_slots=B, state_layout=layout, seed=37,
                      io_dtype=torch.float32, qdq="fp8_e4m3_tile", block_v=64)
    w.inputs["a"] = torch.full((B, HV), -float("inf"))     # softplus(-inf) = 0 -> alpha = 1
    w.inputs["b"] = torch.zeros((B, HV))                   # beta = b = 0 (probability mode)
    w.options["beta_mode"] = "probability"
    grid = np.sort(e4m3.e4m3_table()[:127])
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9)), grid])
    rng = np.random.default_rng(38)
    n = B * HV * K * V
    fill = np.concatenate([vals, -vals, rng.uniform(-448, 448, n)])[:n].astype(np.float32)
    rng.shuffle(fill)
    logical = fill.reshape(B, HV, K, V)
    for h in range(HV):
        for j in range(0, V, 64):
            logical[:, h, 0, j] = 448.0
    tiles = logical if layout == "K_FIRST" else np.swapaxes(logical, -1, -2)
    pool = torch.from_numpy(np.ascontiguousarray(tiles)).cuda()
    rep, _, pool = P.run_and_check(w, pool=pool)
    got = pool.cpu().numpy()
    got_logical = got if layout == "K_FIRST" else np.swapaxes(got, -1, -2)
    assert np.array_equal(got_logical, e4m3.e4m3_round(logical.astype(np.float64)).astype(np.float32))
    _report(f"qdq_exact/{layout}", rep)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_qdq_tiny_tiles_use_the_amax_floor(layout):
    """A tile whose amax is below 2^-100 is rounded as if its amax were 2^-100 (the kernel's floor, so that
    448 / amax stays finite): with alpha = 1 and beta = 0 the stored state is exactly
    fp32(e4m3(x * 448 * 2^100) * fp32(2^-100 / 448)), every product in float32; an all-zero tile stays
    zero."""
    from oracle import e4m3
    B, HV, K, V = 4, 2, 128, 128
    w = wl.gdn_pooled(B, 1, HV, K, V, lengths=[1] * B, num_slots=B, state_layout=layout, seed=39,
                      io_dtype=torch.float32, qdq="fp8_e4m3_tile", block_v=64)
    w.inputs["a"] = torch.full((B, HV), -float("inf"))     # alpha = 1
    w.inputs["b"] = torch.zeros((B, HV))                   # beta = 0 (probability mode)
    w.options["beta_mode"] = "probability"
    rng = np.random.default_rng(40)
    logical = (rng.standard_normal((B, HV, K, V)) * 1e-33).astype(np.float32)   # amax ~ 5e-33 < 2^-100
    logical[1, 1, :, 64:] = 0.0                                                  # one all-zero tile
    tiles = logical if layout == "K_FIRST" else np.swapaxes(logical, -1, -2)
    pool = torch.from_numpy(np.ascontiguousarray(tiles)).cuda()
    P.gpu_call(w, pool, P.device_inputs(w))
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    got_logical = got if layout == "K_FIRST" else np.swapaxes(got, -1, -2)
    assert float(np.abs(logical).max()) < 2.0 ** -100
    y = (logical * np.float32(448.0 * 2.0 ** 100)).astype(np.float32)
    codes = e4m3.e4m3_round(y.astype(np.float64)).astype(np.float32)
    expect = codes * np.float32(2.0 ** -100 / 448.0)
    assert np.array_equal(got_logical, expect)
    assert not got_logical[1, 1, :, 64:].any()


# ---------------------------------------------------------------- closed forms on the GPU

@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_beta0_gate0_leaves_state_bit_identical(layout):
    w = wl.gdn_pooled(3, 2, 4, 128, 128, lengths=[1, 4, 2], num_slots=5, state_layout=layout, seed=39,
                      io_dtype=torch.float32, beta_mode="probability")
    T = w.T
    w.inputs["a"] = torch.full((T, 4), -float("inf"))
    w.inputs["b"] = torch.zeros((T, 4))
    pool = wl.make_pool(w, "cuda")
    before = pool.clone()
    rep, _, pool = P.run_and_check(w, pool=pool)
    assert torch.equal(pool, before)
    _report(f"beta0_gate0/{layout}", rep)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_alpha1_beta1_signed_basis_keys_recover_values_exactly(layout):
    K = V = 128
    T = 40
    w = wl.gdn_pooled(1, 1, 1, K, V, lengths=[T], num_slots=2, state_layout=layout, seed=40,
                      io_dtype=torch.float32, out_dtype=torch.float32, beta_mode="probability",
                      use_qk_l2norm=False, zero_state=True)
    perm = np.random.default_rng(41).permutation(K)[:T]
    keys = np.zeros((T, 1, K), np.float32)
    keys[np.arange(T), 0, perm] = np.where(np.arange(T) % 2, -1.0, 1.0)
    w.inputs["k"] = torch.from_numpy(keys)
    w.inputs["a"] = torch.full((T, 1), -float("inf"))
    w.inputs["b"] = torch.ones((T, 1))
    rep, _, pool = P.run_and_check(w)
    slot = int(w.inputs["state_indices"][0])
    S = pool[slot, 0].cpu().numpy()
    S = S if layout == "K_FIRST" else S.T
    vals = w.inputs["v"][:, 0].numpy()
    for t in range(T):
        assert np.array_equal(keys[t, 0] @ S, vals[t])
    _report(f"recovery/{layout}", rep)


def test_two_calls_equal_one_call_on_gpu():
    """A suffix split into two calls gives the same state as one call (the pool carries the state)."""
    w = wl.gdn_pooled(2, 1, 2, 128, 128, lengths=[5, 3], num_slots=3, seed=42)
    d = P.device_inputs(w)
    pool1 = wl.make_pool(w, "cuda")
    pool2 = pool1.clone()
    out_all = P.gpu_call(w, pool1, d)
    # first call: tokens [0,2) of seq 0 and [5,6) of seq 1; second call: the rest
    cu = w.inputs["cu_seqlens"].numpy()
    part1 = [np.arange(0, 2), np.arange(5, 6)]
    part2 = [np.arange(2, 5), np.arange(6, 8)]
    for parts in (part1, part2):
        rows = np.concatenate(parts)
        sub = {k: v for k, v in d.items()}
        for k in ("q", "k", "v", "a", "b"):
            sub[k] = d[k][torch.from_numpy(rows).cuda()].contiguous()
        sub["cu_seqlens"] = torch.tensor([0, len(parts[0]), len(rows)], dtype=torch.int32, device="cuda")
        w2 = wl.Workload(w.kind, w.name, w.B, w.HK, w.HV, w.K, w.V, w.io_dtype, w.out_dtype, w.state_layout,
                         w.num_rows, w.inputs, w.options)
        P.gpu_call(w2, pool2, sub)
    torch.cuda.synchronize()
    # the kernel keeps the state as scale * registers inside a call, so a split
    # call rounds differently; the two schedules agree to float32 accuracy
    torch.testing.assert_close(pool1, pool2, rtol=1e-5, atol=1e-6)
    assert cu[-1] == 8


# ---------------------------------------------------------------- narrow V-blocks (about one token per sequence)

@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_single_token_vfirst_narrow_blocks(kind, io):
    # T <= 1.5 B selects the 8-column V-blocks for V_FIRST pools; lengths mix 0, 1 and 2 tokens
    lens = [1, 1, 2, 0, 1, 1, 2, 1]
    if kind == "gdn":
        w = wl.gdn_pooled(len(lens), 2, 4, 128, 128, lengths=lens, num_slots=9, state_layout="V_FIRST",
                          io_dtype=io, seed=43)
    else:
        w = wl.kda_pooled(len(lens), 4, 4, 128, 128, lengths=lens, num_slots=9, state_layout="V_FIRST",
                          io_dtype=io, seed=44)
    assert 2 * w.T <= 3 * w.B
    rep, _, _ = P.run_and_check(w)
    _report(f"narrow/{kind}/{io}", rep)


def test_single_token_vfirst_no_cu_seqlens():
    w = wl.gdn_pooled(24, 4, 8, 128, 256, lengths=None, num_slots=30, state_layout="V_FIRST", seed=45)
    rep, _, _ = P.run_and_check(w)
    _report("narrow/no_cu", rep)


@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_single_token_shapes_v192(layout, kind, io):
    # one token per sequence selects the narrow single-token workgroups of each layout and
    # kind; V = 192 is 24, 12 and 6 of their V-blocks and 3 of the general 64-column block
    if kind == "gdn":
        w = wl.gdn_pooled(20, 2, 4, 128, 192, lengths=None, num_slots=23, state_layout=layout, io_dtype=io, seed=49)
    else:
        w = wl.kda_pooled(20, 4, 4, 128, 192, lengths=[1] * 20, num_slots=23, state_layout=layout, io_dtype=io,
                          seed=49)
    rep, _, _ = P.run_and_check(w)
    _report(f"single/{kind}/{layout}/{io}", rep)


# ---------------------------------------------------------------- paged KDA, paged suffixes, precomputed slots

@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
def test_paged_kda_b256(layout):
    w = wl.paged_kda_b256(state_layout=layout)
    rep, _, _ = P.run_and_check(w)
    _report(f"{w.name}/{layout}", rep)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
@pytest.mark.parametrize("idx", [torch.int32, torch.int64])
def test_paged_varlen_small(kind, layout, idx):
    # page_size 4 and suffixes of 0..9 tokens: suffixes that fill 0, 1 and 2 pages, start on a
    # page boundary (state read from a full, possibly shared page) and cross the 8-token chunks
    suffix = np.array([0, 1, 2, 3, 4, 5, 8, 9, 7, 1, 4, 0, 6, 2, 9, 3])
    w = wl.paged(kind, len(suffix), 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3,
                 suffix_lengths=suffix, state_layout=layout, index_dtype=idx, seed=46)
    rep, _, _ = P.run_and_check(w)
    _report(f"paged_varlen/{kind}/{layout}/{idx}", rep)


@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
def test_paged_varlen_qdq(layout):
    suffix = np.array([3, 5, 1, 0, 8, 4])
    w = wl.paged("gdn", len(suffix), 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3,
                 suffix_lengths=suffix, state_layout=layout, seed=47, qdq="fp8_e4m3_tile", block_v=64)
    rep, _, _ = P.run_and_check(w)
    _report(f"paged_varlen_qdq/{layout}", rep)


def test_paged_varlen_b256_t4():
    w = wl.paged_gdn_varlen_b256_t4()
    rep, _, _ = P.run_and_check(w)
    _report(w.name, rep)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("idx", [torch.int32, torch.int64])
def test_precomputed_slots_match_table_and_inline_resolution(kind, idx):
    import recurrent_state_decode_amd as rsd
    w = wl.paged(kind, 48, 2, 4, 128, 128, max_prefix=40, page_size=4, share_frac=0.3, index_dtype=idx, seed=48)
    d = P.device_inputs(w)
    slots = rsd.gdn_paged_decode_slots(d["page_indices"], d["page_indptr"], d["last_page_len"])
    torch.cuda.synchronize()
    reads, writes = P.rows_for(w)
    assert slots[:, 0].cpu().tolist() == reads and slots[:, 1].cpu().tolist() == writes
    pool_a = wl.make_pool(w, "cuda")
    pool_b = pool_a.clone()
    out_a = P.gpu_call(w, pool_a, d)
    out_b = P.gpu_call(w, pool_b, d, slots=slots)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(pool_a, pool_b)
    rep, _, _ = P.run_and_check(w, slots=slots)
    _report(f"slots/{kind}/{idx}", rep)


# ---------------------------------------------------------------- int8_hadamard32 state codec

@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("extra", [dict(), dict(quantize_initial=True), dict(readout="stored")])
def test_codec_variants(layout, kind, extra):
    mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
    w = mk(6, 2, 4, 128, 128, lengths=[4, 1, 0, 9, 2, 3], num_slots=8, state_layout=layout, seed=50,
           qdq="int8_hadamard32", block_v=64, **extra)
    rep, _, _ = P.run_and_check(w)
    _report(f"codec/{kind}/{layout}/{extra}", rep)


def _half_code_grid_pool(B, HV, K, V, rng):
    """Logical states whose rotated groups are z = (n + f) 2^k with amax|z| = 127 2^k (k per group),
    ties included, one all-zero group per head; returns (x, expected codec result), both exact."""
    from oracle import hadamard as ohad
    Hm = ohad.hadamard_matrix()
    G = V // 32
    n = rng.integers(-126, 127, (B, HV, K, G, 32)).astype(np.float64)
    f = rng.choice([0.0, 0.5, -0.5, 0.25, 0.75], n.shape)
    k = rng.integers(-12, 3, (B, HV, K, G, 1)).astype(np.float64)
    z = (n + f) * 2.0 ** k
    pos = rng.integers(0, 32, (B, HV, K, G))
    sign = rng.choice([-1.0, 1.0], (B, HV, K, G))
    np.put_along_axis(z, pos[..., None], (sign * 127)[..., None] * 2.0 ** k, axis=-1)
    z[:, :, 5, 1, :] = 0.0
    x = (z @ Hm) / 32
    code = np.rint(z * 2.0 ** -k)
    expect = (code @ Hm) * 2.0 ** (k - 5)
    return x.reshape(B, HV, K, V), expect.reshape(B, HV, K, V)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_codec_decisions_exact_on_the_half_code_grid(layout):
    """alpha = 1 and beta = 0 leave the state unchanged, so the stored state is the codec of the
    initial pool.  Its rotated groups sit on the half-code grid with power-of-two scales, where every
    float32 step of the codec is exact: the GPU result must equal (rint_even(z / 2^k) H) 2^k / 32
    bit for bit, ties to even included."""
    B, HV, K, V = 4, 4, 128, 128
    w = wl.gdn_pooled(B, 1, HV, K, V, lengths=[1] * B, num_slots=B, state_layout=layout, seed=51,
                      io_dtype=torch.float32, qdq="int8_hadamard32", block_v=64)
    w.inputs["a"] = torch.full((B, HV), -float("inf"))     # softplus(-inf) = 0 -> alpha = 1
    w.inputs["b"] = torch.zeros((B, HV))                   # beta = b = 0 (probability mode)
    w.options["beta_mode"] = "probability"
    x, expect = _half_code_grid_pool(B, HV, K, V, np.random.default_rng(52))
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    tiles = x if layout == "K_FIRST" else np.swapaxes(x, -1, -2)
    pool = torch.from_numpy(np.ascontiguousarray(tiles).astype(np.float32)).cuda()
    rep, _, pool = P.run_and_check(w, pool=pool)
    got = pool.cpu().numpy().astype(np.float64)
    got_logical = got if layout == "K_FIRST" else np.swapaxes(got, -1, -2)
    assert np.array_equal(got_logical, expect)
    _report(f"codec_exact/{layout}", rep)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_codec_tiny_groups_use_the_amax_floor(layout):
    """A (key row, 32 values) group whose rotated amax is below 2^-100 is rounded as if its amax were
    2^-100 (the kernel's floor, so that 127 / amax stays finite): with alpha = 1 and beta = 0 the stored
    state is (rint(127 z / 2^-100) H) (2^-100 / 127) / 32 for z = x H, up to float32 rounding.  The groups
    here have amax|z| = 127 2^-107, so the floored codes are 128 times coarser than the unfloored ones
    and the two models differ by far more than the tolerance; an all-zero group stays zero."""
    from oracle import hadamard as ohad
    B, HV, K, V = 2, 2, 128, 128
    w = wl.gdn_pooled(B, 1, HV, K, V, lengths=[1] * B, num_slots=B, state_layout=layout, seed=53,
                      io_dtype=torch.float32, qdq="int8_hadamard32", block_v=64)
    w.inputs["a"] = torch.full((B, HV), -float("inf"))     # alpha = 1
    w.inputs["b"] = torch.zeros((B, HV))                   # beta = b = 0 (probability mode)
    w.options["beta_mode"] = "probability"
    rng = np.random.default_rng(54)
    Hm = ohad.hadamard_matrix()
    G = V // 32
    k = -107.0
    z = (rng.integers(-126, 127, (B, HV, K, G, 32)) + rng.choice([0.0, 0.5, -0.25], (B, HV, K, G, 32))) * 2.0 ** k
    z[..., 0] = 127 * 2.0 ** k                            # amax|z| = 127 2^-107 in every group
    z[1, 0, 7, 2, :] = 0.0                                # one all-zero group
    x = (z @ Hm) / 32
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)          # exact float32 inputs
    floor = 2.0 ** -100
    expect = (np.rint(127 * z / floor) @ Hm) * (floor / 127) / 32             # floored rounding
    unfloored = (np.rint(127 * z / (127 * 2.0 ** k)) @ Hm) * 2.0 ** k / 32    # the same rule without it
    expect, unfloored = expect.reshape(B, HV, K, V), unfloored.reshape(B, HV, K, V)
    tiles = x.reshape(B, HV, K, V)
    tiles = tiles if layout == "K_FIRST" else np.swapaxes(tiles, -1, -2)
    pool = torch.from_numpy(np.ascontiguousarray(tiles).astype(np.float32)).cuda()
    P.gpu_call(w, pool, P.device_inputs(w))
    torch.cuda.synchronize()
    got = pool.cpu().numpy().astype(np.float64)
    got = got if layout == "K_FIRST" else np.swapaxes(got, -1, -2)
    tol = 1e-5 * np.abs(expect).max()
    assert np.abs(got - expect).max() <= tol, np.abs(got - expect).max() / tol
    assert np.abs(unfloored - expect).max() > 100 * tol
    assert not got[1, 0, 7, 64:96].any()


@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_codec_paged_varlen(layout, kind):
    suffix = np.array([3, 5, 1, 0, 8, 4])
    w = wl.paged(kind, len(suffix), 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3,
                 suffix_lengths=suffix, state_layout=layout, seed=53, qdq="int8_hadamard32", block_v=64)
    rep, _, _ = P.run_and_check(w)
    _report(f"codec_paged_varlen/{kind}/{layout}", rep)


@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
def test_codec_paged_single_token(layout):
    w = wl.paged("gdn", 40, 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3,
                 state_layout=layout, seed=54, qdq="int8_hadamard32", block_v=128)
    rep, _, _ = P.run_and_check(w)
    _report(f"codec_paged/{layout}", rep)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_codec_gdn_b512_t4(precision):
    """All 512 sequences, the oracle's codec decisions in float64 (the reference) and in float32 (a
    diagnostic of code agreement at the kernel's precision)."""
    w = wl.int8h32_gdn_b512()
    rep, _, _ = P.run_and_check(w, qdq_precision=precision)
    _report(f"{w.name}/{precision}", rep)


# ---------------------------------------------------------------- chunked prefill on the paged pool

@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("layout,idx,page_size", [("V_FIRST", torch.int64, 16), ("K_FIRST", torch.int32, 16),
                                                  ("V_FIRST", torch.int32, 32), ("K_FIRST", torch.int64, 64)])
def test_prefill_small(layout, idx, page_size, kind):
    """Suffixes of 0..70 tokens after prefixes that end on and off page and chunk boundaries."""
    suffix = np.array([1, 5, 16, 17, 0, 40, 33, 70, 2, 31, 15, 64])
    prefix = np.array([15, 16, 1, 31, 7, 32, 48, 5, 63, 64, 100, 17])
    w = wl.paged(kind, len(suffix), 2, 4, 128, 128, prefix_lengths=prefix, page_size=page_size, share_frac=0.3,
                 suffix_lengths=suffix, state_layout=layout, index_dtype=idx, seed=60, chunked=True)
    rep, _, _ = P.run_and_check(w)
    _report(f"prefill_small/{kind}/{layout}/{idx}/ps{page_size}", rep)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_prefill_options(io):
    """fp32 I/O and outputs, probability beta, no L2 norm with an explicit scale, V = 256, GQA 4."""
    suffix = np.array([9, 40, 23])
    w = wl.paged("gdn", 3, 2, 8, 128, 256, max_prefix=50, page_size=16, share_frac=0.0, suffix_lengths=suffix,
                 state_layout="V_FIRST", io_dtype=io, out_dtype=torch.float32, seed=61, chunked=True,
                 beta_mode="probability", use_qk_l2norm=False, scale=0.05)
    w.inputs["b"] = torch.rand(w.inputs["b"].shape).to(io)
    for key in ("q", "k"):
        w.inputs[key] = (w.inputs[key].float() / 8).to(io)
    rep, _, _ = P.run_and_check(w)
    _report(f"prefill_options/{io}", rep)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_prefill_equals_token_path(kind):
    """The chunked call and the token-by-token call agree on outputs and every written page to float32
    rounding of two different summation orders: 2e-5 of |x| + rms (a hundredth of the oracle tolerance)."""
    import recurrent_state_decode_amd as rsd
    suffix = np.array([3, 64, 29, 100, 16, 1])
    w = wl.paged(kind, len(suffix), 2, 4, 128, 128, max_prefix=90, page_size=16, share_frac=0.2,
                 suffix_lengths=suffix, state_layout="V_FIRST", out_dtype=torch.float32, seed=62, chunked=True)
    d = P.device_inputs(w)
    pool_a = wl.make_pool(w, "cuda")
    pool_b = pool_a.clone()
    out_a = P.gpu_call(w, pool_a, d)
    w.chunked = False
    out_b = P.gpu_call(w, pool_b, d)
    torch.cuda.synchronize()
    for a, b in ((out_a, out_b), (pool_a, pool_b)):
        a, b = a.double(), b.double()
        rms = b.pow(2).mean().sqrt()
        err = ((a - b).abs() / (b.abs() + rms)).max().item()
        assert err <= 2e-5, f"chunked vs token-by-token: {err}"


@pytest.mark.timeout(600)
def test_prefill_b16_t1024():
    """All 16 sequences, every output row and every page the suffixes fill."""
    w = wl.paged_gdn_prefill_b16_t1024()
    rep, _, _ = P.run_and_check(w)
    _report(w.name, rep)


@pytest.mark.timeout(600)
def test_kda_prefill_b16_t1024():
    w = wl.paged_kda_prefill_b16_t1024()
    rep, _, _ = P.run_and_check(w)
    _report(w.name, rep)


def test_kda_prefill_strong_decay():
    """Per-channel gates down to exp(-60) per token: pairwise decays underflow to 0 without overflow."""
    suffix = np.array([40, 23])
    w = wl.paged("kda", 2, 2, 2, 128, 128, max_prefix=40, page_size=16, share_frac=0.0, suffix_lengths=suffix,
                 state_layout="V_FIRST", io_dtype=torch.float32, out_dtype=torch.float32, seed=63, chunked=True)
    w.inputs["raw_gate"] = (w.inputs["raw_gate"] * 4).to(torch.float32)
    w.inputs["a_log"] = torch.full_like(w.inputs["a_log"], float(np.log(16.0)))
    rep, _, _ = P.run_and_check(w)
    _report("kda_prefill_strong_decay", rep)


@pytest.mark.parametrize("qdq", [None, "fp8_e4m3_tile", "int8_hadamard32"])
@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_kda_decode_strong_decay(qdq, layout):
    """Half of the key channels decay by about exp(-190) per token (far below float32's range, so those
    rows of the registers underflow to zero within a token) while the other half decay normally: the
    per-channel decay acts on the state's key rows directly, with no per-row scale to overflow."""
    extra = dict(qdq=qdq, block_v=64) if qdq else {}
    w = wl.kda_pooled(6, 2, 4, 128, 128, lengths=[4, 1, 9, 2, 3, 12], num_slots=8, state_layout=layout,
                      io_dtype=torch.float32, out_dtype=torch.float32, seed=70, **extra)
    g = w.inputs["raw_gate"].clone()
    g[..., :64] = 12.0                                  # softplus ~ 12, times exp(a_log) = 16
    w.inputs["raw_gate"] = g
    w.inputs["a_log"] = torch.full_like(w.inputs["a_log"], float(np.log(16.0)))
    rep, _, _ = P.run_and_check(w)
    _report(f"kda_decode_strong_decay/{qdq}/{layout}", rep)


# ---------------------------------------------------------------- packed int8_hadamard32 pools (codes + scales)

CODEC = dict(qdq="int8_hadamard32", block_v=64)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_packed_pooled_small(kind, io):
    mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
    w = mk(6, 2, 4, 128, 128, lengths=[4, 1, 0, 9, 2, 3], num_slots=8, state_layout="K_FIRST", io_dtype=io,
           seed=71, **CODEC)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"packed/{kind}/{io}", rep)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("idx", [torch.int32, torch.int64])
def test_packed_paged(kind, idx):
    w = wl.paged(kind, 24, 2, 4, 128, 128, max_prefix=40, page_size=4, share_frac=0.3, state_layout="K_FIRST",
                 index_dtype=idx, seed=72, **CODEC)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"packed_paged/{kind}/{idx}", rep)
    suffix = np.array([0, 1, 2, 3, 4, 5, 8, 9, 7, 1, 4, 0, 6, 2, 9, 3])
    w = wl.paged(kind, len(suffix), 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3,
                 suffix_lengths=suffix, state_layout="K_FIRST", index_dtype=idx, seed=73, **CODEC)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"packed_paged_varlen/{kind}/{idx}", rep)


@pytest.mark.parametrize("extra", [dict(readout="stored"), dict(quantize_initial=True), dict(V=256),
                                   dict(use_qk_l2norm=False, scale=0.2)])
def test_packed_options(extra):
    extra = dict(extra)
    V = extra.pop("V", 128)
    w = wl.gdn_pooled(5, 1, 2, 128, V, lengths=[2, 7, 1, 0, 3], num_slots=6, state_layout="K_FIRST", seed=74,
                      **CODEC, **{k: v for k, v in extra.items() if k in ("readout", "quantize_initial")})
    over = {k: v for k, v in extra.items() if k not in ("readout", "quantize_initial")}
    rep, _, _ = P.run_and_check_packed(w, **over)
    _report(f"packed_opts/{extra}/V{V}", rep)


def test_packed_equals_fp32_codec_path():
    """The packed pool and an fp32 pool holding its decoded states give the same outputs and, decoded,
    the same states (the registers start from code * scale either way; float32 rounding apart)."""
    from oracle import hadamard as ohad
    w = wl.gdn_pooled(8, 2, 4, 128, 128, lengths=[3, 1, 4, 2, 5, 1, 2, 6], num_slots=10, state_layout="K_FIRST",
                      seed=75, **CODEC)
    d = P.device_inputs(w)
    packed = P.make_packed_pool(w, "cuda")
    tiles = packed.cpu().numpy()
    code, scale = ohad.unpack_tiles(tiles, w.K, w.V)
    fp32 = torch.from_numpy(ohad.int8_hadamard32_decode(code.reshape(-1, w.K, w.V), scale.reshape(-1, w.K, w.V // 32))
                            .reshape(w.pool_shape()).astype(np.float32)).cuda()
    out_p = P.gpu_call(w, packed, d)
    out_f = P.gpu_call(w, fp32, d)
    torch.cuda.synchronize()
    a, b = out_p.float(), out_f.float()
    assert float((a - b).abs().max()) <= 2e-3 * float(b.abs().max())
    assert float((a - b).norm() / b.norm()) < 1e-3
    c2, s2 = ohad.unpack_tiles(packed.cpu().numpy(), w.K, w.V)
    dec = ohad.int8_hadamard32_decode(c2.reshape(-1, w.K, w.V), s2.reshape(-1, w.K, w.V // 32)).reshape(w.pool_shape())
    ref = fp32.cpu().numpy().astype(np.float64)
    rows = sorted(set(P.rows_for(w)[1]))
    err = np.abs(dec[rows] - ref[rows]).max() / np.abs(ref[rows]).max()
    assert err < 2e-2, err          # a code flip moves an element by up to a step / sqrt(32) of the group


@pytest.mark.timeout(600)
def test_packed_b512_t4():
    w = wl.gdn_pooled(512, 16, 32, 128, 128, lengths=np.full(512, 4), num_slots=1024, state_layout="K_FIRST",
                      seed=1008, **CODEC)
    reads, _ = P.rows_for(w)
    pool = P.make_packed_pool(w, "cuda", rows=reads)
    rep, _, _ = P.run_and_check_packed(w, pool=pool)
    _report("packed/b512_t4", rep)


# ---------------------------------------------------------------- packed fp8 tile pools (E4M3 bytes + tile scales)

FP8 = dict(qdq="fp8_e4m3_tile", block_v=64)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_fp8_packed_pooled_small(kind, layout):
    mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
    w = mk(6, 2, 4, 128, 128, lengths=[4, 1, 0, 9, 2, 3], num_slots=8, state_layout=layout, seed=81, **FP8)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"fp8_packed/{kind}/{layout}", rep)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("layout,idx", [("K_FIRST", torch.int32), ("V_FIRST", torch.int64)])
def test_fp8_packed_paged(kind, layout, idx):
    w = wl.paged(kind, 24, 2, 4, 128, 128, max_prefix=40, page_size=4, share_frac=0.3, state_layout=layout,
                 index_dtype=idx, seed=82, **FP8)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"fp8_packed_paged/{kind}/{layout}", rep)
    suffix = np.array([0, 1, 2, 3, 4, 5, 8, 9, 7, 1, 4, 0, 6, 2, 9, 3])
    w = wl.paged(kind, len(suffix), 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3,
                 suffix_lengths=suffix, state_layout=layout, index_dtype=idx, seed=83, **FP8)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"fp8_packed_paged_varlen/{kind}/{layout}", rep)


@pytest.mark.parametrize("extra", [dict(readout="stored"), dict(quantize_initial=True), dict(V=256),
                                   dict(use_qk_l2norm=False, scale=0.2), dict(io_dtype=torch.float32),
                                   dict(K=16, V=48)])
def test_fp8_packed_options(extra):
    extra = dict(extra)
    K, V = extra.pop("K", 128), extra.pop("V", 128)
    fp8 = dict(FP8, block_v=16) if K == 16 else FP8
    wkeys = ("readout", "quantize_initial", "io_dtype")
    w = wl.gdn_pooled(5, 1, 2, K, V, lengths=[2, 7, 1, 0, 3], num_slots=6, state_layout="V_FIRST", seed=84,
                      **fp8, **{k: v for k, v in extra.items() if k in wkeys})
    over = {k: v for k, v in extra.items() if k not in wkeys}
    rep, _, _ = P.run_and_check_packed(w, **over)
    _report(f"fp8_packed_opts/{extra}/K{K}V{V}", rep)


@pytest.mark.parametrize("layout", ["V_FIRST", "K_FIRST"])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_fp8_packed_single_token_shapes(layout, io):
    """Single-token calls on packed fp8 pools (GDN on a V_FIRST pool has its own 128-thread shape): pooled
    with one token per sequence, and paged varlen with mostly one-token suffixes."""
    w = wl.gdn_pooled(12, 2, 4, 128, 128, num_slots=16, state_layout=layout, io_dtype=io, seed=88, **FP8)
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"fp8_packed_t1/{layout}/{io}", rep)
    suffix = np.array([1, 1, 0, 1, 2, 1, 1, 1, 1, 3, 1, 1])
    w = wl.paged("gdn", len(suffix), 2, 4, 128, 128, max_prefix=30, page_size=4, share_frac=0.3,
                 suffix_lengths=suffix, state_layout=layout, io_dtype=io, seed=89, **FP8)
    assert 2 * w.T <= 3 * w.B
    rep, _, _ = P.run_and_check_packed(w)
    _report(f"fp8_packed_varlen_t1/{layout}/{io}", rep)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_fp8_packed_equals_fp32_fp8_path(kind):
    """The packed pool and an fp32 pool holding its decoded states give the same outputs and the same
    states (the registers start from the same grid values and scales; float32 rounding apart)."""
    mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
    w = mk(8, 2, 4, 128, 128, lengths=[3, 1, 4, 2, 5, 1, 2, 6], num_slots=10, state_layout="V_FIRST", seed=85,
           **FP8)
    d = P.device_inputs(w)
    packed = P.make_packed_pool(w, "cuda")
    dec = lambda pool: np.stack([P.decode_fp8(*P.gather_fp8(pool, [r], w)[r], w) for r in range(w.num_rows)])
    fp32 = torch.from_numpy(np.ascontiguousarray(dec(packed), dtype=np.float32)).cuda()
    out_p = P.gpu_call(w, packed, d)
    out_f = P.gpu_call(w, fp32, d)
    torch.cuda.synchronize()
    a, b = out_p.float(), out_f.float()
    assert float((a - b).abs().max()) <= 8e-3 * float(b.abs().max())   # one bf16 step at the largest output
    assert float((a - b).norm() / b.norm()) < 1e-3
    rows = sorted(set(P.rows_for(w)[1]))
    got, ref = dec(packed)[rows], fp32.cpu().numpy().astype(np.float64)[rows]
    flips = np.abs(got - ref) > 1e-6 * np.abs(ref).max()
    assert flips.mean() < 1e-3, flips.mean()
    assert np.abs(got - ref).max() <= 0.07 * np.abs(ref).max()   # at most one grid step (32 / 448 of amax)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_fp8_packed_identity_step_keeps_every_byte(layout):
    """alpha = 1 and beta = 0 leave the state unchanged: the tile QDQ of a decoded tile is the tile itself
    (its amax is 448 s, so the scale is s again and every code maps to itself), so every byte written equals
    the byte read, all-zero tiles (scale 0) included.  The one exception is the sign of a zero: the update
    adds beta k (...) = +-0 to every element, and -0 + +0 is +0, so a -0 code (0x80) may come back as +0."""
    B, HV, nb = 4, 4, 128 * 128
    w = wl.gdn_pooled(B, 1, HV, 128, 128, lengths=[1] * B, num_slots=B, state_layout=layout, seed=86,
                      io_dtype=torch.float32, **FP8)
    w.inputs["a"] = torch.full((B, HV), -float("inf"))     # softplus(-inf) = 0 -> alpha = 1
    w.inputs["b"] = torch.zeros((B, HV))                   # beta = b = 0 (probability mode)
    w.options["beta_mode"] = "probability"
    pool = P.make_packed_pool(w, "cuda")
    pool[1, 2, :nb] = 0                                    # an all-zero head ...
    pool[1, 2, nb:nb + 8] = 0                              # ... with scales 0
    col = torch.arange(nb, device="cuda") % 128 if layout == "K_FIRST" else torch.arange(nb, device="cuda") // 128
    pool[2, 0, :nb][col < 64] = 0                          # an all-zero first tile next to a non-zero one
    pool[2, 0, nb:nb + 4] = 0
    before = pool.clone()
    P.gpu_call(w, pool, P.device_inputs(w))
    torch.cuda.synchronize()
    plus0 = lambda t: torch.where(t[..., :nb] == 0x80, torch.zeros_like(t[..., :nb]), t[..., :nb])
    diff = torch.nonzero(plus0(pool) != plus0(before))
    assert diff.numel() == 0, f"codes changed at {diff[:5].tolist()}"
    assert torch.equal(pool[..., nb:], before[..., nb:]), "tile scales or padding changed"
    n_neg0 = int((before[..., :nb] == 0x80).sum())
    print(f"[identity] -0 codes before {n_neg0}, after {int((pool[..., :nb] == 0x80).sum())}")


def test_fp8_packed_zero_state_tiles():
    """A zero initial state and zero values in a head's first 64 columns keep that tile zero: its codes stay
    0 and its scale 0, next to a non-zero tile of the same head."""
    w = wl.gdn_pooled(4, 2, 4, 128, 128, lengths=[3, 1, 2, 4], num_slots=6, state_layout="K_FIRST", seed=87,
                      zero_state=True, **FP8)
    w.inputs["v"][:, 1, :64] = 0
    rep, _, pool = P.run_and_check_packed(w)
    rows = sorted(set(P.rows_for(w)[1]))
    for r, (codes, scales) in P.gather_fp8(pool, rows, w).items():
        assert scales[1, 0] == 0 and not codes[1, :, :64].any() and scales[1, 1] > 0
    _report("fp8_packed/zero_tiles", rep)


@pytest.mark.timeout(600)
def test_fp8_packed_gdn_b512_t4():
    w = wl.fp8_qdq_gdn_b512()
    reads, _ = P.rows_for(w)
    pool = P.make_packed_pool(w, "cuda", rows=reads)
    rep, _, _ = P.run_and_check_packed(w, pool=pool)
    _report("fp8_packed/b512_t4", rep)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("storage", ["fp8", "i8h32"])
def test_packed_paged_gdn_b256(storage):
    """The headline paged shape (B=256, HV=32, K=V=128, page size 16) on a packed pool, as bench.py
    --storage times it (fp8: its V_FIRST pool and 128-thread shape; i8h32: K_FIRST), every sequence."""
    layout = "V_FIRST" if storage == "fp8" else "K_FIRST"
    w = wl.paged_gdn_b256(state_layout=layout)
    w.options.update(qdq="fp8_e4m3_tile" if storage == "fp8" else "int8_hadamard32", block_v=64)
    reads, _ = P.rows_for(w)
    pool = P.make_packed_pool(w, "cuda", rows=reads)
    rep, _, _ = P.run_and_check_packed(w, pool=pool)
    _report(f"packed_{storage}/paged_gdn_b256", rep)

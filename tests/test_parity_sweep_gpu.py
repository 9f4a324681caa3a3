"""Seeded randomised parity sweep: small cases drawn over kind, path (pooled / paged / paged suffixes /
chunked prefill), layout, state storage, QDQ policy, head sizes, dtypes and activation options.  Each
case is its own test, named by its index; the draw depends only on that index."""
import numpy as np
import pytest
import torch

from recurrent_state_decode_amd import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu
N_CASES = 200
N_LARGE = 120


def _case(i, large=False):
    """Case i of the small draw, or (large) of the draw with 20-63 sequences, 8 value heads and V up to 320
    (several V-blocks per head, ragged tails of the grid)."""
    rng = np.random.default_rng([777 if large else 20261203, i])
    kind = str(rng.choice(["gdn", "kda"]))
    layout = str(rng.choice(["K_FIRST", "V_FIRST"]))
    path = str(rng.choice(["pooled", "paged", "varlen", "prefill", "k16"]))
    q = str(rng.choice(["none", "fp8", "fp8p", "codec", "codecp"]))
    io = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    out = torch.float32 if rng.random() < 0.3 else None
    seed = int(rng.integers(1, 10 ** 6))
    opts = {}
    if rng.random() < 0.2:
        opts["beta_mode"] = "probability"
    if path in ("prefill", "k16"):
        q = "none" if path == "prefill" else str(rng.choice(["none", "fp8", "fp8p"]))
    if q.startswith("codec"):
        opts.update(qdq="int8_hadamard32", block_v=64)
        if q == "codecp":
            layout = "K_FIRST"
    elif q != "none":
        opts.update(qdq="fp8_e4m3_tile", block_v=16 if path == "k16" else 64)
    if q != "none":
        if rng.random() < 0.3:
            opts["readout"] = "stored"
        if rng.random() < 0.3:
            opts["quantize_initial"] = True
    B = int(rng.integers(20, 64)) if large else int(rng.integers(1, 20))
    if large:
        V = int(rng.choice([128, 256, 320])) if not q.startswith("codec") else int(rng.choice([128, 256]))
    else:
        V = int(rng.choice([64, 128, 192])) if not q.startswith("codec") else int(rng.choice([64, 128]))
    HK, HV = (2, 8) if large else (1, 2)
    if path == "pooled":
        lens = rng.integers(0, 7, B).tolist()
        lens[0] = max(1, lens[0])
        mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
        w = mk(B, HK, HV, 128, V, lengths=lens, num_slots=B + 3, state_layout=layout, io_dtype=io, out_dtype=out,
               seed=seed, **opts)
    elif path == "paged":
        w = wl.paged(kind, B, HK, HV, 128, V, max_prefix=40, page_size=4, share_frac=0.3, state_layout=layout,
                     io_dtype=io, out_dtype=out, seed=seed, **opts)
    elif path == "varlen":
        suf = rng.integers(0, 8, B)
        suf[0] = max(1, suf[0])
        w = wl.paged(kind, B, HK, HV, 128, V, max_prefix=30, page_size=int(rng.choice([2, 4, 16])), share_frac=0.3,
                     suffix_lengths=suf, state_layout=layout, io_dtype=io, out_dtype=out, seed=seed, **opts)
    elif path == "prefill":
        suf = rng.integers(0, 70, min(B, 5))
        suf[0] = max(1, suf[0])
        w = wl.paged(kind, len(suf), 2, 4, 128, 128, max_prefix=50, page_size=int(rng.choice([16, 32])),
                     share_frac=0.0, suffix_lengths=suf, state_layout=layout, io_dtype=io, out_dtype=out, seed=seed,
                     chunked=True, **opts)
    else:
        lens = rng.integers(0, 9, B).tolist()
        lens[0] = max(1, lens[0])
        mk = wl.gdn_pooled if kind == "gdn" else wl.kda_pooled
        w = mk(B, 1, 2, 16, int(rng.choice([16, 32, 48])), lengths=lens, num_slots=B + 2, state_layout=layout,
               io_dtype=io, out_dtype=out, seed=seed, **opts)
    return w, q in ("fp8p", "codecp")


def _run(i, large):
    w, packed = _case(i, large)
    print(f"[sweep {'large ' if large else ''}{i}] {w.kind} {w.state_layout} B={w.B} K={w.K} V={w.V} T={w.T} "
          f"chunked={w.chunked} packed={packed} options={w.options}", flush=True)
    rep, _, _ = P.run_and_check_packed(w) if packed else P.run_and_check(w)
    print(f"[sweep {i}] {rep}", flush=True)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    _run(i, large=False)


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_case(i):
    _run(i, large=True)


@pytest.mark.parametrize("i", range(0, N_CASES, 4))
def test_random_case_checked_build_accepts_and_matches(i):
    """The GDN_DEVICE_CHECKS build accepts every drawn (valid) call and gives the release build's outputs
    and pool bit for bit."""
    import recurrent_state_decode_amd as rsd
    w, packed = _case(i)
    d = P.device_inputs(w)
    pool_a = P.make_packed_pool(w, "cuda") if packed else wl.make_pool(w, "cuda")
    pool_b = pool_a.clone()
    out_a = P.gpu_call(w, pool_a, d)
    with rsd.checked_library() as lib:
        assert lib.gdn_checked_build() == 1
        out_b = P.gpu_call(w, pool_b, d)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(pool_a, pool_b)

// Chunked (WY-form) GDN prefill on a CSR-paged state pool: the same result as
// the token-by-token paged suffix decode (every page a suffix token fills
// receives the state after that token), computed chunk by chunk with MFMA.
//
// Math per chunk of C = 16 tokens with initial state S0 [K, V]
// (modelopt ... linear_attention.config, LinearAttentionConfig: the chunked
// step names gate_prefix ... state_add; LinearAttentionSolveConfig: an exact
// solve; Circuit.LLM.Mixer, "Chunked additive linear": chunked equals
// sequential):
//     G_t  = sum_{s<=t} g_s                       (g = log alpha, so G <= 0)
//     A'   = strict_lower( beta_t exp(G_t - G_s) k_t . k_s )
//     T    = (I + A')^-1                          (forward substitution)
//     U    = T diag(beta) (V - diag(exp G) K S0)
//          (= U~ - W S0 with U~ = T diag(beta) V, W = T diag(beta exp G) K)
//     O    = diag(exp G) Q S0 + P U,  P = lower( exp(G_t - G_s) q_t . k_s )
//     S_C  = exp(G_C) S0 + sum_s exp(G_C - G_s) k_s u_s^T
// KDA (max.nn.state_space.kda_decode: one gate per key channel): G is a
// vector per token, exp(G) acts on key channels (the rows of S), so K S0
// and Q S0 use the gated rows k_t exp(G_t), q_t exp(G_t), the update uses
// exp(G_C - G_s) k_s and scales row c of S0 by exp(G_C,c), and A' / P need
// sum_c x_tc k_sc exp(G_tc - G_sc), which is formed on the VALU pair by pair
// (one thread per (t, s)) since splitting exp(G_t - G_s) into two factors can
// overflow one of them.
// Every exponent is <= 0.  Chunks are aligned to absolute token positions
// (16 j + 1 .. 16 j + 16), so with a page size that is a multiple of 16 every
// page end is a chunk end and its state is S_C of that chunk.  Positions of a
// chunk outside the suffix are identity tokens (k = q = v = 0, beta = 0,
// g = 0): their rows of A', W, U~ and U are zero and T is the identity on
// them, so they change nothing.
//
// One workgroup per (sequence, value head, 128-column V-block), 8 / VT waves;
// wave w owns value columns [16 VT w, 16 VT (w + 1)) of the block and keeps
// S[:, those] (128 x 16 VT) as 8 VT MFMA accumulator tiles for the whole
// suffix.  The
// products that involve S use the accumulator registers directly as the B
// operand of v_mfma_f32_16x16x4_f32: a lane holds S rows 4 g + r of a tile
// (g = lane / 16), so the k-step r pairs B = element r with A = the matching
// column 16 ct + 4 g + r of the left factor.  K S0 and Q S0 do not depend on
// the solve and are formed while waves 0 and 1 build A' and P; every wave
// then solves for T itself (16 lanes, forward substitution), so the solve
// needs no workgroup barrier.  A chunk's inputs are loaded one chunk ahead.
//
// MFMA 16x16x4 f32 lane layout (checked on the device): A[i][k] from lane
// i + 16 k, B[k][j] from lane j + 16 k, D[4 (l / 16) + r][l % 16] in lane l,
// element r.
#pragma once

#include "decode_kernel.hpp"

namespace gdn {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;        // GDN: a [T, HV]; KDA: raw_gate [T, HV, K]
  const void* beta;        // b / beta_logits [T, HV]
  const float* a_log;      // [HV]
  const float* dt_bias;    // GDN: [HV]; KDA: [HV, K]
  const int32_t* cu_seqlens;
  const void* page_indices;
  const void* page_indptr;
  const void* last_page_len;
  int32_t page_size;
  float* pool;
  void* out;
  int32_t B, HK, HV, V;
  int32_t nvb;             // V / VBLK
  int32_t gqa;
  float scale;
  int32_t l2norm, out_bf16, beta_prob, idx64;
  int32_t xcd_shift;       // log2 of the run of consecutive work units kept on one XCD
};

constexpr int kChunk = 16;

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// VT value tiles (16 columns each) per wave, NW waves per workgroup: a
// workgroup covers VBLK = 16 VT NW value columns.
template <int VT, int NW>
constexpr int kPrefillVBlk = 16 * VT * NW;

template <int VT, int NW, bool KDA, bool VF, typename TIn>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(8 / (2 * VT), 8 / (2 * VT))))
void prefill_kernel(const PrefillParams p) {
  constexpr int K = 128, C = kChunk, SPW = C / NW;
  constexpr int VBLK = kPrefillVBlk<VT, NW>;
  constexpr int VPL = VBLK / 64;   // staged v elements per lane
  constexpr int PPT = C * C / (NW * 64);   // KDA: (t, s) pairs per thread
  static_assert(VBLK % 64 == 0 && VPL <= 2 && C % NW == 0 && (C * C) % (NW * 64) == 0, "prefill shape");
  constexpr int LDK = K + 4;       // padded LDS rows
  constexpr int LDC = C + 1;

  __shared__ __align__(16) float s_q[C][LDK];   // q_hat (scaled)
  __shared__ __align__(16) float s_k[C][LDK];   // k_hat
  __shared__ __align__(16) float s_v[C][LDK];   // v of this V-block
  __shared__ float s_a[C][LDC];                 // A' (strict lower)
  __shared__ float s_p[C][LDC];                 // P (lower, diagonal included)
  __shared__ float s_t[NW][C][LDC];             // T = (I + A')^-1, one copy per wave
  __shared__ float s_g[C], s_b[C];
  // KDA: per-channel gates.  s_G holds g, then G (in place); s_kg / s_qg =
  // k / q times exp(G); s_kd = exp(G_C - G) k; s_eC = exp(G_C) per channel
  constexpr int KC = KDA ? C : 1, KK = KDA ? LDK : 1;
  __shared__ __align__(16) float s_G[KC][KK], s_kg[KC][KK], s_qg[KC][KK], s_kd[KC][KK];
  __shared__ __align__(16) float s_eC[KDA ? K : 1];

  const TIn* __restrict__ gq = static_cast<const TIn*>(p.q);
  const TIn* __restrict__ gk = static_cast<const TIn*>(p.k);
  const TIn* __restrict__ gv = static_cast<const TIn*>(p.v);
  const TIn* __restrict__ gg = static_cast<const TIn*>(p.gate);
  const TIn* __restrict__ gb = static_cast<const TIn*>(p.beta);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;       // MFMA row / column inside a tile
  const int g4 = lane >> 4;        // MFMA k group

  // Consecutive workgroup ids go to the 8 XCDs in turn.  Renumber them so
  // that each run of 2^xcd_shift consecutive units (the value heads that read
  // one key head's q / k, and their V-blocks) lands on one XCD and shares its
  // L2; ids past the last whole span of 8 runs keep their number.  A
  // permutation of [0, gridDim.x).
  const int bx = blockIdx.x;
  const int gs = p.xcd_shift;
  const int nfull = (static_cast<int>(gridDim.x) >> (gs + 3)) << (gs + 3);
  const int unit = bx < nfull ? (((bx >> (gs + 3)) << (gs + 3)) | ((bx & 7) << gs) | ((bx >> 3) & ((1 << gs) - 1)))
                              : bx;
  const int q1 = unit / p.nvb;
  const int vb = unit - q1 * p.nvb;
  const int bs = q1 / p.HV;
  const int h = q1 - bs * p.HV;
  const int hk = h / p.gqa;

  const int t0 = p.cu_seqlens[bs];
  const int t1 = p.cu_seqlens[bs + 1];
  if (t1 <= t0) return;            // empty suffix: no read, no write

  // the sequence holds pos_last tokens after the suffix; the suffix is
  // positions pos0 .. pos_last (1-based); the state before it lives on the
  // page of position pos0 - 1
  // (token positions of one sequence fit in 32 bits; table offsets may not)
  const int64_t pg_start = load_index(p.page_indptr, bs, p.idx64);
  const int64_t pg_end = load_index(p.page_indptr, bs + 1, p.idx64);
  const int lpl = static_cast<int>(load_index(p.last_page_len, bs, p.idx64));
  const int pos_last = static_cast<int>(pg_end - pg_start - 1) * p.page_size + lpl;
  const int pos0 = pos_last - (t1 - t0) + 1;
  const int64_t rrow = load_index(p.page_indices, pg_start + max(pos0 - 2, 0) / p.page_size, p.idx64);
  const int64_t wrow = load_index(p.page_indices, pg_end - 1, p.idx64);

  const int64_t tile_elems = static_cast<int64_t>(K) * p.V;
  const int vcol = vb * VBLK + 16 * VT * w;   // first value column of this wave

  // ---- raw inputs of one chunk's slots 4 w .. 4 w + 3 (issued a chunk ahead)
  constexpr int GPL = KDA ? 2 : 1;  // gate elements per lane
  Raw<TIn, 2> rq[SPW], rk[SPW];
  Raw<TIn, VPL> rv[SPW];
  Raw<TIn, GPL> ra[SPW];
  Raw<TIn, 1> rb[SPW];
  auto load_chunk = [&](int cpos) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int pos = cpos + w * SPW + i;
      if (pos >= pos0 && pos <= pos_last) {  // uniform per wave
        const int64_t t = t0 + (pos - pos0);
        load_raw_n<2>(gq, (t * p.HK + hk) * K + 2 * lane, rq[i]);
        load_raw_n<2>(gk, (t * p.HK + hk) * K + 2 * lane, rk[i]);
        load_raw_n<VPL>(gv, (t * p.HV + h) * p.V + vb * VBLK + VPL * lane, rv[i]);
        if constexpr (KDA) load_raw_n<2>(gg, (t * p.HV + h) * K + 2 * lane, ra[i]);
        else load_raw_n<1>(gg, t * p.HV + h, ra[i]);
        load_raw_n<1>(gb, t * p.HV + h, rb[i]);
      }
    }
  };
  const float rate = exp_hw(p.a_log[h]);
  float dtb[GPL];
#pragma unroll
  for (int e = 0; e < GPL; ++e) dtb[e] = KDA ? p.dt_bias[h * K + 2 * lane + e] : p.dt_bias[h];
  // normalise, gate and stage the slots in LDS (positions outside the suffix: identity tokens)
  auto stage_chunk = [&](int cpos) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int slot = w * SPW + i;
      const int pos = cpos + slot;
      float xq[2] = {0.0f, 0.0f}, xk[2] = {0.0f, 0.0f}, xv[VPL] = {};
      float gt[GPL] = {}, bt = 0.0f;
      if (pos >= pos0 && pos <= pos_last) {
        decode_raw(rq[i], xq);
        decode_raw(rk[i], xk);
        decode_raw(rv[i], xv);
        float xa[GPL], xb[1];
        decode_raw(ra[i], xa);
        decode_raw(rb[i], xb);
        float iq = p.scale, ik = 1.0f;
        if (p.l2norm) {
          iq = p.scale * rsqrtf(lane_reduce<0, 6>(fmaf(xq[0], xq[0], xq[1] * xq[1])) + kL2Eps);
          ik = rsqrtf(lane_reduce<0, 6>(fmaf(xk[0], xk[0], xk[1] * xk[1])) + kL2Eps);
        }
        xq[0] *= iq;
        xq[1] *= iq;
        xk[0] *= ik;
        xk[1] *= ik;
#pragma unroll
        for (int e = 0; e < GPL; ++e) gt[e] = -rate * softplus_f(xa[e] + dtb[e]);
        bt = p.beta_prob ? xb[0] : sigmoid_f(xb[0]);
      }
      *reinterpret_cast<float2*>(&s_q[slot][2 * lane]) = make_float2(xq[0], xq[1]);
      *reinterpret_cast<float2*>(&s_k[slot][2 * lane]) = make_float2(xk[0], xk[1]);
#pragma unroll
      for (int e = 0; e < VPL; ++e) s_v[slot][VPL * lane + e] = xv[e];
      if constexpr (KDA) *reinterpret_cast<float2*>(&s_G[slot][2 * lane]) = make_float2(gt[0], gt[1]);
      if (lane == 0) {
        if constexpr (!KDA) s_g[slot] = gt[0];
        s_b[slot] = bt;
      }
    }
  };

  const int jfirst = (pos0 - 1) / C;
  const int jlast = (pos_last - 1) / C;
  // page ends met by the chunk loop: the first one at or after the end of
  // chunk jfirst, then one every page_size / C chunks
  const int cpp = p.page_size / C;
  int to_page_end = (cpp - 1) - jfirst % cpp;   // chunks until one ends a page
  int64_t page_slot = pg_start + jfirst / cpp;  // table entry of that page
  load_chunk(jfirst * C + 1);      // in flight while the state tile loads

  // S[ct][vt] element r = S[16 ct + 4 g4 + r][vcol + 16 vt + n16]
  f32x4 S[8][VT];
  // offset of element r of tile (ct, vt) inside one (row, head) state: a
  // per-lane base plus a uniform part (32-bit: a state holds K V < 2^31 floats)
  const int lane_base = VF ? (vcol + n16) * K + 4 * g4 : 4 * g4 * p.V + vcol + n16;
  auto state_off = [&](int ct, int vt, int r) -> int {
    return VF ? lane_base + 16 * vt * K + 16 * ct + r : lane_base + (16 * ct + r) * p.V + 16 * vt;
  };
  {
    const float* src = p.pool + (rrow * p.HV + h) * tile_elems;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        if constexpr (VF) {
          S[ct][vt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + state_off(ct, vt, 0)));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // uniform row pointer + 32-bit lane offset (K_FIRST: one key row per element)
            const float* rowp = src + static_cast<uint32_t>((16 * ct + r) * p.V + 16 * vt);
            S[ct][vt][r] = __builtin_nontemporal_load(rowp + static_cast<uint32_t>(lane_base));
          }
        }
      }
  }
  // (plain stores: non-temporal ones, which help the decode kernel, measured
  // ~8 % slower here, where a page is written every chunk while computing)
  // key rows 16 ct .. 16 ct + 15 of this wave's columns of S to a pool row
  auto store_rows = [&](int64_t row, int ct) {
    float* dst = p.pool + (row * p.HV + h) * tile_elems;
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      if constexpr (VF) {
        *reinterpret_cast<f32x4*>(dst + state_off(ct, vt, 0)) = S[ct][vt];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* rowp = dst + static_cast<uint32_t>((16 * ct + r) * p.V + 16 * vt);
          rowp[static_cast<uint32_t>(lane_base)] = S[ct][vt][r];
        }
      }
    }
  };
  auto store_state = [&](int64_t row) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) store_rows(row, ct);
  };
  // A page that a chunk fills receives the state after that chunk.  The
  // registers keep that state until the next chunk's update, so KDA defers
  // the store into the next chunk's K S0 / Q S0 products and issues it 16
  // key rows at a time between their matrix instructions (5 % faster on
  // 16 x 1024 tokens); GDN, 5 % slower that way, stores at the chunk's end.
  constexpr bool kDeferStore = KDA;
  bool store_pending = false;
  int64_t pending_row = 0;

  // GDN stages chunk j at the end of iteration j - 1 (the first one before
  // the loop), so the raw input registers never cross the loop's back edge
  // and waiting for them never waits for the stores of earlier chunks
  // (about 10 % on 16 x 1024 tokens).  KDA, whose chunk starts with the
  // per-channel gate prefix, measured 4 % slower that way and stages each
  // chunk at the top of its own iteration.
  constexpr bool kStageLate = !KDA;
  if constexpr (kStageLate) {
    stage_chunk(jfirst * C + 1);
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);   // the state tile (see kWaitVmem0)
  }
  for (int j = jfirst; j <= jlast; ++j) {
    const int cpos = j * C + 1;              // position of slot 0
    // the pool row of a page this chunk fills (GDN: scalar load, see load_index_uniform)
    const bool page_end = to_page_end == 0 && cpos + C - 1 < pos_last;
    const int64_t page_row = (page_end && kStageLate) ? load_index_uniform(p.page_indices, page_slot, p.idx64) : 0;
    if constexpr (!kStageLate) stage_chunk(cpos);
    if (j < jlast) load_chunk(cpos + C);     // next chunk's inputs, in flight during this chunk
    __syncthreads();

    if constexpr (KDA) {
      // ---- per-channel gate prefix and the gated keys / queries (one thread
      //      per channel); every exponent is <= 0 since g <= 0
      if (tid < K) {
        const int c = tid;
        float G = 0.0f;
#pragma unroll
        for (int t = 0; t < C; ++t) {
          G += s_G[t][c];
          s_G[t][c] = G;
          const float e = exp_hw(G);
          s_kg[t][c] = s_k[t][c] * e;
          s_qg[t][c] = s_q[t][c] * e;
        }
#pragma unroll
        for (int t = 0; t < C; ++t) s_kd[t][c] = exp_hw(fminf(G - s_G[t][c], 0.0f)) * s_k[t][c];
        s_eC[c] = exp_hw(G);
      }
      __syncthreads();
    }

    // ---- gate prefix (GDN, every wave): inclusive scan of g over the 16 lanes
    //      of each row (row_shr:n with bound_ctrl, so the first n lanes add 0)
    float Gc = KDA ? 0.0f : s_g[n16];         // becomes G of column s = n16
    Gc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Gc), 0x111, 0xF, 0xF, true));
    Gc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Gc), 0x112, 0xF, 0xF, true));
    Gc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Gc), 0x114, 0xF, 0xF, true));
    Gc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Gc), 0x118, 0xF, 0xF, true));
    float Gr[4];                              // G of rows t = 4 g4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) Gr[r] = __shfl(Gc, 4 * g4 + r);
    const float GC = __shfl(Gc, C - 1);       // G of the last slot

    // ---- key interaction A' and output score P, 16 x 16 over K
    if constexpr (KDA) {
      // per-channel decay: sum_c x_tc k_sc exp(G_tc - G_sc) does not factor into
      // one product without overflow risk; pairs (t, s) on the VALU, PPT per thread
#pragma unroll
      for (int pp = 0; pp < PPT; ++pp) {
        const int pi = tid + pp * NW * 64;
        const int t = pi >> 4, s = pi & 15;
        float a = 0.0f, pq = 0.0f;
        if (s <= t) {
#pragma unroll 4
          for (int c = 0; c < K; c += 4) {
            const float4 kt = *reinterpret_cast<const float4*>(&s_k[t][c]);
            const float4 qt = *reinterpret_cast<const float4*>(&s_q[t][c]);
            const float4 Gt = *reinterpret_cast<const float4*>(&s_G[t][c]);
            const float4 ks = *reinterpret_cast<const float4*>(&s_k[s][c]);
            const float4 Gs = *reinterpret_cast<const float4*>(&s_G[s][c]);
            const float e0 = exp_hw(fminf(Gt.x - Gs.x, 0.0f)) * ks.x, e1 = exp_hw(fminf(Gt.y - Gs.y, 0.0f)) * ks.y;
            const float e2 = exp_hw(fminf(Gt.z - Gs.z, 0.0f)) * ks.z, e3 = exp_hw(fminf(Gt.w - Gs.w, 0.0f)) * ks.w;
            a = fmaf(kt.x, e0, fmaf(kt.y, e1, fmaf(kt.z, e2, fmaf(kt.w, e3, a))));
            pq = fmaf(qt.x, e0, fmaf(qt.y, e1, fmaf(qt.z, e2, fmaf(qt.w, e3, pq))));
          }
        }
        s_a[t][s] = (s < t) ? s_b[t] * a : 0.0f;
        s_p[t][s] = (s <= t) ? pq : 0.0f;
      }
    } else if (w < 2) {
      const float(*left)[LDK] = (w == 0) ? s_k : s_q;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c4 = 0; c4 < K / 4; ++c4) acc = mfma_16x16x4(left[n16][4 * c4 + g4], s_k[n16][4 * c4 + g4], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * g4 + r, s = n16;
        const float d = exp_hw(fminf(Gr[r] - Gc, 0.0f));
        if (w == 0) s_a[t][s] = (s < t) ? s_b[t] * d * acc[r] : 0.0f;
        else s_p[t][s] = (s <= t) ? d * acc[r] : 0.0f;
      }
    }

    // ---- KS = K S0 and QS = Q S0 for this wave's columns (A operands: row n16,
    //      columns 16 ct + 4 g4 + r; B: the state accumulators)
    f32x4 KS[VT], O[VT];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      KS[vt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      O[vt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      if (kDeferStore && store_pending) store_rows(pending_row, ct);   // the previous chunk's page
      // (KDA: the per-channel exp(G_t) is folded into the gated rows)
      const float4 kv = *reinterpret_cast<const float4*>(KDA ? &s_kg[n16][16 * ct + 4 * g4] : &s_k[n16][16 * ct + 4 * g4]);
      const float4 qv = *reinterpret_cast<const float4*>(KDA ? &s_qg[n16][16 * ct + 4 * g4] : &s_q[n16][16 * ct + 4 * g4]);
      const float kr[4] = {kv.x, kv.y, kv.z, kv.w};
      const float qr[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          KS[vt] = mfma_16x16x4(kr[r], S[ct][vt][r], KS[vt]);
          O[vt] = mfma_16x16x4(qr[r], S[ct][vt][r], O[vt]);
        }
    }
    __syncthreads();                          // A' and P visible

    // ---- exact solve T = (I + A')^-1 by forward substitution (every wave its
    //      own copy: lane n16 < 16 computes column n16)
    if (lane < C) {
      float x[C];
#pragma unroll
      for (int t = 0; t < C; ++t) {
        float acc = (t == lane) ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < t; ++s) acc = fmaf(-s_a[t][s], x[s], acc);
        x[t] = acc;
        s_t[w][t][lane] = acc;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // T is read by the other lanes of this wave
    __builtin_amdgcn_wave_barrier();

    // ---- U = T diag(beta) (V - diag(exp G) K S0): R in accumulator layout
    //      (rows s = 4 g4 + r) is the B operand; A = T[n16][4 g4 + r] beta
    float eG[4];                    // GDN: exp(G_t) of rows t = 4 g4 + r (KDA: folded, 1)
#pragma unroll
    for (int r = 0; r < 4; ++r) eG[r] = KDA ? 1.0f : exp_hw(Gr[r]);
    f32x4 U[VT];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      f32x4 R;
#pragma unroll
      for (int r = 0; r < 4; ++r) R[r] = s_v[4 * g4 + r][16 * VT * w + 16 * vt + n16] - eG[r] * KS[vt][r];
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mfma_16x16x4(s_t[w][n16][4 * g4 + r] * s_b[4 * g4 + r], R[r], acc);
      U[vt] = acc;
    }

    // ---- O = diag(exp G) Q S0 + P U   (B = U rows s = 4 g4 + r)
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) O[vt][r] *= eG[r];   // (KDA: times 1)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pa = s_p[n16][4 * g4 + r];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) O[vt] = mfma_16x16x4(pa, U[vt][r], O[vt]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = cpos + 4 * g4 + r;
      if (pos >= pos0 && pos <= pos_last) {
        const int64_t t = t0 + (pos - pos0);
        const int64_t oi = (t * p.HV + h) * p.V + vcol + n16;
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
          if (p.out_bf16) static_cast<uint16_t*>(p.out)[oi + 16 * vt] = to_bf16_bits(O[vt][r]);
          else static_cast<float*>(p.out)[oi + 16 * vt] = O[vt][r];
        }
      }
    }

    // ---- S_C = exp(G_C) S0 + sum_s exp(G_C - G_s) k_s u_s^T
    const float eC = exp_hw(GC);
    float dk[4];                    // exp(G_C - G_s) for s = 4 g4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) dk[r] = exp_hw(fminf(GC - Gr[r], 0.0f));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      float ka[4];                  // A[ch = 16 ct + n16][s = 4 g4 + r]
#pragma unroll
      for (int r = 0; r < 4; ++r) ka[r] = KDA ? s_kd[4 * g4 + r][16 * ct + n16] : dk[r] * s_k[4 * g4 + r][16 * ct + n16];
      f32x4 dec = {eC, eC, eC, eC};   // decay of rows 16 ct + 4 g4 + r (KDA: per channel)
      if constexpr (KDA) dec = *reinterpret_cast<const f32x4*>(&s_eC[16 * ct + 4 * g4]);
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        f32x4 acc = S[ct][vt] * dec;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mfma_16x16x4(ka[r], U[vt][r], acc);
        S[ct][vt] = acc;
      }
    }

    // ---- a page that ends inside the suffix gets the state after its last token
    store_pending = false;
    if (to_page_end == 0) {
      if (page_end) {
        const int64_t row = kStageLate ? page_row : load_index(p.page_indices, page_slot, p.idx64);
        if constexpr (kDeferStore) {   // stored during the next chunk (page_end implies that chunk exists)
          store_pending = true;
          pending_row = row;
        } else {
          store_state(row);
        }
      }
      to_page_end = cpp;
      ++page_slot;
    }
    --to_page_end;
    __syncthreads();                // LDS is rewritten by the next chunk
    if constexpr (kStageLate) {
      if (j < jlast) stage_chunk(cpos + C);
    }
  }

  store_state(wrow);
}

}  // namespace gdn

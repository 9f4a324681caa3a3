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
//     W    = T diag(beta exp(G)) K,   U~ = T diag(beta) V
//     U    = U~ - W S0
//     O    = diag(exp G) Q S0 + P U,  P = lower( exp(G_t - G_s) q_t . k_s )
//     S_C  = exp(G_C) S0 + sum_s exp(G_C - G_s) k_s u_s^T
// Every exponent is <= 0.  Chunks are aligned to absolute token positions
// (16 j + 1 .. 16 j + 16), so with a page size that is a multiple of 16 every
// page end is a chunk end and its state is S_C of that chunk.  Positions of a
// chunk outside the suffix are identity tokens (k = q = v = 0, beta = 0,
// g = 0): their rows of A', W, U~ and U are zero and T is the identity on
// them, so they change nothing.
//
// One workgroup per (sequence, value head, 128-column V-block), 4 waves; wave
// w owns value columns [32 w, 32 w + 32) of the block and keeps S[:, those]
// (128 x 32) as 16 MFMA accumulator tiles for the whole suffix.  The
// products that involve S use the accumulator registers directly as the B
// operand of v_mfma_f32_16x16x4_f32: a lane holds S rows 4 g + r of a tile
// (g = lane / 16), so the k-step r pairs B = element r with A = the matching
// column 16 ct + 4 g + r of the left factor.  The K-side quantities (A', P,
// T, W) are computed once per workgroup and shared through LDS.
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
  const void* gate;        // a [T, HV]
  const void* beta;        // b [T, HV]
  const float* a_log;      // [HV]
  const float* dt_bias;    // [HV]
  const int32_t* cu_seqlens;
  const void* page_indices;
  const void* page_indptr;
  const void* last_page_len;
  int32_t page_size;
  float* pool;
  void* out;
  int32_t B, HK, HV, V;
  int32_t nvb;             // V / 128
  int32_t gqa;
  float scale;
  int32_t l2norm, out_bf16, beta_prob, idx64;
};

constexpr int kChunk = 16;

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <bool VF, typename TIn>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillParams p) {
  constexpr int K = 128, C = kChunk, NW = 4;
  constexpr int LDK = K + 4;       // padded LDS rows
  constexpr int LDC = C + 1;

  __shared__ __align__(16) float s_q[C][LDK];   // q_hat (scaled)
  __shared__ __align__(16) float s_k[C][LDK];   // k_hat
  __shared__ __align__(16) float s_v[C][LDK];   // v of this V-block
  __shared__ __align__(16) float s_w[C][LDK];   // W
  __shared__ float s_a[C][LDC];                 // A' (strict lower)
  __shared__ float s_p[C][LDC];                 // P (lower, diagonal included)
  __shared__ float s_t[C][LDC];                 // T = (I + A')^-1
  __shared__ float s_g[C], s_b[C], s_G[C];

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

  const int unit = blockIdx.x;
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
  const int64_t pg_start = load_index(p.page_indptr, bs, p.idx64);
  const int64_t pg_end = load_index(p.page_indptr, bs + 1, p.idx64);
  const int64_t lpl = load_index(p.last_page_len, bs, p.idx64);
  const int64_t pos_last = (pg_end - pg_start - 1) * p.page_size + lpl;
  const int64_t pos0 = pos_last - (t1 - t0) + 1;
  const int64_t rrow =
      load_index(p.page_indices, pg_start + max(pos0 - 2, static_cast<int64_t>(0)) / p.page_size, p.idx64);
  const int64_t wrow = load_index(p.page_indices, pg_end - 1, p.idx64);

  const int64_t tile_elems = static_cast<int64_t>(K) * p.V;
  const int vcol = vb * 128 + 32 * w;   // first value column of this wave

  // S[ct][vt] element r = S[16 ct + 4 g4 + r][vcol + 16 vt + n16]
  f32x4 S[8][2];
  auto state_off = [&](int ct, int vt, int r) -> int64_t {
    const int64_t ch = 16 * ct + 4 * g4 + r;
    const int64_t v = vcol + 16 * vt + n16;
    return VF ? v * K + ch : ch * p.V + v;
  };
  {
    const float* src = p.pool + (rrow * p.HV + h) * tile_elems;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        if constexpr (VF) {
          S[ct][vt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + state_off(ct, vt, 0)));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) S[ct][vt][r] = __builtin_nontemporal_load(src + state_off(ct, vt, r));
        }
      }
  }
  auto store_state = [&](int64_t row) {
    float* dst = p.pool + (row * p.HV + h) * tile_elems;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        if constexpr (VF) {
          *reinterpret_cast<f32x4*>(dst + state_off(ct, vt, 0)) = S[ct][vt];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[state_off(ct, vt, r)] = S[ct][vt][r];
        }
      }
  };

  const float rate = exp_hw(p.a_log[h]);
  const float dtb = p.dt_bias[h];
  const int64_t jfirst = (pos0 - 1) / C;
  const int64_t jlast = (pos_last - 1) / C;

  for (int64_t j = jfirst; j <= jlast; ++j) {
    const int64_t cpos = j * C + 1;          // position of slot 0

    // ---- stage the chunk's inputs: wave w normalises slots 4 w .. 4 w + 3
#pragma unroll
    for (int i = 0; i < C / NW; ++i) {
      const int slot = w * (C / NW) + i;
      const int64_t pos = cpos + slot;
      float xq[2] = {0.0f, 0.0f}, xk[2] = {0.0f, 0.0f}, xv[2] = {0.0f, 0.0f};
      float gt = 0.0f, bt = 0.0f;
      if (pos >= pos0 && pos <= pos_last) {  // uniform per wave
        const int64_t t = t0 + (pos - pos0);
        Raw<TIn, 2> rq, rk, rv;
        Raw<TIn, 1> ra, rb;
        load_raw_n<2>(gq, (t * p.HK + hk) * K + 2 * lane, rq);
        load_raw_n<2>(gk, (t * p.HK + hk) * K + 2 * lane, rk);
        load_raw_n<2>(gv, (t * p.HV + h) * p.V + vb * 128 + 2 * lane, rv);
        load_raw_n<1>(gg, t * p.HV + h, ra);
        load_raw_n<1>(gb, t * p.HV + h, rb);
        decode_raw(rq, xq);
        decode_raw(rk, xk);
        decode_raw(rv, xv);
        float xa[1], xb[1];
        decode_raw(ra, xa);
        decode_raw(rb, xb);
        float iq = p.scale, ik = 1.0f;
        if (p.l2norm) {
          iq = p.scale * rsqrtf(lane_reduce<0, 6>(fmaf(xq[0], xq[0], xq[1] * xq[1])) + kL2Eps);
          ik = rsqrtf(lane_reduce<0, 6>(fmaf(xk[0], xk[0], xk[1] * xk[1])) + kL2Eps);
        }
        xq[0] *= iq;
        xq[1] *= iq;
        xk[0] *= ik;
        xk[1] *= ik;
        gt = -rate * softplus_f(xa[0] + dtb);
        bt = p.beta_prob ? xb[0] : sigmoid_f(xb[0]);
      }
      *reinterpret_cast<float2*>(&s_q[slot][2 * lane]) = make_float2(xq[0], xq[1]);
      *reinterpret_cast<float2*>(&s_k[slot][2 * lane]) = make_float2(xk[0], xk[1]);
      *reinterpret_cast<float2*>(&s_v[slot][2 * lane]) = make_float2(xv[0], xv[1]);
      if (lane == 0) {
        s_g[slot] = gt;
        s_b[slot] = bt;
      }
    }
    __syncthreads();

    // ---- gate prefix, key interaction (wave 0) and output score (wave 1)
    if (w < 2) {
      float G = 0.0f;                         // G of column s = n16
      float Gr[4] = {0.0f, 0.0f, 0.0f, 0.0f}; // G of rows t = 4 g4 + r
#pragma unroll
      for (int s = 0; s < C; ++s) {
        G += (s <= n16) ? s_g[s] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) Gr[r] += (s <= 4 * g4 + r) ? s_g[s] : 0.0f;
      }
      if (w == 0 && lane < C) s_G[lane] = G;
      const float(*left)[LDK] = (w == 0) ? s_k : s_q;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c4 = 0; c4 < K / 4; ++c4) acc = mfma_16x16x4(left[n16][4 * c4 + g4], s_k[n16][4 * c4 + g4], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * g4 + r, s = n16;
        const float d = exp_hw(fminf(Gr[r] - G, 0.0f));
        if (w == 0) s_a[t][s] = (s < t) ? s_b[t] * d * acc[r] : 0.0f;
        else s_p[t][s] = (s <= t) ? d * acc[r] : 0.0f;
      }
    }
    __syncthreads();

    // ---- exact solve T = (I + A')^-1 by forward substitution, column n16 per lane
    if (w == 0 && lane < C) {
      float x[C];
#pragma unroll
      for (int t = 0; t < C; ++t) {
        float acc = (t == lane) ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < t; ++s) acc = fmaf(-s_a[t][s], x[s], acc);
        x[t] = acc;
        s_t[t][lane] = acc;
      }
    }
    __syncthreads();

    // ---- W = T diag(beta exp G) K (two column tiles per wave) and U~ = T diag(beta) V
    f32x4 U[2];
    {
      float tb[4], tbe[4];          // A operands: T[t = n16][s = 4 st + g4] * beta_s (* exp G_s)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int s = 4 * st + g4;
        tb[st] = s_t[n16][s] * s_b[s];
        tbe[st] = tb[st] * exp_hw(s_G[s]);
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int ct = 2 * w + cc;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma_16x16x4(tbe[st], s_k[4 * st + g4][16 * ct + n16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) s_w[4 * g4 + r][16 * ct + n16] = acc[r];
      }
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma_16x16x4(tb[st], s_v[4 * st + g4][32 * w + 16 * vt + n16], acc);
        U[vt] = acc;
      }
    }
    __syncthreads();

    // ---- U = U~ - W S0 and O1 = Q S0 (A operands: row n16, columns 16 ct + 4 g4 + r)
    f32x4 O[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const float4 wv = *reinterpret_cast<const float4*>(&s_w[n16][16 * ct + 4 * g4]);
      const float4 qv = *reinterpret_cast<const float4*>(&s_q[n16][16 * ct + 4 * g4]);
      const float wr[4] = {-wv.x, -wv.y, -wv.z, -wv.w};
      const float qr[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          U[vt] = mfma_16x16x4(wr[r], S[ct][vt][r], U[vt]);
          O[vt] = mfma_16x16x4(qr[r], S[ct][vt][r], O[vt]);
        }
    }

    // ---- O = diag(exp G) O1 + P U   (B = U rows s = 4 g4 + r)
    float eG[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) eG[r] = exp_hw(s_G[4 * g4 + r]);
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) O[vt][r] *= eG[r];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pa = s_p[n16][4 * g4 + r];
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) O[vt] = mfma_16x16x4(pa, U[vt][r], O[vt]);
    }
    // outputs of the suffix tokens among rows t = 4 g4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t pos = cpos + 4 * g4 + r;
      if (pos >= pos0 && pos <= pos_last) {
        const int64_t t = t0 + (pos - pos0);
        const int64_t oi = (t * p.HV + h) * p.V + vcol + n16;
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
          if (p.out_bf16) static_cast<uint16_t*>(p.out)[oi + 16 * vt] = to_bf16_bits(O[vt][r]);
          else static_cast<float*>(p.out)[oi + 16 * vt] = O[vt][r];
        }
      }
    }

    // ---- S_C = exp(G_C) S0 + sum_s exp(G_C - G_s) k_s u_s^T
    const float GC = s_G[C - 1];
    const float eC = exp_hw(GC);
    float dk[4];                    // exp(G_C - G_s) for s = 4 g4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) dk[r] = exp_hw(fminf(GC - s_G[4 * g4 + r], 0.0f));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      float ka[4];                  // A[ch = 16 ct + n16][s = 4 g4 + r]
#pragma unroll
      for (int r = 0; r < 4; ++r) ka[r] = dk[r] * s_k[4 * g4 + r][16 * ct + n16];
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        f32x4 acc = S[ct][vt] * eC;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mfma_16x16x4(ka[r], U[vt][r], acc);
        S[ct][vt] = acc;
      }
    }

    // ---- a page that ends inside the suffix gets the state after its last token
    const int64_t pend = cpos + C - 1;
    if (pend % p.page_size == 0 && pend < pos_last)
      store_state(load_index(p.page_indices, pg_start + (pend - 1) / p.page_size, p.idx64));
    __syncthreads();                // LDS is rewritten by the next chunk
  }

  store_state(wrow);
}

}  // namespace gdn

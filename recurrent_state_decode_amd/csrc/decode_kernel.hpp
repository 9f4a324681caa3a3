// Device side of the gated delta-rule decode: one workgroup per
// (sequence, value head, V-block) work unit.
//
// Math per token (Circuit.LLM.Mixer, "Delta rule" and "Gated memory";
// max.nn.state_space.kda_decode, description): decay the state, read what
// the key retrieves, write the delta, read the updated state out.  The
// kernel evaluates it in a fused form that needs one pass over the state
// per token:
//     r = k'^T S, p = q'^T S          (k' = k_hat*alpha, q' = q_hat*alpha)
//     u = beta * (v - r)
//     o = p + (q_hat . k_hat) * u     (= q_hat^T S_new)
//     S = alpha*S + k_hat u^T
// which is the same arithmetic regrouped (alpha is a scalar for GDN, applied
// after the reduction, and a per-key-row vector for KDA).
//
// Layout of the state tile in registers.  Each thread owns NS memory rows of
// 4 consecutive floats (one 128-bit load per row); consecutive lanes cover a
// contiguous memory row, so every wave-wide load or store is fully
// coalesced:
//   K_FIRST (V contiguous): memory row = key index i, 4 value columns per
//       thread; the K-reduction is in-thread over NS rows, then across the
//       row groups of a wave (lane bits above log2(VB/4)), then across waves
//       through LDS.
//   V_FIRST (K contiguous): memory row = value index j, 4 key elements per
//       thread; the K-reduction is 4-wide in-thread, then across the K/4
//       lanes of the row (the low lane bits); no cross-wave step.
// Cross-lane sums use DPP (quad permutes, row mirrors and rotates) inside a
// 16-lane row and the gfx950 v_permlane16_swap / v_permlane32_swap across
// rows, so no reduction goes through LDS except the cross-wave one.
//
// Latency: the per-token inputs of the first chunk are loaded before the
// state tile and normalised while the tile is in flight.
//
// Work order: the hardware hands consecutive workgroup ids to the 8 XCDs in
// turn.  The kernel renumbers them so that runs of xcd_group consecutive work
// units (neighbouring V-blocks and heads of one sequence) execute on the same
// XCD: they share that XCD's L2 for q/k/v and stream one contiguous slice of
// the work instead of eight interleaved ones.  The state tile is read with
// non-temporal loads: it is touched once per call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;        // GDN: a [T, HV]; KDA: raw_gate [T, HV, K]
  const void* beta;        // b / beta_logits [T, HV]
  const float* a_log;      // [HV]
  const float* dt_bias;    // GDN: [HV]; KDA: [HV, K]
  const int32_t* cu_seqlens;     // pooled, may be null
  const int32_t* state_indices;  // pooled
  const void* page_indices;      // paged
  const void* page_indptr;
  const void* last_page_len;
  float* pool;
  void* out;
  int32_t B, HK, HV, V;
  int32_t nvb;             // V / VB
  int32_t gqa;             // HV / HK
  float scale;
  int32_t l2norm;
  int32_t out_bf16;
  int32_t beta_prob;
  int32_t idx64;
  int32_t quantize_initial;
  int32_t readout_stored;
  int32_t xcd_group;       // consecutive work units kept on one XCD (>= 1)
};

constexpr float kL2Eps = 1e-6f;
constexpr float kE4M3Max = 448.0f;
constexpr int kTokensPerChunk = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 inputs are carried as their 16-bit patterns
struct bf16_t {
  uint16_t bits;
};

// Raw 32-bit words holding N consecutive input elements; kept undecoded so
// that the loads stay in flight until the values are needed.
template <typename TIn, int N>
struct Raw {
  static constexpr int W = (N * static_cast<int>(sizeof(TIn)) + 3) / 4;
  uint32_t w[W];
};

template <int N, typename TIn>
__device__ __forceinline__ void load_raw_n(const TIn* p, int64_t i, Raw<TIn, N>& r) {
  if constexpr (sizeof(TIn) == 2 && N == 1) {
    r.w[0] = reinterpret_cast<const uint16_t*>(p)[i];
  } else if constexpr (sizeof(TIn) == 2 && N == 2) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p + i);
  } else if constexpr (sizeof(TIn) == 2 && N == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p + i);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else if constexpr (sizeof(TIn) == 4 && N == 1) {
    r.w[0] = reinterpret_cast<const uint32_t*>(p)[i];
  } else if constexpr (sizeof(TIn) == 4 && N == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p + i);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else {
    static_assert(sizeof(TIn) == 4 && N == 4, "unsupported raw load");
    const uint4 v = *reinterpret_cast<const uint4*>(p + i);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  }
}

template <int N, typename TIn>
__device__ __forceinline__ void decode_raw(const Raw<TIn, N>& r, float (&x)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if constexpr (sizeof(TIn) == 2) {
      const uint32_t word = r.w[j / 2];
      x[j] = __uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
    } else {
      x[j] = __uint_as_float(r.w[j]);
    }
  }
}

__device__ __forceinline__ int64_t load_index(const void* p, int64_t i, int idx64) {
  return idx64 ? static_cast<const int64_t*>(p)[i] : static_cast<int64_t>(static_cast<const int32_t*>(p)[i]);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  const __bf16 h = static_cast<__bf16>(x);   // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// ---- cross-lane primitives (wave64)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// x + the value of the lane in the other 16-lane row of the same 32-lane half
__device__ __forceinline__ float sum_rows16(float x) {
  const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// x + the value of the lane in the other 32-lane half
__device__ __forceinline__ float sum_halves32(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Sum over the lanes that differ from this one only in lane-index bits
// [LO, HI); every lane receives the sum.  DPP controls: quad_perm 0xB1 swaps
// lanes 2n and 2n+1, 0x4E swaps pairs 0-1 and 2-3, row_half_mirror (0x141)
// reverses each group of 8, row_ror:8 (0x128) and row_ror:4 (0x124) rotate a
// 16-lane row.  Each step adds a lane set disjoint from the one gathered so
// far, so every lane of the group is counted exactly once.
template <int LO, int HI>
__device__ __forceinline__ float lane_sum(float x) {
  static_assert(0 <= LO && LO < HI && HI <= 6, "lane bits");
  constexpr bool b0 = LO <= 0 && 0 < HI, b1 = LO <= 1 && 1 < HI, b2 = LO <= 2 && 2 < HI;
  constexpr bool b3 = LO <= 3 && 3 < HI, b4 = LO <= 4 && 4 < HI, b5 = LO <= 5 && 5 < HI;
  if constexpr (b0) x += dpp<0xB1>(x);
  if constexpr (b1) x += dpp<0x4E>(x);
  if constexpr (b2) {
    static_assert((b0 && b1) || b3, "bit 2 needs bits 0-1 (mirror) or bit 3 (rotate)");
    if constexpr (b0 && b1) {
      x += dpp<0x141>(x);                  // lanes i and 7-i: together with bits 0,1 covers the 8
      if constexpr (b3) x += dpp<0x128>(x);
    } else {
      x += dpp<0x128>(x);                  // i and i+8
      x += dpp<0x124>(x);                  // then i-4: {i, i-4, i-8, i-12}
    }
  } else if constexpr (b3) {
    x += dpp<0x128>(x);
  }
  if constexpr (b4) x = sum_rows16(x);
  if constexpr (b5) x = sum_halves32(x);
  return x;
}

template <int HI>
__device__ __forceinline__ float lane_max(float x) {
  // max over lane bits [0, HI): butterflies through LDS-free swizzles
#pragma unroll
  for (int o = 1; o < (1 << HI); o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Round x0, x1 (already divided by the tile scale) to the E4M3 grid and back
// with the gfx950 OCP fp8 conversions (nearest even).
__device__ __forceinline__ void e4m3_roundtrip2(float& x0, float& x1) {
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  const auto back = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
  x0 = back[0];
  x1 = back[1];
}

template <int K, int VB, int NT, bool VF>
struct Tile {
  static constexpr int NW = NT / 64;
  static constexpr int LR = VF ? K / 4 : VB / 4;   // lanes covering one memory row
  static constexpr int RPW = 64 / LR;              // memory rows per wave per load step
  static constexpr int ROWS = VF ? VB : K;         // memory rows of the tile
  static constexpr int NS = ROWS / (NW * RPW);     // rows per thread
  static constexpr int LB = __builtin_ctz(LR);     // lane bits inside a memory row
  static_assert(NT % 64 == 0, "whole waves");
  static_assert(LR >= 1 && LR <= 64 && 64 % LR == 0, "row must fit a wave");
  static_assert(ROWS % (NW * RPW) == 0 && NS >= 1, "tile must split evenly");
  static_assert(!VF || NS <= LR, "V_FIRST output store uses one lane per row");
  static_assert(K % 4 == 0 && VB % 4 == 0, "128-bit rows");
};

template <int K, int VB, int NT, bool VF, bool KDA, bool QDQ, bool PAGED, typename TIn>
__global__ __launch_bounds__(NT) void decode_kernel(const Params p) {
  using Cfg = Tile<K, VB, NT, VF>;
  constexpr int NW = Cfg::NW, LR = Cfg::LR, RPW = Cfg::RPW, NS = Cfg::NS, LB = Cfg::LB;
  constexpr int TC = kTokensPerChunk;
  constexpr int TPW = (TC + NW - 1) / NW;          // tokens per wave in a chunk
  constexpr int EPL = (K + 63) / 64;               // q/k/gate elements per lane (contiguous)
  constexpr int EL = K / EPL;                      // lanes holding q/k elements
  constexpr int VPL = (VB + 63) / 64;              // v elements per lane
  constexpr int VL = VB / VPL;                     // lanes holding v elements
  constexpr int GPL = KDA ? EPL : 1;
  constexpr int KX = KDA ? K : 1;                  // extent of KDA-only arrays
  constexpr int TX = KDA ? TC : 1;
  constexpr int TQ = (KDA && QDQ) ? TC : 1;
  constexpr int KQ = (KDA && QDQ) ? K : 1;
  static_assert(K % EPL == 0 && VB % VPL == 0, "input split");

  __shared__ __align__(16) float s_q[TC][K];       // reduction coefficient of p (q_hat, KDA: *alpha)
  __shared__ __align__(16) float s_k[TC][K];       // reduction coefficient of r (k_hat, KDA: *alpha)
  __shared__ __align__(16) float s_kh[TX][KX];     // KDA: k_hat for the write
  __shared__ __align__(16) float s_al[TX][KX];     // KDA: alpha per key channel
  __shared__ __align__(16) float s_qh[TQ][KQ];     // KDA + stored readout: plain q_hat
  __shared__ __align__(16) float s_v[TC][VB];      // this V-block of v
  __shared__ float s_sc[TC][4];                    // alpha (GDN), beta, q_hat . k_hat
  __shared__ __align__(16) float s_red[VF ? 1 : 2][VF ? 1 : NW][2][VB];
  __shared__ float s_max[NW];

  const TIn* __restrict__ gq = static_cast<const TIn*>(p.q);
  const TIn* __restrict__ gk = static_cast<const TIn*>(p.k);
  const TIn* __restrict__ gv = static_cast<const TIn*>(p.v);
  const TIn* __restrict__ gg = static_cast<const TIn*>(p.gate);
  const TIn* __restrict__ gb = static_cast<const TIn*>(p.beta);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane % LR;        // position inside a memory row (x4 floats)
  const int rg = lane / LR;        // row group inside the wave

  // renumber workgroups: within each span of 8 * G ids, XCD x (id % 8) gets
  // units [x * G, (x + 1) * G) of that span; ids past the last full span keep
  // their number.  A permutation of [0, gridDim.x) for every G >= 1.
  const int bx = blockIdx.x;
  const int G = p.xcd_group;
  const int span = 8 * G;
  const int nfull = (static_cast<int>(gridDim.x) / span) * span;
  const int unit = bx < nfull ? (bx / span) * span + (bx % 8) * G + (bx / 8) % G : bx;
  const int vb = unit % p.nvb;
  const int h = (unit / p.nvb) % p.HV;
  const int bs = unit / (p.nvb * p.HV);
  const int hk = h / p.gqa;
  const int64_t out_col0 = static_cast<int64_t>(vb) * VB;

  // ---- which tokens
  int t0, t1;
  if constexpr (PAGED) {
    t0 = bs;
    t1 = bs + 1;
  } else {
    if (p.cu_seqlens) {
      t0 = p.cu_seqlens[bs];
      t1 = p.cu_seqlens[bs + 1];
    } else {
      t0 = bs;
      t1 = bs + 1;
    }
  }
  if (t1 <= t0) return;            // empty suffix: no read, no write

  // ---- raw per-token inputs of one chunk (each wave loads its own tokens)
  Raw<TIn, EPL> rq[TPW], rk[TPW];
  Raw<TIn, GPL> rgt[TPW];
  Raw<TIn, VPL> rv[TPW];
  Raw<TIn, 1> rb[TPW];
  auto load_raw = [&](int c0, int n) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tt = w + NW * i;
      if (tt < n) {
        const int64_t t = c0 + tt;
        if (lane < EL) {
          const int64_t qo = (t * p.HK + hk) * K + EPL * lane;
          load_raw_n<EPL>(gq, qo, rq[i]);
          load_raw_n<EPL>(gk, qo, rk[i]);
          if constexpr (KDA) load_raw_n<EPL>(gg, (t * p.HV + h) * K + EPL * lane, rgt[i]);
        }
        if constexpr (!KDA) load_raw_n<1>(gg, t * p.HV + h, rgt[i]);
        load_raw_n<1>(gb, t * p.HV + h, rb[i]);
        if (lane < VL) load_raw_n<VPL>(gv, (t * p.HV + h) * p.V + out_col0 + VPL * lane, rv[i]);
      }
    }
  };
  // normalise, gate and stage one chunk's tokens in LDS
  auto finish_raw = [&](int n) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tt = w + NW * i;
      if (tt < n) {
        float xq[EPL], xk[EPL], xg[GPL], xv[VPL], xb[1];
        decode_raw(rq[i], xq);
        decode_raw(rk[i], xk);
        decode_raw(rgt[i], xg);
        decode_raw(rv[i], xv);
        decode_raw(rb[i], xb);
        float ssq = 0.0f, ssk = 0.0f;
        if (lane < EL) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            ssq = fmaf(xq[e], xq[e], ssq);
            ssk = fmaf(xk[e], xk[e], ssk);
          }
        }
        float iq = p.scale, ik = 1.0f;
        if (p.l2norm) {
          iq = p.scale * rsqrtf(lane_sum<0, 6>(ssq) + kL2Eps);
          ik = rsqrtf(lane_sum<0, 6>(ssk) + kL2Eps);
        }
        float qk = 0.0f;
        if (lane < EL) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            xq[e] *= iq;
            xk[e] *= ik;
            qk = fmaf(xq[e], xk[e], qk);
          }
        }
        qk = lane_sum<0, 6>(qk);
        const float beta = p.beta_prob ? xb[0] : sigmoid_f(xb[0]);
        if (lane < EL) {
          if constexpr (KDA) {
            const float rate = expf(p.a_log[h]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const int c = EPL * lane + e;
              const float al = expf(-rate * softplus_f(xg[e] + p.dt_bias[h * K + c]));
              s_q[tt][c] = xq[e] * al;
              s_k[tt][c] = xk[e] * al;
              s_kh[tt][c] = xk[e];
              s_al[tt][c] = al;
              if constexpr (QDQ) s_qh[tt][c] = xq[e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              s_q[tt][EPL * lane + e] = xq[e];
              s_k[tt][EPL * lane + e] = xk[e];
            }
          }
        }
        if (lane < VL) {
#pragma unroll
          for (int e = 0; e < VPL; ++e) s_v[tt][VPL * lane + e] = xv[e];
        }
        if (lane == 0) {
          if constexpr (!KDA) s_sc[tt][0] = expf(-expf(p.a_log[h]) * softplus_f(xg[0] + p.dt_bias[h]));
          s_sc[tt][1] = beta;
          s_sc[tt][2] = qk;
        }
      }
    }
  };

  const int n0 = min(TC, t1 - t0);
  load_raw(t0, n0);                // in flight while the pool rows are resolved and the tile loads

  // ---- which pool rows
  int64_t rrow, wrow;
  if constexpr (PAGED) {
    const int64_t end = load_index(p.page_indptr, bs + 1, p.idx64);
    const int64_t last = load_index(p.page_indices, end - 1, p.idx64);
    const int64_t lpl = load_index(p.last_page_len, bs, p.idx64);
    wrow = last;
    rrow = (lpl == 1) ? load_index(p.page_indices, end - 2, p.idx64) : last;
  } else {
    rrow = wrow = p.state_indices[bs];
  }

  const int64_t tile_elems = static_cast<int64_t>(K) * p.V;
  const float* src = p.pool + (rrow * p.HV + h) * tile_elems;
  float* dst = p.pool + (wrow * p.HV + h) * tile_elems;

  // memory offset of this thread's row s (start of its 4 floats)
  auto row_idx = [&](int s) -> int { return s * (NW * RPW) + w * RPW + rg; };
  auto row_off = [&](int s) -> int64_t {
    if constexpr (VF) return static_cast<int64_t>(vb * VB + row_idx(s)) * K + 4 * lr;
    else return static_cast<int64_t>(row_idx(s)) * p.V + vb * VB + 4 * lr;
  };

  float S[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + row_off(s)));
    S[s][0] = x.x;
    S[s][1] = x.y;
    S[s][2] = x.z;
    S[s][3] = x.w;
  }

  finish_raw(n0);                  // overlaps the tile load

  int red_buf = 0;

  auto block_max = [&](float m) -> float {
    m = lane_max<6>(m);
    if constexpr (NW > 1) {
      __syncthreads();             // previous readers of s_max are done
      if (lane == 0) s_max[w] = m;
      __syncthreads();
      m = s_max[0];
#pragma unroll
      for (int i = 1; i < NW; ++i) m = fmaxf(m, s_max[i]);
    }
    return m;
  };

  auto qdq_tile = [&]() {
    float m = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(S[s][e]));
    m = block_max(m);
    if (m > 0.0f) {
      const float inv = kE4M3Max / m;
      const float sc = m / kE4M3Max;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          float x0 = S[s][e] * inv, x1 = S[s][e + 1] * inv;
          e4m3_roundtrip2(x0, x1);
          S[s][e] = x0 * sc;
          S[s][e + 1] = x1 * sc;
        }
    }
  };

  // store 4 consecutive outputs (K_FIRST) or one (V_FIRST)
  auto store_out4 = [&](int64_t oi, const float (&o)[4]) {
    if (p.out_bf16) {
      uint2 pk;
      pk.x = to_bf16_bits(o[0]) | (static_cast<uint32_t>(to_bf16_bits(o[1])) << 16);
      pk.y = to_bf16_bits(o[2]) | (static_cast<uint32_t>(to_bf16_bits(o[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + oi) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.out) + oi) = make_float4(o[0], o[1], o[2], o[3]);
    }
  };
  auto store_out1 = [&](int64_t oi, float o) {
    if (p.out_bf16) static_cast<uint16_t*>(p.out)[oi] = to_bf16_bits(o);
    else static_cast<float*>(p.out)[oi] = o;
  };

  // K_FIRST: wave-level partial sums over this thread's rows -> block sums via LDS.
  // Lanes of a wave with equal lr hold the same 4 columns; they differ in lane bits >= LB.
  auto kfirst_reduce = [&](float (&r)[4], float (&pp)[4], bool need_p) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = lane_sum<LB, 6>(r[e]);
      if (need_p) pp[e] = lane_sum<LB, 6>(pp[e]);
    }
    if constexpr (NW > 1) {
      if (rg == 0) {
        *reinterpret_cast<float4*>(&s_red[red_buf][w][0][4 * lr]) = make_float4(r[0], r[1], r[2], r[3]);
        if (need_p)
          *reinterpret_cast<float4*>(&s_red[red_buf][w][1][4 * lr]) = make_float4(pp[0], pp[1], pp[2], pp[3]);
      }
      __syncthreads();
      float4 ra = *reinterpret_cast<const float4*>(&s_red[red_buf][0][0][4 * lr]);
      float4 pa = need_p ? *reinterpret_cast<const float4*>(&s_red[red_buf][0][1][4 * lr]) : float4{};
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        const float4 x = *reinterpret_cast<const float4*>(&s_red[red_buf][ww][0][4 * lr]);
        ra.x += x.x; ra.y += x.y; ra.z += x.z; ra.w += x.w;
        if (need_p) {
          const float4 y = *reinterpret_cast<const float4*>(&s_red[red_buf][ww][1][4 * lr]);
          pa.x += y.x; pa.y += y.y; pa.z += y.z; pa.w += y.w;
        }
      }
      r[0] = ra.x; r[1] = ra.y; r[2] = ra.z; r[3] = ra.w;
      pp[0] = pa.x; pp[1] = pa.y; pp[2] = pa.z; pp[3] = pa.w;
      red_buf ^= 1;
    }
  };

  if constexpr (QDQ) {
    if (p.quantize_initial) qdq_tile();
  }

  for (int c0 = t0; c0 < t1; c0 += TC) {
    const int n = min(TC, t1 - c0);
    if (c0 != t0) {
      __syncthreads();             // readers of the previous chunk are done
      load_raw(c0, n);
      finish_raw(n);
    }
    __syncthreads();

    for (int tt = 0; tt < n; ++tt) {
      const int t = c0 + tt;
      const float beta = s_sc[tt][1];
      const float qk = s_sc[tt][2];
      const float alpha = KDA ? 1.0f : s_sc[tt][0];   // GDN alpha is applied after the reduction
      const int64_t out_row = (static_cast<int64_t>(t) * p.HV + h) * p.V + out_col0;
      const bool stored = QDQ && p.readout_stored;

      if constexpr (!VF) {
        // K_FIRST: rows are key indices, 4 value columns per thread
        float r[4] = {0.f, 0.f, 0.f, 0.f}, pp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int i = row_idx(s);
          const float kr = s_k[tt][i], qr = s_q[tt][i];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = fmaf(kr, S[s][e], r[e]);
            pp[e] = fmaf(qr, S[s][e], pp[e]);
          }
        }
        kfirst_reduce(r, pp, true);
        float u[4], o[4];
        const float4 v4 = *reinterpret_cast<const float4*>(&s_v[tt][4 * lr]);
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u[e] = beta * (vv[e] - alpha * r[e]);
          o[e] = fmaf(qk, u[e], alpha * pp[e]);
        }
        const bool writer = (w == 0 && rg == 0);
        if (!stored && writer) store_out4(out_row + 4 * lr, o);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int i = row_idx(s);
          const float a_s = KDA ? s_al[tt][i] : alpha;
          const float kh = KDA ? s_kh[tt][i] : s_k[tt][i];
#pragma unroll
          for (int e = 0; e < 4; ++e) S[s][e] = fmaf(a_s, S[s][e], kh * u[e]);
        }
        if constexpr (QDQ) {
          qdq_tile();
          if (stored) {
            // o = q_hat^T S after rounding
            float ps[4] = {0.f, 0.f, 0.f, 0.f}, dummy[4];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              const int i = row_idx(s);
              const float qh = KDA ? s_qh[tt][i] : s_q[tt][i];
#pragma unroll
              for (int e = 0; e < 4; ++e) ps[e] = fmaf(qh, S[s][e], ps[e]);
            }
            kfirst_reduce(ps, dummy, false);
            if (writer) store_out4(out_row + 4 * lr, ps);
          }
        }
      } else {
        // V_FIRST: rows are value columns j, 4 key elements per thread
        const float4 kr4 = *reinterpret_cast<const float4*>(&s_k[tt][4 * lr]);
        const float4 qr4 = *reinterpret_cast<const float4*>(&s_q[tt][4 * lr]);
        float r[NS], pp[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          r[s] = fmaf(kr4.w, S[s][3], fmaf(kr4.z, S[s][2], fmaf(kr4.y, S[s][1], kr4.x * S[s][0])));
          pp[s] = fmaf(qr4.w, S[s][3], fmaf(qr4.z, S[s][2], fmaf(qr4.y, S[s][1], qr4.x * S[s][0])));
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          r[s] = lane_sum<0, LB>(r[s]);
          pp[s] = lane_sum<0, LB>(pp[s]);
        }
        float u[NS];
        float my_o = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          u[s] = beta * (s_v[tt][row_idx(s)] - alpha * r[s]);
          const float os = fmaf(qk, u[s], alpha * pp[s]);
          if (lr == s) my_o = os;
        }
        if (!stored && lr < NS) store_out1(out_row + row_idx(lr), my_o);
        float al4[4], kh4[4];
        if constexpr (KDA) {
          const float4 a = *reinterpret_cast<const float4*>(&s_al[tt][4 * lr]);
          const float4 kk = *reinterpret_cast<const float4*>(&s_kh[tt][4 * lr]);
          al4[0] = a.x; al4[1] = a.y; al4[2] = a.z; al4[3] = a.w;
          kh4[0] = kk.x; kh4[1] = kk.y; kh4[2] = kk.z; kh4[3] = kk.w;
        } else {
          al4[0] = al4[1] = al4[2] = al4[3] = alpha;
          kh4[0] = kr4.x; kh4[1] = kr4.y; kh4[2] = kr4.z; kh4[3] = kr4.w;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[s][e] = fmaf(al4[e], S[s][e], kh4[e] * u[s]);
        if constexpr (QDQ) {
          qdq_tile();
          if (stored) {
            float q4[4];
            if constexpr (KDA) {
              const float4 qq = *reinterpret_cast<const float4*>(&s_qh[tt][4 * lr]);
              q4[0] = qq.x; q4[1] = qq.y; q4[2] = qq.z; q4[3] = qq.w;
            } else {
              q4[0] = qr4.x; q4[1] = qr4.y; q4[2] = qr4.z; q4[3] = qr4.w;
            }
            float mo = 0.0f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              float ps = fmaf(q4[3], S[s][3], fmaf(q4[2], S[s][2], fmaf(q4[1], S[s][1], q4[0] * S[s][0])));
              ps = lane_sum<0, LB>(ps);
              if (lr == s) mo = ps;
            }
            if (lr < NS) store_out1(out_row + row_idx(lr), mo);
          }
        }
      }
    }
  }

#pragma unroll
  for (int s = 0; s < NS; ++s)
    *reinterpret_cast<float4*>(dst + row_off(s)) = make_float4(S[s][0], S[s][1], S[s][2], S[s][3]);
}

}  // namespace gdn

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
// which is the same arithmetic regrouped (alpha is a scalar for GDN and a
// per-key-row vector for KDA).
//
// Layout of the state tile in registers.  Each thread owns NS memory rows of
// 4 consecutive floats (one 128-bit load per row), consecutive lanes cover
// a contiguous row so every wave load is fully coalesced:
//   K_FIRST (V contiguous): memory row = key index i, 4 value columns per
//       thread; the K-reduction is in-thread over NS rows, then across the
//       row groups of a wave (lane xor), then across waves through LDS.
//   V_FIRST (K contiguous): memory row = value index j, 4 key elements per
//       thread; the K-reduction is 4-wide in-thread, then across the K/4
//       lanes of the row (lane xor); no cross-wave step.
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
  int32_t io_bf16;
  int32_t out_bf16;
  int32_t beta_prob;
  int32_t idx64;
  int32_t quantize_initial;
  int32_t readout_stored;
};

constexpr float kL2Eps = 1e-6f;
constexpr float kE4M3Max = 448.0f;
constexpr int kTokensPerChunk = 8;

__device__ __forceinline__ float load_io(const void* p, int64_t i, int bf16) {
  if (bf16) {
    const uint32_t u = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(u << 16);
  }
  return static_cast<const float*>(p)[i];
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

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
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

template <int K, int VB, int NT, bool VF, bool KDA, bool QDQ, bool PAGED>
struct Tile {
  static constexpr int NW = NT / 64;
  static constexpr int LR = VF ? K / 4 : VB / 4;   // lanes covering one memory row
  static constexpr int RPW = 64 / LR;              // memory rows per wave per load step
  static constexpr int ROWS = VF ? VB : K;         // memory rows of the tile
  static constexpr int NS = ROWS / (NW * RPW);     // rows per thread
  static constexpr int TC = kTokensPerChunk;
  static_assert(NT % 64 == 0, "whole waves");
  static_assert(LR >= 1 && LR <= 64 && 64 % LR == 0, "row must fit a wave");
  static_assert(ROWS % (NW * RPW) == 0 && NS >= 1, "tile must split evenly");
  static_assert(!VF || NS <= LR, "V_FIRST output store uses one lane per row");
  static_assert(K % 4 == 0 && VB % 4 == 0, "128-bit rows");
};

// Block-wide max of a per-thread value (all threads get the result).
template <int NW>
__device__ __forceinline__ float block_max(float m, float* s_buf, int w, int lane) {
  m = wave_max(m);
  if constexpr (NW > 1) {
    if (lane == 0) s_buf[w] = m;
    __syncthreads();
    m = s_buf[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, s_buf[i]);
  }
  return m;
}

template <int K, int VB, int NT, bool VF, bool KDA, bool QDQ, bool PAGED>
__global__ __launch_bounds__(NT) void decode_kernel(const Params p) {
  using Cfg = Tile<K, VB, NT, VF, KDA, QDQ, PAGED>;
  constexpr int NW = Cfg::NW, LR = Cfg::LR, RPW = Cfg::RPW, NS = Cfg::NS, TC = Cfg::TC;
  constexpr int KX = KDA ? K : 1;                  // extent of KDA-only arrays
  constexpr int TX = KDA ? TC : 1;
  constexpr int TQ = (KDA && QDQ) ? TC : 1;
  constexpr int KQ = (KDA && QDQ) ? K : 1;

  __shared__ __align__(16) float s_q[TC][K];       // reduction coefficient of p (q_hat, KDA: *alpha)
  __shared__ __align__(16) float s_k[TC][K];       // reduction coefficient of r (k_hat, KDA: *alpha)
  __shared__ __align__(16) float s_kh[TX][KX];     // KDA: k_hat for the write
  __shared__ __align__(16) float s_al[TX][KX];     // KDA: alpha per key channel
  __shared__ __align__(16) float s_qh[TQ][KQ];     // KDA + stored readout: plain q_hat
  __shared__ __align__(16) float s_v[TC][VB];      // this V-block of v
  __shared__ float s_sc[TC][4];                    // alpha (GDN), beta, q_hat . k_hat
  __shared__ __align__(16) float s_red[VF ? 1 : 2][VF ? 1 : NW][2][VB];
  __shared__ float s_max[NW];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane % LR;        // position inside a memory row (x4 floats)
  const int rg = lane / LR;        // row group inside the wave

  const int unit = blockIdx.x;
  const int vb = unit % p.nvb;
  const int h = (unit / p.nvb) % p.HV;
  const int bs = unit / (p.nvb * p.HV);

  // ---- which tokens, which pool rows
  int t0, t1;
  int64_t rrow, wrow;
  if constexpr (PAGED) {
    t0 = bs;
    t1 = bs + 1;
    const int64_t end = load_index(p.page_indptr, bs + 1, p.idx64);
    const int64_t last = load_index(p.page_indices, end - 1, p.idx64);
    const int64_t lpl = load_index(p.last_page_len, bs, p.idx64);
    wrow = last;
    rrow = (lpl == 1) ? load_index(p.page_indices, end - 2, p.idx64) : last;
  } else {
    if (p.cu_seqlens) {
      t0 = p.cu_seqlens[bs];
      t1 = p.cu_seqlens[bs + 1];
    } else {
      t0 = bs;
      t1 = bs + 1;
    }
    rrow = wrow = p.state_indices[bs];
  }
  if (t1 <= t0) return;            // empty suffix: no read, no write

  const int64_t tile_elems = static_cast<int64_t>(K) * p.V;
  const float* src = p.pool + (rrow * p.HV + h) * tile_elems;
  float* dst = p.pool + (wrow * p.HV + h) * tile_elems;

  // memory offset of this thread's row s (start of its 4 floats)
  auto row_off = [&](int s) -> int64_t {
    const int row = s * (NW * RPW) + w * RPW + rg;
    if constexpr (VF) return static_cast<int64_t>(vb * VB + row) * K + 4 * lr;
    else return static_cast<int64_t>(row) * p.V + vb * VB + 4 * lr;
  };
  // key index (K_FIRST: per row s) and value column inside the V-block (V_FIRST: per row s)
  auto row_idx = [&](int s) -> int { return s * (NW * RPW) + w * RPW + rg; };

  float S[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(src + row_off(s));
    S[s][0] = x.x;
    S[s][1] = x.y;
    S[s][2] = x.z;
    S[s][3] = x.w;
  }

  const int hk = h / p.gqa;
  const int64_t out_col0 = static_cast<int64_t>(vb) * VB;
  int red_buf = 0;

  auto qdq_tile = [&]() {
    float m = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(S[s][e]));
    __syncthreads();               // s_max reuse
    m = block_max<NW>(m, s_max, w, lane);
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

  if constexpr (QDQ) {
    if (p.quantize_initial) qdq_tile();
  }

  for (int c0 = t0; c0 < t1; c0 += TC) {
    const int n = min(TC, t1 - c0);
    if (c0 != t0) __syncthreads();   // readers of the previous chunk are done

    // ---- per-token activations into LDS, one wave per token
    for (int tt = w; tt < n; tt += NW) {
      const int t = c0 + tt;
      constexpr int EPL = (K + 63) / 64;
      float qv[EPL], kv[EPL];
      float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int i = lane + 64 * e;
        qv[e] = 0.0f;
        kv[e] = 0.0f;
        if (i < K) {
          const int64_t off = (static_cast<int64_t>(t) * p.HK + hk) * K + i;
          qv[e] = load_io(p.q, off, p.io_bf16);
          kv[e] = load_io(p.k, off, p.io_bf16);
        }
        ssq += qv[e] * qv[e];
        ssk += kv[e] * kv[e];
      }
      float iq = p.scale, ik = 1.0f;
      if (p.l2norm) {
        iq = p.scale * rsqrtf(wave_sum(ssq) + kL2Eps);
        ik = rsqrtf(wave_sum(ssk) + kL2Eps);
      }
      float qk = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        qv[e] *= iq;
        kv[e] *= ik;
        qk += qv[e] * kv[e];
      }
      qk = wave_sum(qk);
      const float bin = load_io(p.beta, static_cast<int64_t>(t) * p.HV + h, p.io_bf16);
      const float beta = p.beta_prob ? bin : sigmoid_f(bin);
      if constexpr (KDA) {
        const float rate = expf(p.a_log[h]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int i = lane + 64 * e;
          if (i < K) {
            const float x = load_io(p.gate, (static_cast<int64_t>(t) * p.HV + h) * K + i, p.io_bf16) +
                            p.dt_bias[h * K + i];
            const float al = expf(-rate * softplus_f(x));
            s_q[tt][i] = qv[e] * al;
            s_k[tt][i] = kv[e] * al;
            s_kh[tt][i] = kv[e];
            s_al[tt][i] = al;
            if constexpr (QDQ) s_qh[tt][i] = qv[e];
          }
        }
      } else {
        const float x = load_io(p.gate, static_cast<int64_t>(t) * p.HV + h, p.io_bf16) + p.dt_bias[h];
        const float al = expf(-expf(p.a_log[h]) * softplus_f(x));
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int i = lane + 64 * e;
          if (i < K) {
            s_q[tt][i] = qv[e];
            s_k[tt][i] = kv[e];
          }
        }
        if (lane == 0) s_sc[tt][0] = al;
      }
      if (lane == 0) {
        s_sc[tt][1] = beta;
        s_sc[tt][2] = qk;
      }
      for (int j = lane; j < VB; j += 64)
        s_v[tt][j] = load_io(p.v, (static_cast<int64_t>(t) * p.HV + h) * p.V + out_col0 + j, p.io_bf16);
    }
    __syncthreads();

    // ---- the recurrence over this chunk's tokens
    for (int tt = 0; tt < n; ++tt) {
      const int t = c0 + tt;
      const float beta = s_sc[tt][1];
      const float qk = s_sc[tt][2];
      const float alpha = KDA ? 1.0f : s_sc[tt][0];   // GDN alpha is applied after the reduction
      const int64_t out_row = (static_cast<int64_t>(t) * p.HV + h) * p.V + out_col0;

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
#pragma unroll
        for (int o = LR; o < 64; o <<= 1)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] += __shfl_xor(r[e], o, 64);
            pp[e] += __shfl_xor(pp[e], o, 64);
          }
        if constexpr (NW > 1) {
          if (rg == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s_red[red_buf][w][0][4 * lr + e] = r[e];
              s_red[red_buf][w][1][4 * lr + e] = pp[e];
            }
          }
          __syncthreads();
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float rs = 0.f, ps = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
              rs += s_red[red_buf][ww][0][4 * lr + e];
              ps += s_red[red_buf][ww][1][4 * lr + e];
            }
            r[e] = rs;
            pp[e] = ps;
          }
          red_buf ^= 1;
        }
        float u[4], o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u[e] = beta * (s_v[tt][4 * lr + e] - alpha * r[e]);
          o[e] = alpha * pp[e] + qk * u[e];
        }
        const bool writer = (w == 0 && rg == 0);
        if (!(QDQ && p.readout_stored) && writer) {
          if (p.out_bf16) {
            uint2 pk;
            pk.x = to_bf16_bits(o[0]) | (static_cast<uint32_t>(to_bf16_bits(o[1])) << 16);
            pk.y = to_bf16_bits(o[2]) | (static_cast<uint32_t>(to_bf16_bits(o[3])) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + out_row + 4 * lr) = pk;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + out_row + 4 * lr) =
                make_float4(o[0], o[1], o[2], o[3]);
          }
        }
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
          if (p.readout_stored) {
            // o = q_hat^T S after rounding
            float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              const int i = row_idx(s);
              const float qh = KDA ? s_qh[tt][i] : s_q[tt][i];
#pragma unroll
              for (int e = 0; e < 4; ++e) ps[e] = fmaf(qh, S[s][e], ps[e]);
            }
#pragma unroll
            for (int o2 = LR; o2 < 64; o2 <<= 1)
#pragma unroll
              for (int e = 0; e < 4; ++e) ps[e] += __shfl_xor(ps[e], o2, 64);
            if constexpr (NW > 1) {
              if (rg == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s_red[red_buf][w][1][4 * lr + e] = ps[e];
              }
              __syncthreads();
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) acc += s_red[red_buf][ww][1][4 * lr + e];
                ps[e] = acc;
              }
              red_buf ^= 1;
            }
            if (writer) {
              if (p.out_bf16) {
                uint2 pk;
                pk.x = to_bf16_bits(ps[0]) | (static_cast<uint32_t>(to_bf16_bits(ps[1])) << 16);
                pk.y = to_bf16_bits(ps[2]) | (static_cast<uint32_t>(to_bf16_bits(ps[3])) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + out_row + 4 * lr) = pk;
              } else {
                *reinterpret_cast<float4*>(static_cast<float*>(p.out) + out_row + 4 * lr) =
                    make_float4(ps[0], ps[1], ps[2], ps[3]);
              }
            }
          }
        }
      } else {
        // V_FIRST: rows are value columns j, 4 key elements per thread
        const float4 kr4 = *reinterpret_cast<const float4*>(&s_k[tt][4 * lr]);
        const float4 qr4 = *reinterpret_cast<const float4*>(&s_q[tt][4 * lr]);
        float r[NS], pp[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          r[s] = kr4.x * S[s][0] + kr4.y * S[s][1] + kr4.z * S[s][2] + kr4.w * S[s][3];
          pp[s] = qr4.x * S[s][0] + qr4.y * S[s][1] + qr4.z * S[s][2] + qr4.w * S[s][3];
        }
#pragma unroll
        for (int o = 1; o < LR; o <<= 1)
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            r[s] += __shfl_xor(r[s], o, 64);
            pp[s] += __shfl_xor(pp[s], o, 64);
          }
        float u[NS];
        float my_o = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          u[s] = beta * (s_v[tt][row_idx(s)] - alpha * r[s]);
          const float os = alpha * pp[s] + qk * u[s];
          if (lr == s) my_o = os;
        }
        if (!(QDQ && p.readout_stored) && lr < NS) {
          const int64_t oi = out_row + row_idx(lr);
          if (p.out_bf16) static_cast<uint16_t*>(p.out)[oi] = to_bf16_bits(my_o);
          else static_cast<float*>(p.out)[oi] = my_o;
        }
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
          if (p.readout_stored) {
            float q4[4];
            if constexpr (KDA) {
              const float4 qq = *reinterpret_cast<const float4*>(&s_qh[tt][4 * lr]);
              q4[0] = qq.x; q4[1] = qq.y; q4[2] = qq.z; q4[3] = qq.w;
            } else {
              q4[0] = qr4.x; q4[1] = qr4.y; q4[2] = qr4.z; q4[3] = qr4.w;
            }
            float ps[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s)
              ps[s] = q4[0] * S[s][0] + q4[1] * S[s][1] + q4[2] * S[s][2] + q4[3] * S[s][3];
#pragma unroll
            for (int o = 1; o < LR; o <<= 1)
#pragma unroll
              for (int s = 0; s < NS; ++s) ps[s] += __shfl_xor(ps[s], o, 64);
            float mo = 0.0f;
#pragma unroll
            for (int s = 0; s < NS; ++s)
              if (lr == s) mo = ps[s];
            if (lr < NS) {
              const int64_t oi = out_row + row_idx(lr);
              if (p.out_bf16) static_cast<uint16_t*>(p.out)[oi] = to_bf16_bits(mo);
              else static_cast<float*>(p.out)[oi] = mo;
            }
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

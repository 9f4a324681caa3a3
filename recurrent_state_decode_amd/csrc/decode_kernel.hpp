// Device side of the gated delta-rule decode: one workgroup per
// (sequence, value head, V-block) work unit.
//
// Math per token (Circuit.LLM.Mixer, "Delta rule" and "Gated memory";
// max.nn.state_space.kda_decode, description): decay the state, read what
// the key retrieves, write the delta, read the updated state out.
//
// Scaled state.  Registers hold S_reg with the true state S = c * S_reg,
// where c is one scalar per workgroup.  GDN's decay is one factor per head,
// so it goes into c and a token needs one pass over the tile and one FMA per
// element for the write:
//     c' = c * alpha                                 (the decay)
//     r  = k_hat^T S = c' (k_hat^T S_reg),  p = c' (q_hat^T S_reg)
//     u  = beta (v - r),   o = p + (q_hat . k_hat) u  (= q_hat^T S_new)
//     S_reg += k_hat (u / c')                         (S_new = c' S_reg)
// KDA's decay is one factor per key channel: it multiplies the registers'
// key rows directly (c' = c), one multiply per element.  A scale below 1e-20
// is applied to the registers and reset to 1, so S_reg never overflows.  The
// fp8 tile quantisation keeps the codes in S_reg and moves the tile scale
// amax/448 into c.  With the int8_hadamard32 codec the registers carry the
// state rotated along V (each 32-value group times the Hadamard matrix) from
// load to store, and each token rounds the rotated groups; the codes do not
// depend on c, so c is left alone.  The tile is multiplied out (and rotated
// back) once, when it is stored.
//
// Layout of the state tile in registers.  Each thread owns NS memory rows of
// EV floats (128-bit loads); consecutive lanes cover a contiguous memory row,
// so every wave-wide load or store is fully coalesced:
//   K_FIRST (V contiguous): memory row = key index i, 4 value columns per
//       thread; the K-reduction is in-thread over NS rows, then across the
//       row groups of a wave (v_permlane32_swap / v_permlane16_swap), then
//       across waves through LDS.
//   V_FIRST (K contiguous): memory row = value index j, 8 key elements per
//       thread (two float4 half a row apart; 4 for small K); the K-reduction
//       is in-thread, then across the 16 lanes of the row with DPP (quad
//       permutes, row mirror, row rotate); no cross-wave step.  With the
//       int8_hadamard32 codec a V_FIRST tile is transposed through LDS into
//       the K_FIRST arrangement at load and back at store.
//
// Latency: the per-token inputs of the first chunk are loaded before the
// state tile and normalised while the tile is in flight.
//
// Work order: the hardware hands consecutive workgroup ids to the 8 XCDs in
// turn.  The kernel renumbers them so that runs of xcd_group consecutive work
// units (neighbouring V-blocks and heads of one sequence) execute on the same
// XCD: they share that XCD's L2 for q/k/v and stream one contiguous slice of
// the work instead of eight interleaved ones.  The state tile is read and
// written with non-temporal loads and stores: it is touched once per call.
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
  const int64_t* slots;          // paged, single token: precomputed (read, write) rows, or null
  int32_t page_size;             // paged suffixes of several tokens
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
  int32_t xcd_shift;       // log2 of the number of consecutive work units kept on one XCD
  // n / d as (n * m) >> sh for n < 2^31 (host-computed), for d = nvb, HV, HV / HK
  uint64_t div_nvb_m, div_hv_m, div_gqa_m;
  int32_t div_nvb_s, div_hv_s, div_gqa_s;
};

// Work unit run by workgroup id bx of a grid of n workgroups.  The hardware
// hands consecutive workgroup ids to the 8 XCDs in turn; within each span of
// 8 * 2^gs ids, XCD x (= id % 8) gets the units [x 2^gs, (x + 1) 2^gs) of
// that span, so each run of 2^gs consecutive units executes on one XCD and
// shares its L2.  Ids past the last whole span keep their number.  A
// permutation of [0, n) for every gs >= 0 (host and device share this code;
// gdn_workgroup_order exports it for the host-side test of that property).
__host__ __device__ inline int xcd_unit(int bx, int n, int gs) {
  const int span = gs + 3;
  const int nfull = (n >> span) << span;
  if (bx >= nfull) return bx;
  return ((bx >> span) << span) | ((bx & 7) << gs) | ((bx >> 3) & ((1 << gs) - 1));
}

__device__ __forceinline__ int fast_div(int n, uint64_t m, int sh) {
  return static_cast<int>((static_cast<uint64_t>(static_cast<uint32_t>(n)) * m) >> sh);
}

// How a work unit finds its tokens and pool rows.
enum Addr : int {
  kPooled = 0,      // state_indices[b]; tokens from cu_seqlens (or one per sequence)
  kPaged1 = 1,      // one token per sequence, CSR page table, copy-on-new-page
  kPagedVar = 2,    // cu_seqlens suffixes on a CSR page table: every page a suffix
                    // token fills gets the state after that token
};

// State quantise/dequantise after every token.
enum Qdq : int {
  kQdqNone = 0,
  kQdqTile = 1,     // fp8 e4m3, one amax/448 scale per [K, VB] tile
  kQdqHad = 2,      // int8 codes of the 32-point Hadamard rotation, one scale per (key row, 32 values)
  kQdqHadPacked = 3,  // the same codec with the pool holding the codes and scales (packed tiles)
  kQdqTilePacked = 4, // fp8 tiles with the pool holding the e4m3 bytes and the tile scales
};

constexpr float kL2Eps = 1e-6f;
constexpr float kE4M3Max = 448.0f;
constexpr int kTokensPerChunk = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
  } else if constexpr (sizeof(TIn) == 2 && N == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + i);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
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

// The same entry read through the constant address space: with a uniform
// index it becomes a scalar-cache load, which is counted apart from the
// vector memory operations, so waiting for it never waits for earlier
// stores.  Only for tables the kernel never writes (the page table).
// s_waitcnt vmcnt(0), with expcnt and lgkmcnt at their maxima (gfx9 encoding).
// Issued where only a tile's loads are in flight: the compiler cannot prove
// that they complete on every path to the tile's later uses and would
// otherwise wait there, behind the stores issued since (the counter retires
// loads and stores in order).
constexpr int kWaitVmem0 = 0x0F70;

typedef const __attribute__((address_space(4))) int64_t* ConstI64;
typedef const __attribute__((address_space(4))) int32_t* ConstI32;
typedef const __attribute__((address_space(4))) float* ConstF32;
__device__ __forceinline__ int64_t load_index_uniform(const void* p, int64_t i, int idx64) {
  return idx64 ? ((ConstI64)p)[i] : static_cast<int64_t>(((ConstI32)p)[i]);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  const __bf16 h = static_cast<__bf16>(x);   // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Activations on the hardware transcendental units (v_exp_f32 = 2^x,
// v_log_f32 = log2 x, v_rcp_f32): about one ulp each, far inside the
// decode tolerance, and a few instructions instead of a library sequence.
constexpr float kLog2E = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2E); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// max(x, 0) + log(1 + exp(-|x|))
__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + __builtin_amdgcn_logf(1.0f + exp_hw(-fabsf(x))) * kLn2;
}

__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.0f + exp_hw(-x)); }

// ---- cross-lane primitives (wave64)

// Every control used here (quad_perm, row_mirror, row_half_mirror,
// row_ror) reads a lane of the same row, so no lane is out of bounds and
// bound_ctrl only tells the compiler that no old value needs keeping: the
// move can then fold into the consuming add or max as its DPP operand.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// x with its sign flipped where sm has the sign bit (a lane-dependent +-x
// that, unlike a multiply, cannot be contracted into an fma)
__device__ __forceinline__ float flip_sign(float x, uint32_t sm) { return __uint_as_float(__float_as_uint(x) ^ sm); }

struct OpAdd {
  __device__ static float f(float a, float b) { return a + b; }
};
// Maximum of non-negative floats (amax reductions) as an unsigned compare
// of their bit patterns: same order, no NaN canonicalisation, and the DPP
// operand folds into v_max_u32.
struct OpMaxNonNeg {
  __device__ static float f(float a, float b) {
    return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
  }
};

// x combined with the value of the lane in the other 16-lane row of the same 32-lane half
template <class Op>
__device__ __forceinline__ float with_rows16(float x) {
  const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

// x combined with the value of the lane in the other 32-lane half
template <class Op>
__device__ __forceinline__ float with_halves32(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

// Reduce over the lanes that differ from this one only in lane-index bits
// [LO, HI); every lane receives the result.  DPP controls: quad_perm 0xB1
// swaps lanes 2n and 2n+1, 0x4E swaps pairs 0-1 and 2-3, row_half_mirror
// (0x141) reverses each group of 8, row_ror:8 (0x128) and row_ror:4 (0x124)
// rotate a 16-lane row.  Each step adds a lane set disjoint from the one
// gathered so far, so every lane of the group is counted exactly once.
template <int LO, int HI, class Op = OpAdd>
__device__ __forceinline__ float lane_reduce(float x) {
  static_assert(0 <= LO && LO < HI && HI <= 6, "lane bits");
  constexpr bool b0 = LO <= 0 && 0 < HI, b1 = LO <= 1 && 1 < HI, b2 = LO <= 2 && 2 < HI;
  constexpr bool b3 = LO <= 3 && 3 < HI, b4 = LO <= 4 && 4 < HI, b5 = LO <= 5 && 5 < HI;
  if constexpr (b0) x = Op::f(x, dpp<0xB1>(x));
  if constexpr (b1) x = Op::f(x, dpp<0x4E>(x));
  if constexpr (b2) {
    static_assert((b0 && b1) || b3, "bit 2 needs bits 0-1 (mirror) or bit 3 (rotate)");
    if constexpr (b0 && b1) {
      x = Op::f(x, dpp<0x141>(x));         // lanes i and 7-i: with bits 0,1 covers the 8
      if constexpr (b3) x = Op::f(x, dpp<0x128>(x));
    } else {
      x = Op::f(x, dpp<0x128>(x));         // i and i+8
      x = Op::f(x, dpp<0x124>(x));         // then i-4: {i, i-4, i-8, i-12}
    }
  } else if constexpr (b3) {
    x = Op::f(x, dpp<0x128>(x));
  }
  if constexpr (b4) x = with_rows16<Op>(x);
  if constexpr (b5) x = with_halves32<Op>(x);
  return x;
}

// Reduce-scatter of two values across lane bit 5: lanes 0-31 get a summed
// over the two halves, lanes 32-63 get b summed.
__device__ __forceinline__ float rs_halves32(float a, float b) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Reduce-scatter of two values across lane bit 4: 16-lane rows 0 and 2 get a
// summed with the next row, rows 1 and 3 get b summed.
__device__ __forceinline__ float rs_rows16(float a, float b) {
  const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Round x0 .. x3 (already divided by the tile scale) to the E4M3 grid and
// back with the gfx950 OCP fp8 conversions (nearest even).  The two pairs
// fill the low and the high half of one packed word, so no destination needs
// clearing first (the first conversion's "old" operand is any value whose
// high half the second conversion replaces).  The scaled conversions of
// gfx950 are no help here: they take only the exponent of their scale
// operand (checked on the device), and the tile scale amax / 448 is not a
// power of two.
__device__ __forceinline__ void e4m3_roundtrip4(float& x0, float& x1, float& x2, float& x3) {
  int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __float_as_int(x0), false);
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, pk, true);
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
  x0 = lo[0];
  x1 = lo[1];
  x2 = hi[0];
  x3 = hi[1];
}

// 448 / m and m / 448 for the tile scale, m >= 2^-100: the hardware
// reciprocal (or the rounded constant 1/448) and one residual correction
// q + (n - q d) / d, a few instructions instead of a full division; the
// result is the correctly rounded quotient except within an ulp of a
// rounding boundary, and exact whenever the quotient is representable
// (m = 448 * 2^k: an exact scale keeps the grid exact).
__device__ __forceinline__ float div448_by(float m) {
  const float r = __builtin_amdgcn_rcpf(m);
  const float q = 448.0f * r;
  return fmaf(fmaf(-q, m, 448.0f), r, q);
}
__device__ __forceinline__ float div_by448(float m) {
  constexpr float c = 1.0f / 448.0f;
  const float q = m * c;
  return fmaf(fmaf(-q, 448.0f, m), c, q);
}

// ---- int8_hadamard32 codec (modelopt ... linear_attention.config,
// LinearAttentionDecodeConfig, state_codec; ... linear_attention.decode,
// LinearAttentionCarry, value_basis / reconstruct)
//
// A 32-value group sits in 8 consecutive lanes x 4 registers, value index
// 4 * (lane % 8) + j.  wht32 is the unnormalised Walsh-Hadamard transform
// (Sylvester order) of the group, in place: the two register bits by
// in-thread butterflies, lane bits 0, 1, 2 by a partner lane (quad_perm
// 0xB1 = xor 1, 0x4E = xor 2; xor 4 as row_half_mirror (xor 7) after the
// quad reversal 0x1B (xor 3)).  A butterfly leaves a + b at the lower index
// and a - b at the upper one; flipping the own value's sign on lanes at the
// upper index (sign masks sm1, sm2, sm4) gives both as partner + (+-own).
// NR independent groups (rows) go through each stage together, so that a
// lane move's result is not needed by the very next instruction.
template <int NR>
__device__ __forceinline__ void wht32(float (&x)[NR][4], uint32_t sm1, uint32_t sm2, uint32_t sm4) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float a0 = x[r][0] + x[r][1], a1 = x[r][0] - x[r][1], a2 = x[r][2] + x[r][3], a3 = x[r][2] - x[r][3];
    x[r][0] = a0 + a2;
    x[r][1] = a1 + a3;
    x[r][2] = a0 - a2;
    x[r][3] = a1 - a3;
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) x[r][j] = dpp<0xB1>(x[r][j]) + flip_sign(x[r][j], sm1);
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) x[r][j] = dpp<0x4E>(x[r][j]) + flip_sign(x[r][j], sm2);
  float t[NR][4];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) t[r][j] = dpp<0x1B>(x[r][j]);
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) x[r][j] = dpp<0x141>(t[r][j]) + flip_sign(x[r][j], sm4);
}

// The same transform with one value per lane: the group is lane bits 0-4
// (each 32-lane half is its own group).  Lane bit 3 pairs lanes i and i ^ 8
// as row_mirror (xor 15) after row_half_mirror (xor 7); lane bit 4 uses
// v_permlane16_swap, which hands every lane the values of the lower and the
// upper 16-lane row of its pair.
__device__ __forceinline__ float wht32_lanes(float x, int lane) {
  const uint32_t ul = static_cast<uint32_t>(lane);
  x = dpp<0xB1>(x) + flip_sign(x, (ul & 1u) << 31);
  x = dpp<0x4E>(x) + flip_sign(x, (ul & 2u) << 30);
  x = dpp<0x141>(dpp<0x1B>(x)) + flip_sign(x, (ul & 4u) << 29);
  x = dpp<0x140>(dpp<0x141>(x)) + flip_sign(x, (ul & 8u) << 28);
  const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + flip_sign(__uint_as_float(pr[1]), (ul & 16u) << 27);
}

// 127 / m for m > 0: hardware reciprocal (about 1 ulp) and one residual
// correction, q + (127 - q m) / m (exact for m = 127 * 2^k)
__device__ __forceinline__ float div127_by(float m) {
  const float r = __builtin_amdgcn_rcpf(m);
  const float q = 127.0f * r;
  return fmaf(fmaf(-q, m, 127.0f), r, q);
}

constexpr float kTinyScale = 1e-20f;
constexpr float kTinyAmax = 0x1p-100f;

template <int K, int VB, int NT, bool VF>
struct Tile {
  static constexpr int NW = NT / 64;
  static constexpr int EV = VF ? (K >= 64 ? 8 : 4) : 4;   // floats per thread per memory row
  static constexpr int LR = VF ? K / EV : VB / 4;         // lanes covering one memory row
  static constexpr int RPW = 64 / LR;                     // memory rows per wave per load step
  static constexpr int ROWS = VF ? VB : K;                // memory rows of the tile
  static constexpr int NS = ROWS / (NW * RPW);            // rows per thread
  static constexpr int LB = __builtin_ctz(LR);            // lane bits inside a memory row
  static constexpr int NKEY = VF ? EV : NS;               // key indices a thread touches
  static constexpr bool KF_RS = !VF && LB == 4 && NW > 1; // K_FIRST reduce-scatter path
  static_assert(NT % 64 == 0, "whole waves");
  static_assert(LR >= 1 && LR <= 64 && 64 % LR == 0, "row must fit a wave");
  static_assert(ROWS % (NW * RPW) == 0 && NS >= 1, "tile must split evenly");
  static_assert(!VF || NS <= LR, "V_FIRST output store uses one lane per row");
  static_assert(K % 4 == 0 && VB % 4 == 0, "128-bit rows");
  static_assert(!VF || EV == 4 || K / 2 == 4 * LR, "two float4 half a row apart");
};

template <int K, int VB, int NT, bool VF, bool KDA, int QDQ, int ADDR, typename TIn>
__global__ __launch_bounds__(NT) void decode_kernel(const Params p) {
  // Register arrangement: V_FIRST rows (value columns) for a V_FIRST pool,
  // except with the int8_hadamard32 codec, which needs each key row's values
  // in lanes; the pool layout VF itself only shapes the tile's load and store.
  // PACKED: each (row, head) tile of the pool is K V int8 codes in
  // [V / 32][K][32] order (the +-1 Hadamard basis of each 32-value group;
  // a group's codes for all key rows contiguous) followed by K V / 32
  // float32 scales in [V / 32][K] order; the codes load straight into the
  // rotated registers.  A workgroup's V-block is then whole groups: every
  // line it reads or writes is its own.
  constexpr bool PACKED = QDQ == kQdqHadPacked;
  constexpr bool HAD = QDQ == kQdqHad || PACKED;
  // FP8P: each (row, head) tile of the pool is its K V e4m3 bytes in the pool
  // layout's order, then its V / VB float32 tile scales (amax / 448; VB is
  // the fp8 tile width), the tile rounded up to whole 128-byte lines.  The registers of the fp8 path
  // hold grid values with the tile scale in cs, so bytes load and store as
  // they are.
  constexpr bool FP8P = QDQ == kQdqTilePacked;
  constexpr bool TILE = QDQ == kQdqTile || FP8P;
  static_assert(!PACKED || !VF, "packed tiles have one layout");
  constexpr bool AV = VF && !HAD;
  using Cfg = Tile<K, VB, NT, AV>;
  constexpr int NW = Cfg::NW, LR = Cfg::LR, RPW = Cfg::RPW, NS = Cfg::NS, LB = Cfg::LB;
  constexpr int EV = Cfg::EV, NKEY = Cfg::NKEY;
  // CONTIG: a packed fp8 V_FIRST tile keeps a row lane's 8 keys contiguous
  // (8 lr .. 8 lr + 7) instead of two 4-key pieces half a row apart, so that
  // each row loads and stores as one 8-byte piece per lane: 16 lanes, one
  // whole 128-byte line (paged GDN B=256: 66.0 -> 62.5 us).  Not for KDA: its
  // three per-token key arrays then come out of LDS at a 32-byte lane stride
  // with bank conflicts (75.7 -> 76.2 us)
  constexpr bool CONTIG = FP8P && AV && !KDA && EV == 8 && K == 8 * LR;
  // Tokens staged per chunk.  A one-token paged call on a packed pool stages
  // exactly one: the compiler cannot see that n <= 1 there and would keep
  // every wave's raw-input registers for a whole chunk live across the tile
  // load (paged B=256: fp8 GDN 156 -> 114 VGPRs, 3 -> 4 waves per SIMD,
  // 64.9 -> 59.8 us; fp8 KDA 105 -> 74 VGPRs, 76.4 -> 67.6 us; the
  // int8_hadamard32 codec 114 -> 82 VGPRs, 88.2 -> 75.5 us).  On fp32 pools
  // the one-token shapes measured 1-3 % slower that way, with or without
  // QDQ, and keep the chunk.
  constexpr int TC = (ADDR == kPaged1 && (FP8P || PACKED)) ? 1 : kTokensPerChunk;
  constexpr int TPW = (TC + NW - 1) / NW;          // tokens per wave in a chunk
  constexpr int EPL = (K + 63) / 64;               // q/k/gate elements per lane (contiguous)
  constexpr int EL = K / EPL;                      // lanes holding q/k elements
  constexpr int VPL = (VB + 63) / 64;              // v elements per lane
  constexpr int VL = VB / VPL;                     // lanes holding v elements
  constexpr int GPL = KDA ? EPL : 1;
  constexpr int KX = KDA ? K : 4;                  // extent of the KDA-only array
  constexpr int TX = KDA ? TC : 1;
  static_assert(K % EPL == 0 && VB % VPL == 0, "input split");

  // Per-token values in LDS.  Key-indexed arrays are stored at lds_pos(key):
  // V_FIRST keeps key order; K_FIRST stores each thread's NS keys together.
  __shared__ __align__(16) float s_q[TC][K];       // q_hat
  __shared__ __align__(16) float s_k[TC][K];       // k_hat
  __shared__ __align__(16) float s_al[TX][KX];     // KDA: alpha per key channel
  __shared__ __align__(16) float s_v[TC][VB];      // this V-block of v
  __shared__ float s_sc[TC][4];                    // alpha (GDN), beta, q_hat . k_hat
  __shared__ __align__(16) float s_red[AV ? 1 : 2][AV ? 1 : NW][2][VB];
  __shared__ float s_max[2][NW];
  // V_FIRST rows with several tokens: a chunk's outputs are collected here
  // and written once per chunk, 8 values per lane, instead of one value per
  // row lane and token (kPaged1 calls have one token)
  constexpr bool OUT_LDS = AV && ADDR != kPaged1;
  static_assert(!OUT_LDS || VB % 8 == 0, "8-value output pieces");
  __shared__ __align__(16) float s_o[OUT_LDS ? TC : 1][OUT_LDS ? VB : 8];
  __shared__ __align__(16) float s_wv[Cfg::KF_RS ? VB : 4];   // K_FIRST, 64 columns: u / c' per column
  // V_FIRST pool with the codec: the tile passes through LDS between the
  // pool's [V][K] rows and the [K][V] register arrangement (row stride K + 1
  // keeps both directions free of bank conflicts)
  constexpr bool TRANS = VF && HAD;
  constexpr int LD = K + 1;
  __shared__ float s_t[TRANS ? VB * LD : 1];
  // the codec works on 8-lane groups of 32 values; the V_FIRST transpose
  // through LDS is written for the 64-column, 4-wave shape
  static_assert(!HAD || (K == 128 && EV == 4 && VPL == 1 && VB % 32 == 0 &&
                         (!TRANS || (VB == 64 && NT == 256 && LR == 16 && NS == K / 16))),
                "int8_hadamard32 codec shape");

  const TIn* __restrict__ gq = static_cast<const TIn*>(p.q);
  const TIn* __restrict__ gk = static_cast<const TIn*>(p.k);
  const TIn* __restrict__ gv = static_cast<const TIn*>(p.v);
  const TIn* __restrict__ gg = static_cast<const TIn*>(p.gate);
  const TIn* __restrict__ gb = static_cast<const TIn*>(p.beta);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane % LR;        // position inside a memory row
  const int rg = lane / LR;        // row group inside the wave

  // runs of 2^xcd_shift consecutive work units on one XCD (xcd_unit)
  const int unit = xcd_unit(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), p.xcd_shift);
  const int q1 = fast_div(unit, p.div_nvb_m, p.div_nvb_s);
  const int vb = unit - q1 * p.nvb;
  const int bs = fast_div(q1, p.div_hv_m, p.div_hv_s);
  const int h = q1 - bs * p.HV;
  const int hk = fast_div(h, p.div_gqa_m, p.div_gqa_s);
  const int64_t out_col0 = static_cast<int64_t>(vb) * VB;

  // key index of this thread's key slot m, and the LDS position of key c
  auto key_of = [&](int m) -> int {
    if constexpr (CONTIG) return 8 * lr + m;
    else if constexpr (AV) return (EV == 8 ? (m / 4) * (K / 2) : 0) + 4 * lr + (m % 4);
    else return m * (NW * RPW) + w * RPW + rg;
  };
  auto lds_pos = [](int c) -> int {
    if constexpr (AV) return c;
    else return (c % (NW * RPW)) * NS + c / (NW * RPW);
  };
  // first LDS position of this thread's key slots (they are contiguous in
  // both layouts, per half row for V_FIRST unless CONTIG)
  const int kbase = CONTIG ? 8 * lr : AV ? 4 * lr : (w * RPW + rg) * NS;

  // ---- which tokens
  int t0, t1;
  if constexpr (ADDR == kPaged1) {
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

  // the head's gate parameters, loaded before the tile: vector loads retire in
  // order, so a value loaded after the tile could only be waited for together
  // with the whole tile (and the input normalisation could not overlap it);
  // the head-uniform ones come through the scalar cache
  const float rate_h = exp_hw(((ConstF32)p.a_log)[h]);
  float dtb[GPL];
  if constexpr (KDA) {
    if (lane < EL) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) dtb[e] = p.dt_bias[h * K + EPL * lane + e];
    }
  } else {
    dtb[0] = ((ConstF32)p.dt_bias)[h];
  }

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
          iq = p.scale * rsqrtf(lane_reduce<0, 6>(ssq) + kL2Eps);
          ik = rsqrtf(lane_reduce<0, 6>(ssk) + kL2Eps);
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
        qk = lane_reduce<0, 6>(qk);
        const float beta = p.beta_prob ? xb[0] : sigmoid_f(xb[0]);
        if (lane < EL) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const int c = EPL * lane + e;
            const int pos = lds_pos(c);
            s_q[tt][pos] = xq[e];
            s_k[tt][pos] = xk[e];
            if constexpr (KDA) s_al[tt][pos] = exp_hw(-rate_h * softplus_f(xg[e] + dtb[e]));
          }
        }
        if constexpr (HAD) xv[0] = wht32_lanes(xv[0], lane);   // v in the rotated basis (VPL == 1)
        if (lane < VL) {
#pragma unroll
          for (int e = 0; e < VPL; ++e) s_v[tt][VPL * lane + e] = xv[e];
        }
        if (lane == 0) {
          if constexpr (!KDA) s_sc[tt][0] = exp_hw(-rate_h * softplus_f(xg[0] + dtb[0]));
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
  int64_t pg_start = 0, pos0 = 0, pos_last = 0;   // kPagedVar: first table entry, token positions
  if constexpr (ADDR == kPaged1) {
    if (p.slots) {
      rrow = p.slots[2 * bs];
      wrow = p.slots[2 * bs + 1];
    } else {
      const int64_t end = load_index(p.page_indptr, bs + 1, p.idx64);
      const int64_t last = load_index(p.page_indices, end - 1, p.idx64);
      const int64_t lpl = load_index(p.last_page_len, bs, p.idx64);
      wrow = last;
      rrow = (lpl == 1) ? load_index(p.page_indices, end - 2, p.idx64) : last;
    }
  } else if constexpr (ADDR == kPagedVar) {
    // the sequence holds n tokens after the suffix; the suffix is positions
    // pos0 .. n (1-based); the state before it lives on the page of pos0 - 1
    pg_start = load_index(p.page_indptr, bs, p.idx64);
    const int64_t end = load_index(p.page_indptr, bs + 1, p.idx64);
    const int64_t lpl = load_index(p.last_page_len, bs, p.idx64);
    pos_last = (end - pg_start - 1) * p.page_size + lpl;
    pos0 = pos_last - (t1 - t0) + 1;
    // (clamped so that a table that breaks the one-prior-token precondition
    // still addresses its own pages)
    rrow = load_index(p.page_indices, pg_start + max(pos0 - 2, static_cast<int64_t>(0)) / p.page_size, p.idx64);
    wrow = load_index(p.page_indices, end - 1, p.idx64);
  } else {
    rrow = wrow = p.state_indices[bs];
  }

  const int64_t tile_elems = static_cast<int64_t>(K) * p.V;
  const int64_t tile_bytes = PACKED ? static_cast<int64_t>(K) * p.V + 4 * static_cast<int64_t>(K) * (p.V / 32)
                                     : 128 * ((static_cast<int64_t>(K) * p.V + 4 * p.nvb + 127) / 128);
  auto tile_base = [&](int64_t row) -> float* {
    if constexpr (PACKED || FP8P)
      return reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(p.pool) + (row * p.HV + h) * tile_bytes);
    else return p.pool + (row * p.HV + h) * tile_elems;
  };
  const float* src = tile_base(rrow);
  float* dst = tile_base(wrow);

  auto row_idx = [&](int s) -> int { return s * (NW * RPW) + w * RPW + rg; };
  // memory offset of this thread's float4 number f (0 .. EV/4-1) in row s
  // (pool layout == register arrangement)
  auto row_off = [&](int s, int f) -> int64_t {
    if constexpr (AV) return static_cast<int64_t>(vb * VB + row_idx(s)) * K + f * (K / 2) + 4 * lr;
    else return static_cast<int64_t>(row_idx(s)) * p.V + vb * VB + 4 * lr;
  };
  // TRANS: the [V][K] rows of the pool are read and written with the
  // V_FIRST geometry (value rows s * 16 + w * 4 + rg, key float4s at
  // f * K / 2 + 4 * lr) and staged in s_t as [value][key]
  auto trans_off = [&](int s, int f) -> int64_t {
    return static_cast<int64_t>(vb * VB + s * 16 + w * 4 + rg) * K + f * (K / 2) + 4 * lr;
  };
  auto trans_lds = [&](int s, int f) -> int { return (s * 16 + w * 4 + rg) * LD + f * (K / 2) + 4 * lr; };
  auto kf_lds = [&](int s, int j) -> int { return (4 * lr + j) * LD + row_idx(s); };

  float S[NS][EV];
  float fp8_scale = 1.0f;          // FP8P: the stored tile scale
  if constexpr (FP8P) {
    // 4 e4m3 bytes for every 4 floats of the fp32 layout (same element order)
    const unsigned char* sb = reinterpret_cast<const unsigned char*>(src);
    auto unpack4 = [&](uint32_t c4, float* x) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c4), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c4), true);
      x[0] = lo[0];
      x[1] = lo[1];
      x[2] = hi[0];
      x[3] = hi[1];
    };
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (CONTIG) {
        const u32x2 c8 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
            sb + static_cast<int64_t>(vb * VB + row_idx(s)) * K + 8 * lr));
        unpack4(c8.x, &S[s][0]);
        unpack4(c8.y, &S[s][4]);
      } else {
#pragma unroll
        for (int f = 0; f < EV / 4; ++f)
          unpack4(__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sb + row_off(s, f))), &S[s][4 * f]);
      }
    }
    const float sc = __builtin_nontemporal_load(reinterpret_cast<const float*>(sb + tile_elems) + vb);
    fp8_scale = sc > 0.0f ? sc : 1.0f;   // an all-zero tile stores scale 0
    finish_raw(n0);                // overlaps the tile load
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);   // the tile (see kWaitVmem0)
  } else if constexpr (PACKED) {
    // 4 codes (one dword) and their group's scale per row: R = code * scale
    const unsigned char* sb = reinterpret_cast<const unsigned char*>(src);
    const float* sc = reinterpret_cast<const float*>(sb + tile_elems);
    const int col = vb * VB + 4 * lr, grp = col / 32;
    const unsigned char* gb = sb + grp * (K * 32) + col % 32;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int r = row_idx(s);
      const uint32_t c4 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(gb + r * 32));
      const float scale = __builtin_nontemporal_load(sc + grp * K + r);
#pragma unroll
      for (int j = 0; j < 4; ++j) S[s][j] = static_cast<float>(static_cast<int8_t>(c4 >> (8 * j))) * scale;
    }
    finish_raw(n0);                // overlaps the tile load
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);   // the tile (see kWaitVmem0)
  } else if constexpr (!TRANS) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int f = 0; f < EV / 4; ++f) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + row_off(s, f)));
        S[s][4 * f + 0] = x.x;
        S[s][4 * f + 1] = x.y;
        S[s][4 * f + 2] = x.z;
        S[s][4 * f + 3] = x.w;
      }
    finish_raw(n0);                // overlaps the tile load
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);   // the tile (see kWaitVmem0)
  } else {
    f32x4 L[VB / 16][2];
#pragma unroll
    for (int s = 0; s < VB / 16; ++s)
#pragma unroll
      for (int f = 0; f < 2; ++f) L[s][f] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + trans_off(s, f)));
    finish_raw(n0);                // overlaps the tile load
#pragma unroll
    for (int s = 0; s < VB / 16; ++s)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int a = trans_lds(s, f);
        s_t[a + 0] = L[s][f].x;
        s_t[a + 1] = L[s][f].y;
        s_t[a + 2] = L[s][f].z;
        s_t[a + 3] = L[s][f].w;
      }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[s][j] = s_t[kf_lds(s, j)];
  }

  // int8_hadamard32: the registers carry R = S H (H the +-1 Hadamard matrix
  // of each 32-value group, H H = 32 I) for the whole suffix.  The rotation
  // acts on the value axis, so it commutes with the decay, the scale and
  // every K-reduction: with v staged as v H, the token's r, p, u and o all
  // come out rotated (u H = beta (v H - k^T R)), the write is R += k (u H),
  // and only o is rotated back (o = (o H) H / 32) for the output.  The codec
  // then rounds R directly.
  const uint32_t sg1 = (static_cast<uint32_t>(lane) & 1u) << 31;   // sign masks of the butterflies
  const uint32_t sg2 = (static_cast<uint32_t>(lane) & 2u) << 30;
  const uint32_t sg4 = (static_cast<uint32_t>(lane) & 4u) << 29;
  if constexpr (HAD && !PACKED) wht32(S, sg1, sg2, sg4);

  // true state = cs * S: one scale per workgroup.  The GDN decay (one factor
  // per head) goes into it; the KDA decay (one factor per key channel) is
  // applied to the registers, one multiply per element, which is no more work
  // than folding per-row factors into the coefficients and keeps no per-row
  // scales live.  fp8 tile QDQ puts the tile scale in cs.
  float cs = fp8_scale;
  // key slot of element (s, e)
  auto slot = [](int s, int e) -> int { return AV ? e : s; };

  int red_buf = 0, max_buf = 0;

  auto block_max = [&](float m) -> float {
    m = lane_reduce<0, 6, OpMaxNonNeg>(m);
    if constexpr (NW > 1) {
      if (lane == 0) s_max[max_buf][w] = m;
      __syncthreads();
      m = s_max[max_buf][0];
#pragma unroll
      for (int i = 1; i < NW; ++i) m = fmaxf(m, s_max[max_buf][i]);
      max_buf ^= 1;
    }
    return m;
  };

  // fp8 tile QDQ of the true state cs * S: the codes stay in S, the tile
  // scale goes to cs (one scale per workgroup for GDN and KDA alike)
  bool tile_nz = true;             // the last qdq_tile saw a non-zero tile
  auto qdq_tile = [&]() {
    // in-thread amax: v_max3_f32 with |x| source modifiers
    float m = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < EV; e += 2)
        m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(fabsf(S[s][e]), fabsf(S[s][e + 1])));
    const float ms = block_max(m);       // amax of S_reg; the true amax is cs * ms
    tile_nz = ms > 0.0f;
    if (ms > 0.0f) {
      const float msf = fmaxf(ms, kTinyAmax);   // 448 / amax stays finite
      const float inv = div448_by(msf);
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < EV; e += 4) {
          float x0 = S[s][e] * inv, x1 = S[s][e + 1] * inv, x2 = S[s][e + 2] * inv, x3 = S[s][e + 3] * inv;
          e4m3_roundtrip4(x0, x1, x2, x3);
          S[s][e] = x0;
          S[s][e + 1] = x1;
          S[s][e + 2] = x2;
          S[s][e + 3] = x3;
        }
      cs = cs * div_by448(msf);
    }
  };

  // int8_hadamard32 codec of every (key row, 32 values) group, on R: the
  // codes rint(127 R / amax|R|) equal rint(127 y / amax|y|) for the
  // orthonormal rotation y = c R / sqrt(32), and the dequantised group is
  // codes * amax|R| / 127 (still rotated; c untouched)
  auto had_quant = [&]() {
    // amax of each row's group (8 lanes), one reduction step for all rows at
    // a time so that the steps of different rows interleave
    // (in-thread: v_maximum3_f32 with |x| source modifiers, two per row)
    float m[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
      m[s] = __builtin_elementwise_maximum(
          __builtin_elementwise_maximum(fabsf(S[s][0]), fabsf(S[s][1])),
          __builtin_elementwise_maximum(fabsf(S[s][2]), fabsf(S[s][3])));
#pragma unroll
    for (int s = 0; s < NS; ++s) m[s] = OpMaxNonNeg::f(m[s], dpp<0xB1>(m[s]));
#pragma unroll
    for (int s = 0; s < NS; ++s) m[s] = OpMaxNonNeg::f(m[s], dpp<0x4E>(m[s]));
#pragma unroll
    for (int s = 0; s < NS; ++s) m[s] = OpMaxNonNeg::f(m[s], dpp<0x141>(m[s]));
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // (an amax below 2^-100, zero included, is raised to 2^-100: the codes
      // of such a group only get coarser, and 127 / m stays finite)
      const float mf = OpMaxNonNeg::f(m[s], kTinyAmax);
      const float inv = div127_by(mf);
      const float c = mf * (1.0f / 127.0f);
      // |R inv| <= 127 (1 + 2^-22) rounds to at most 127: no clamp needed
#pragma unroll
      for (int j = 0; j < 4; ++j) S[s][j] = __builtin_rintf(S[s][j] * inv) * c;
    }
  };
  auto quantize = [&]() {
    if constexpr (TILE) qdq_tile();
    else if constexpr (HAD) had_quant();
  };

  // output stores: 4 consecutive values (K_FIRST) or one (V_FIRST)
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

  // load NKEY consecutive LDS floats starting at pos (float4 pieces)
  auto lds_keys = [&](const float* base, float (&x)[NKEY]) {
    if constexpr (AV) {
#pragma unroll
      for (int f = 0; f < EV / 4; ++f) {
        const float4 v = *reinterpret_cast<const float4*>(base + (CONTIG ? 4 * f : f * (K / 2)) + kbase);
        x[4 * f + 0] = v.x; x[4 * f + 1] = v.y; x[4 * f + 2] = v.z; x[4 * f + 3] = v.w;
      }
    } else if constexpr (NS % 4 == 0) {
#pragma unroll
      for (int f = 0; f < NS / 4; ++f) {
        const float4 v = *reinterpret_cast<const float4*>(base + kbase + 4 * f);
        x[4 * f + 0] = v.x; x[4 * f + 1] = v.y; x[4 * f + 2] = v.z; x[4 * f + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < NKEY; ++m) x[m] = base[kbase + m];
    }
  };

  // K_FIRST: per-thread partial sums over its rows -> block sums of r and p for its 4 columns
  auto kfirst_reduce = [&](float (&r)[4], float (&pp)[4]) {
    if constexpr (Cfg::KF_RS) {
      // lanes of a wave with equal lr hold the same columns and differ in lane bits 4, 5
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = rs_halves32(r[e], pp[e]);   // lanes < 32: r_e, else p_e
      const float y0 = rs_rows16(x[0], x[1]);                        // column par
      const float y1 = rs_rows16(x[2], x[3]);                        // column par + 2
      const int kind = lane >> 5;
      const int par = (lane >> 4) & 1;
      s_red[red_buf][w][kind][4 * lr + par] = y0;
      s_red[red_buf][w][kind][4 * lr + par + 2] = y1;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r[e] = lane_reduce<LB, 6>(r[e]);
        pp[e] = lane_reduce<LB, 6>(pp[e]);
      }
      if constexpr (NW > 1) {
        if (rg == 0) {
          *reinterpret_cast<float4*>(&s_red[red_buf][w][0][4 * lr]) = make_float4(r[0], r[1], r[2], r[3]);
          *reinterpret_cast<float4*>(&s_red[red_buf][w][1][4 * lr]) = make_float4(pp[0], pp[1], pp[2], pp[3]);
        }
      }
    }
    if constexpr (NW > 1) {
      __syncthreads();
      float4 ra = *reinterpret_cast<const float4*>(&s_red[red_buf][0][0][4 * lr]);
      float4 pa = *reinterpret_cast<const float4*>(&s_red[red_buf][0][1][4 * lr]);
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        const float4 x = *reinterpret_cast<const float4*>(&s_red[red_buf][ww][0][4 * lr]);
        const float4 y = *reinterpret_cast<const float4*>(&s_red[red_buf][ww][1][4 * lr]);
        ra.x += x.x; ra.y += x.y; ra.z += x.z; ra.w += x.w;
        pa.x += y.x; pa.y += y.y; pa.z += y.z; pa.w += y.w;
      }
      r[0] = ra.x; r[1] = ra.y; r[2] = ra.z; r[3] = ra.w;
      pp[0] = pa.x; pp[1] = pa.y; pp[2] = pa.z; pp[3] = pa.w;
      red_buf ^= 1;
    }
  };

  // one pass: r = kr^T S and p = qr^T S over K, complete sums for this thread's outputs
  // (K_FIRST: its 4 columns; V_FIRST: its NS rows)
  constexpr int NO = AV ? NS : 4;
  auto reduce_pass = [&](const float (&kr)[NKEY], const float (&qr)[NKEY], float (&r)[NO], float (&pp)[NO]) {
    if constexpr (!AV) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r[e] = kr[0] * S[0][e];
        pp[e] = qr[0] * S[0][e];
      }
#pragma unroll
      for (int s = 1; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] = fmaf(kr[s], S[s][e], r[e]);
          pp[e] = fmaf(qr[s], S[s][e], pp[e]);
        }
      kfirst_reduce(r, pp);
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float a = kr[0] * S[s][0], b = qr[0] * S[s][0];
#pragma unroll
        for (int e = 1; e < EV; ++e) {
          a = fmaf(kr[e], S[s][e], a);
          b = fmaf(qr[e], S[s][e], b);
        }
        r[s] = lane_reduce<0, LB>(a);
        pp[s] = lane_reduce<0, LB>(b);
      }
    }
  };

  const bool staged = OUT_LDS && t1 - t0 > 1;   // uniform per workgroup
  auto store_outputs = [&](int tt, int64_t out_row, const float (&o)[NO]) {
    if constexpr (!AV) {
      if (w == 0 && rg == 0) store_out4(out_row + 4 * lr, o);
    } else {
      // a select per row; the empty asm keeps the compiler from turning the
      // chain into an indexed load from a stack copy of o (scratch memory)
      float my_o = o[0];
#pragma unroll
      for (int s = 1; s < NS; ++s) {
        my_o = (lr == s) ? o[s] : my_o;
        asm volatile("" : "+v"(my_o));
      }
      if (lr < NS) {
        if (OUT_LDS && staged) s_o[tt][row_idx(lr)] = my_o;
        else store_out1(out_row + row_idx(lr), my_o);
      }
    }
  };
  // the staged outputs of tokens c0 .. c0 + n - 1 (after a barrier)
  auto flush_outputs = [&](int c0, int n) {
    constexpr int PL = OUT_LDS ? VB / 8 : 1;   // lanes per token
    for (int idx = tid; idx < n * PL; idx += NT) {
      const int tt = idx / PL, piece = idx - tt * PL;
      const int64_t oi = (static_cast<int64_t>(c0 + tt) * p.HV + h) * p.V + out_col0 + 8 * piece;
      const float4 a = *reinterpret_cast<const float4*>(&s_o[tt][8 * piece]);
      const float4 b = *reinterpret_cast<const float4*>(&s_o[tt][8 * piece + 4]);
      if (p.out_bf16) {
        uint4 pk;
        pk.x = to_bf16_bits(a.x) | (static_cast<uint32_t>(to_bf16_bits(a.y)) << 16);
        pk.y = to_bf16_bits(a.z) | (static_cast<uint32_t>(to_bf16_bits(a.w)) << 16);
        pk.z = to_bf16_bits(b.x) | (static_cast<uint32_t>(to_bf16_bits(b.y)) << 16);
        pk.w = to_bf16_bits(b.z) | (static_cast<uint32_t>(to_bf16_bits(b.w)) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + oi) = pk;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + oi) = a;
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + oi + 4) = b;
      }
    }
  };

  // write the true state (scale * registers) to a pool row, with
  // non-temporal stores like the loads: the row is not read again by this call
  auto store_tile = [&](float* row_base) {
    if constexpr (PACKED) {
      // The registers hold the last token's state, either rounded already
      // (code * c per (row, group): the group's amax is 127 c up to one
      // rounding, so rint(R * 127 / amax) gives the codes back exactly) or
      // not (then this is that token's rounding).  The stored scale carries
      // the workgroup's decay scale: true R = scale * code.
      unsigned char* tb = reinterpret_cast<unsigned char*>(row_base);
      float* tsc = reinterpret_cast<float*>(tb + tile_elems);
      const int col = vb * VB + 4 * lr, grp = col / 32;
      unsigned char* gb = tb + grp * (K * 32) + col % 32;
      float m[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        m[s] = __builtin_elementwise_maximum(
            __builtin_elementwise_maximum(fabsf(S[s][0]), fabsf(S[s][1])),
            __builtin_elementwise_maximum(fabsf(S[s][2]), fabsf(S[s][3])));
#pragma unroll
      for (int s = 0; s < NS; ++s) m[s] = OpMaxNonNeg::f(m[s], dpp<0xB1>(m[s]));
#pragma unroll
      for (int s = 0; s < NS; ++s) m[s] = OpMaxNonNeg::f(m[s], dpp<0x4E>(m[s]));
#pragma unroll
      for (int s = 0; s < NS; ++s) m[s] = OpMaxNonNeg::f(m[s], dpp<0x141>(m[s]));
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int r = row_idx(s);
        const float mf = OpMaxNonNeg::f(m[s], kTinyAmax);
        const float inv = div127_by(mf);
        uint32_t c4 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          c4 |= (static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(S[s][j] * inv))) & 0xffu) << (8 * j);
        __builtin_nontemporal_store(c4, reinterpret_cast<uint32_t*>(gb + r * 32));
        // a plain store: the group's scales are 4-byte pieces from many lanes and waves, which L2 merges into
        // whole lines before writing them back (streamed past L2 each would cost a line)
        if ((lr & 7) == 0) tsc[grp * K + r] = cs * (mf * (1.0f / 127.0f));
      }
    } else if constexpr (FP8P) {
      // every token ends with qdq_tile: grid values, converted exactly; the
      // tile scale is cs (one value: GDN's single scale, KDA's are equal),
      // 0 for an all-zero tile
      unsigned char* tb = reinterpret_cast<unsigned char*>(row_base);
      auto pack4 = [&](const float* x) -> uint32_t {
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __float_as_int(x[0]), false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pk, true);
        return static_cast<uint32_t>(pk);
      };
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if constexpr (CONTIG) {
          const u32x2 c8{pack4(&S[s][0]), pack4(&S[s][4])};
          __builtin_nontemporal_store(
              c8, reinterpret_cast<u32x2*>(tb + static_cast<int64_t>(vb * VB + row_idx(s)) * K + 8 * lr));
        } else {
#pragma unroll
          for (int f = 0; f < EV / 4; ++f)
            __builtin_nontemporal_store(pack4(&S[s][4 * f]), reinterpret_cast<uint32_t*>(tb + row_off(s, f)));
        }
      }
      if (tid == 0)
        __builtin_nontemporal_store(tile_nz ? cs : 0.0f, reinterpret_cast<float*>(tb + tile_elems) + vb);
    } else if constexpr (!HAD) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int f = 0; f < EV / 4; ++f) {
          f32x4 x;
          x.x = S[s][4 * f + 0] * cs;
          x.y = S[s][4 * f + 1] * cs;
          x.z = S[s][4 * f + 2] * cs;
          x.w = S[s][4 * f + 3] * cs;
          __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(row_base + row_off(s, f)));
        }
    } else {
      // back to the original value basis: S = c R H / 32
      float X[NS][4];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) X[s][j] = S[s][j];
      wht32(X, sg1, sg2, sg4);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float sc = cs * 0.03125f;
#pragma unroll
        for (int j = 0; j < 4; ++j) X[s][j] *= sc;
      }
      if constexpr (!TRANS) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
          __builtin_nontemporal_store(f32x4{X[s][0], X[s][1], X[s][2], X[s][3]},
                                      reinterpret_cast<f32x4*>(row_base + row_off(s, 0)));
      } else {
        __syncthreads();           // earlier readers of s_t are done
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int j = 0; j < 4; ++j) s_t[kf_lds(s, j)] = X[s][j];
        __syncthreads();
#pragma unroll
        for (int s = 0; s < VB / 16; ++s)
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const int a = trans_lds(s, f);
            __builtin_nontemporal_store(f32x4{s_t[a + 0], s_t[a + 1], s_t[a + 2], s_t[a + 3]},
                                        reinterpret_cast<f32x4*>(row_base + trans_off(s, f)));
          }
      }
    }
  };

  if constexpr (QDQ != kQdqNone) {
    if (p.quantize_initial) quantize();
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
      const int64_t out_row = (static_cast<int64_t>(t) * p.HV + h) * p.V + out_col0;
      const bool stored = QDQ != kQdqNone && p.readout_stored;

      float kh[NKEY], qh[NKEY];
      lds_keys(&s_k[tt][0], kh);
      lds_keys(&s_q[tt][0], qh);

      // the decay: GDN into the scale, KDA onto the registers' key rows
      float cn = KDA ? cs : cs * s_sc[tt][0];
      if (cn < kTinyScale) {                   // uniform: one scale per workgroup
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int e = 0; e < EV; ++e) S[s][e] *= cn;
        cn = 1.0f;
      }
      cs = cn;
      const float icn = rcp_hw(cn);
      if constexpr (KDA) {
        float al[NKEY];
        lds_keys(&s_al[tt][0], al);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int e = 0; e < EV; ++e) S[s][e] *= al[slot(s, e)];
      }

      float wv[NO];
      if constexpr (Cfg::KF_RS) {
        // the waves' partial sums go to LDS reduce-scattered (one (kind,
        // column) pair per lane and value); wave 0 then finishes each column
        // once, one lane per column (VB == 64), and hands the write
        // coefficients u / c' to every wave through LDS
        float r[4], pp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] = kh[0] * S[0][e];
          pp[e] = qh[0] * S[0][e];
        }
#pragma unroll
        for (int s = 1; s < NS; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = fmaf(kh[s], S[s][e], r[e]);
            pp[e] = fmaf(qh[s], S[s][e], pp[e]);
          }
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = rs_halves32(r[e], pp[e]);   // lanes < 32: r_e, else p_e
        const int kind = lane >> 5, par = (lane >> 4) & 1;
        s_red[red_buf][w][kind][4 * lr + par] = rs_rows16(x[0], x[1]);
        s_red[red_buf][w][kind][4 * lr + par + 2] = rs_rows16(x[2], x[3]);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(w) == 0) {
          float rj = s_red[red_buf][0][0][lane], pj = s_red[red_buf][0][1][lane];
#pragma unroll
          for (int ww = 1; ww < NW; ++ww) {
            rj += s_red[red_buf][ww][0][lane];
            pj += s_red[red_buf][ww][1][lane];
          }
          const float uj = beta * (s_v[tt][lane] - cn * rj);
          s_wv[lane] = uj * icn;
          if (!stored) {
            float oj = fmaf(qk, uj, cn * pj);
            if constexpr (HAD) oj = wht32_lanes(oj, lane) * 0.03125f;   // o back to the original basis
            store_out1(out_row + lane, oj);
          }
        }
        __syncthreads();
        const float4 wx = *reinterpret_cast<const float4*>(&s_wv[4 * lr]);
        wv[0] = wx.x; wv[1] = wx.y; wv[2] = wx.z; wv[3] = wx.w;
        red_buf ^= 1;
      } else {
        float r[NO], pp[NO];
        reduce_pass(kh, qh, r, pp);

        float u[NO], o[NO];
#pragma unroll
        for (int j = 0; j < NO; ++j) {
          const int col = AV ? row_idx(j) : 4 * lr + j;
          u[j] = beta * (s_v[tt][col] - cn * r[j]);
          o[j] = fmaf(qk, u[j], cn * pp[j]);
          wv[j] = u[j] * icn;
        }
        if constexpr (!HAD) {
          if (!stored) store_outputs(tt, out_row, o);
        } else if (!stored && __builtin_amdgcn_readfirstlane(w) == 0) {   // o back to the original basis (wave 0 stores it)
          float ow[1][NO];
#pragma unroll
          for (int j = 0; j < NO; ++j) ow[0][j] = o[j];
          wht32(ow, sg1, sg2, sg4);
#pragma unroll
          for (int j = 0; j < NO; ++j) o[j] = ow[0][j] * 0.03125f;
          store_outputs(tt, out_row, o);
        }
      }

      // S_reg += k_hat (x) wv
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          if constexpr (AV) S[s][e] = fmaf(kh[e], wv[s], S[s][e]);
          else S[s][e] = fmaf(kh[s], wv[e], S[s][e]);
        }

      if constexpr (QDQ != kQdqNone) {
        // (packed tiles: the store after the last token encodes the same
        // codes and scales from the unrounded registers, so that token's
        // rounding is skipped unless the readout needs the rounded state)
        if (!(PACKED && !stored && t == t1 - 1)) quantize();
        if (stored) {
          // o = q_hat^T S after rounding
          float q2[NKEY];
#pragma unroll
          for (int m = 0; m < NKEY; ++m) q2[m] = qh[m] * cs;
          float ps[NO], dummy[NO];
          reduce_pass(q2, q2, ps, dummy);
          if constexpr (HAD) {
            float pw[1][NO];
#pragma unroll
            for (int j = 0; j < NO; ++j) pw[0][j] = ps[j];
            wht32(pw, sg1, sg2, sg4);
#pragma unroll
            for (int j = 0; j < NO; ++j) ps[j] = pw[0][j] * 0.03125f;
          }
          store_outputs(tt, out_row, ps);
        }
      }
      if constexpr (ADDR == kPagedVar) {
        // a token that fills its page leaves the state there (the last token's
        // page is written after the loop)
        const int64_t pos = pos0 + (t - t0);
        if (pos > 0 && pos % p.page_size == 0 && pos != pos_last) {
          const int64_t row = load_index_uniform(p.page_indices, pg_start + (pos - 1) / p.page_size, p.idx64);
          store_tile(tile_base(row));
        }
      }
    }
    if constexpr (OUT_LDS) {
      if (staged && c0 + TC < t1) {   // more chunks follow: this chunk's outputs now
        __syncthreads();
        flush_outputs(c0, n);
      }
    }
  }

  store_tile(dst);
  if constexpr (OUT_LDS) {
    if (staged) {                     // the last chunk's outputs, after the tile's stores are issued
      __syncthreads();
      const int cl = t0 + ((t1 - t0 - 1) / TC) * TC;
      flush_outputs(cl, t1 - cl);
    }
  }
}

// The state traffic of a single-token step without its arithmetic
// (gdn_stream_rows): work unit u = r * chunks + c copies floats
// [512 c, 512 (c + 1)) of pair r's read row to its write row, 64 threads with
// two 128-bit non-temporal loads and stores each, half a chunk apart, in the
// decode kernels' XCD order.  Of the read-modify-write stream shapes measured
// over the paged B=256 rows (64 to 256 threads, 2 to 32 KiB per workgroup,
// plain or non-temporal), this one (2 KiB, 64 threads, non-temporal) moved
// the bytes fastest.
__global__ __launch_bounds__(64) void stream_rows_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                         const int64_t* __restrict__ slots, int64_t row_floats,
                                                         int32_t chunks, int32_t xcd_shift) {
  const int unit = xcd_unit(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), xcd_shift);
  const int r = unit / chunks;
  const int c = unit - r * chunks;
  const int64_t off = static_cast<int64_t>(c) * 512 + 4 * static_cast<int>(threadIdx.x);
  const f32x4* s = reinterpret_cast<const f32x4*>(src + slots[2 * r] * row_floats + off);
  f32x4* d = reinterpret_cast<f32x4*>(dst + slots[2 * r + 1] * row_floats + off);
  const f32x4 a = __builtin_nontemporal_load(s);
  const f32x4 b = __builtin_nontemporal_load(s + 64);
  __builtin_nontemporal_store(a, d);
  __builtin_nontemporal_store(b, d + 64);
}

// (read row, write row) of every sequence for one decoded token on a CSR
// page table (flashinfer.gdn_paged.gated_delta_rule_decode_paged, slots):
// computed once per decode step and shared by every layer's call.
__global__ __launch_bounds__(256) void paged_slots_kernel(const void* page_indices, const void* page_indptr,
                                                          const void* last_page_len, int32_t B, int32_t idx64,
                                                          int64_t* slots) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int64_t end = load_index(page_indptr, b + 1, idx64);
  const int64_t last = load_index(page_indices, end - 1, idx64);
  const int64_t lpl = load_index(last_page_len, b, idx64);
  slots[2 * b] = (lpl == 1) ? load_index(page_indices, end - 2, idx64) : last;
  slots[2 * b + 1] = last;
}

}  // namespace gdn

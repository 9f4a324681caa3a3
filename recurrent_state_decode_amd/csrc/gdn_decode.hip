// Host side of libgdn_decode: argument checks, kernel selection and launch
// for the C ABI declared in include/gdn_decode.h.
//
// Error convention (max.nn.state_space.kda_decode, Raises): a request whose
// types or extents bind no kernel is refused on the host before anything is
// launched; device-side index ranges are not checked.  A build compiled with
// GDN_DEVICE_CHECKS copies every call's index arrays to the host and
// validates them (host_checks.hpp) before it launches anything.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <type_traits>
#include <vector>

#include "gdn_decode.h"
#include "decode_kernel.hpp"
#include "host_checks.hpp"
#include "prefill_kernel.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

enum class Kind { GdnPooled, GdnPaged, KdaPooled, KdaPaged, GdnPagedVar, KdaPagedVar };

#ifdef GDN_DEVICE_CHECKS
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif

// Host copy of n elements of `bytes` each from device memory, after the work
// queued on `stream` before the call (which may produce the array) is done.
bool fetch(const void* dev, int64_t n, size_t bytes, std::vector<unsigned char>& host, hipStream_t stream) {
  host.resize(static_cast<size_t>(n > 0 ? n : 0) * bytes);
  if (n <= 0) return true;
  if (hipMemcpyAsync(host.data(), dev, host.size(), hipMemcpyDeviceToHost, stream) != hipSuccess) return false;
  return hipStreamSynchronize(stream) == hipSuccess;
}

// Checked builds: the preconditions of a pooled call (no-op otherwise).
int checked_pooled(const int32_t* cu, const int32_t* si, int32_t B, int32_t T, int64_t rows, void* stream) {
  if (!kChecked) return GDN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<unsigned char> hcu, hsi;
  if ((cu && !fetch(cu, B + 1, 4, hcu, s)) || !fetch(si, B, 4, hsi, s))
    return fail(GDN_ERR_HIP, "copying the index arrays to the host failed");
  std::string msg;
  if (!gdn_host::check_pooled(cu ? reinterpret_cast<const int32_t*>(hcu.data()) : nullptr,
                              reinterpret_cast<const int32_t*>(hsi.data()), B, T, rows, msg))
    return fail(GDN_ERR_PRECONDITION, "%s", msg.c_str());
  return GDN_OK;
}

// Checked builds: the preconditions of a paged call (no-op otherwise).
// page_size 0 and cu NULL: one token per sequence (with optional slots).
int checked_paged(const int32_t* cu, const void* pi, const void* ptr, const void* lpl, bool i64, const int64_t* slots,
                  int32_t B, int32_t T, int32_t page_size, int64_t rows, int64_t nnz, void* stream) {
  if (!kChecked) return GDN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t ib = i64 ? 8 : 4;
  std::vector<unsigned char> hcu, hpi, hptr, hlpl, hsl;
  if ((cu && !fetch(cu, B + 1, 4, hcu, s)) || !fetch(pi, nnz, ib, hpi, s) || !fetch(ptr, B + 1, ib, hptr, s) ||
      !fetch(lpl, B, ib, hlpl, s) || (slots && !fetch(slots, 2 * int64_t(B), 8, hsl, s)))
    return fail(GDN_ERR_HIP, "copying the index arrays to the host failed");
  std::string msg;
  const bool ok = cu ? gdn_host::check_paged_varlen(reinterpret_cast<const int32_t*>(hcu.data()), hpi.data(),
                                                    hptr.data(), hlpl.data(), i64, B, T, page_size, rows, nnz, msg)
                     : gdn_host::check_paged(hpi.data(), hptr.data(), hlpl.data(), i64,
                                             slots ? reinterpret_cast<const int64_t*>(hsl.data()) : nullptr, B,
                                             page_size, rows, nnz, msg);
  if (!ok) return fail(GDN_ERR_PRECONDITION, "%s", msg.c_str());
  return GDN_OK;
}

// Workgroup shapes: V-block width VB (one workgroup per V-block of one
// sequence and value head) and threads per workgroup NT.  Chosen per key
// head dim, pool layout, whether the tile is quantised, and tokens per
// sequence (every workgroup normalises and gates its sequence's tokens, so
// narrow V-blocks pay that work V/VB times over):
//   K=128, V_FIRST, no QDQ, about one token per sequence (T <= 1.5 B):
//                            GDN: VB=8,  NT=128 (4 KiB of state per workgroup)
//                            KDA: VB=16, NT=128 (its per-channel gates cost
//                            more per V-block; measured 12 % faster than VB=8)
//   K=128, K_FIRST, no QDQ, T <= 1.5 B:
//                            VB=32, NT=256 (128-byte row segments; 5-7 %
//                            faster than VB=64, VB=16 is 25 % slower)
//   K=128, V_FIRST, GDN, no QDQ, longer suffixes:
//                            VB=32, NT=256 (5-6 % faster than VB=64 on 4-token
//                            suffixes; on a K_FIRST pool it is 5 % slower,
//                            and KDA's per-channel gates favour VB=64)
//   K=128, GDN, packed fp8 tiles on a V_FIRST pool, T <= 1.5 B:
//                            VB=64, NT=128 (launch_fp8p_gdn_vfirst)
//   K=128, otherwise:        VB=64, NT=256 (fp8 tiles need block_v == VB; the
//                            int8_hadamard32 codec is compiled for this shape)
//   K=16:                    VB=16, NT=64
// V must be a multiple of VB.
struct Shape {
  int VB, NT;
};

bool is_kda(Kind k) { return k == Kind::KdaPooled || k == Kind::KdaPaged || k == Kind::KdaPagedVar; }

// Packed int8_hadamard32 tiles, about one token per sequence.
constexpr int kPackedVB = 64, kPackedNT = 256;

Shape shape_for(int K, bool vfirst, bool qdq, int64_t T, int64_t B, bool kda, bool packed) {
  if (K == 128 && packed && 2 * T <= 3 * B) return Shape{kPackedVB, kPackedNT};
  if (K == 128 && !qdq && 2 * T <= 3 * B) return vfirst ? Shape{kda ? 16 : 8, 128} : Shape{32, 256};
  if (K == 128 && !qdq && !kda && vfirst) return Shape{32, 256};
  if (K == 128) return Shape{64, 256};
  if (K == 16) return Shape{16, 64};
  return Shape{0, 0};
}

// Key head dims with kernels, and the V multiple every shape of that K accepts.
struct HeadCfg {
  int K, VB;
};
constexpr HeadCfg kHeads[] = {{16, 16}, {128, 64}};

// LDS reserved per workgroup (static plus dynamic shared memory the kernel
// never touches) for shapes whose state stream moves faster with fewer
// workgroups resident per CU (160 KiB of LDS per CU).  Measured with
// interleaved timing rounds:
//   paged GDN, one token, V_FIRST 8-column blocks:   12 288 bytes (13 per CU
//       instead of the 14 the registers allow): B=256 174.7 -> 172.4 us
//   paged KDA, one token, V_FIRST 16-column blocks:  20 992 bytes (7 instead
//       of 10): B=256 179.4 -> 174.5 us
//   pooled KDA, several tokens, V_FIRST 64-column blocks: 41 472 bytes (3
//       instead of 4): B=128 x 1..8 tokens 104.6 -> 103.0 us
// Fewer are slower again (paged GDN at 9 per CU 180 us), and the other
// shapes measured flat.  (hipFuncGetAttributes gives the static part; the
// reservation is the same on every device, so one cached value serves all.)
// 0: no reservation.
template <int VB, int NT, bool VF, bool KDA, int QDQ, int ADDR>
constexpr int kLdsPerWorkgroup =
    (QDQ != gdn::kQdqNone || !VF) ? 0
    : (VB == 8 && NT == 128 && !KDA && ADDR == gdn::kPaged1)  ? 12288
    : (VB == 16 && NT == 128 && KDA && ADDR == gdn::kPaged1)  ? 20992
    : (VB == 64 && NT == 256 && KDA && ADDR == gdn::kPooled)  ? 41472
                                                             : 0;

template <int K, int VB, int NT, bool VF, bool KDA, int QDQ, int ADDR, typename TIn>
hipError_t launch_one(const gdn::Params& p, int64_t units, hipStream_t stream) {
  auto kernel = gdn::decode_kernel<K, VB, NT, VF, KDA, QDQ, ADDR, TIn>;
  size_t pad = 0;
  if constexpr (kLdsPerWorkgroup<VB, NT, VF, KDA, QDQ, ADDR> > 0) {
    static size_t cached = 0;      // (the kernel's static LDS does not change at run time)
    static bool known = false;
    if (!known) {
      hipFuncAttributes a{};
      if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(kernel)) == hipSuccess) {
        const size_t want = kLdsPerWorkgroup<VB, NT, VF, KDA, QDQ, ADDR>;
        cached = a.sharedSizeBytes < want ? want - a.sharedSizeBytes : 0;
      }
      known = true;
    }
    pad = cached;
  }
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(units)), dim3(NT), pad, stream, p);
  return hipGetLastError();
}

struct Sel {
  bool vfirst;
  int qdq;          // gdn::Qdq
  bool bf16;
};

// The int8_hadamard32 codec is compiled for the K=128, VB=64 shape only.
template <int K, int VB, int NT>
constexpr bool kHadShape = K == 128 && VB == 64 && NT == 256;

template <int K, int VB, int NT, bool VF, bool KDA, int ADDR, typename TIn>
hipError_t launch_qdq(const gdn::Params& p, int64_t units, int qdq, hipStream_t s) {
  if (qdq == gdn::kQdqTile) return launch_one<K, VB, NT, VF, KDA, gdn::kQdqTile, ADDR, TIn>(p, units, s);
  if (qdq == gdn::kQdqTilePacked) return launch_one<K, VB, NT, VF, KDA, gdn::kQdqTilePacked, ADDR, TIn>(p, units, s);
  if (qdq == gdn::kQdqHad) {
    if constexpr (kHadShape<K, VB, NT>) return launch_one<K, VB, NT, VF, KDA, gdn::kQdqHad, ADDR, TIn>(p, units, s);
    return hipErrorInvalidValue;
  }
  if (qdq == gdn::kQdqHadPacked) {   // packed tiles: one layout, so VF is not instantiated
    if constexpr (kHadShape<K, VB, NT> && !VF)
      return launch_one<K, VB, NT, false, KDA, gdn::kQdqHadPacked, ADDR, TIn>(p, units, s);
    return hipErrorInvalidValue;
  }
  return launch_one<K, VB, NT, VF, KDA, gdn::kQdqNone, ADDR, TIn>(p, units, s);
}

template <int K, int VB, int NT, bool KDA, int ADDR, typename TIn>
hipError_t launch_layout_qdq(const gdn::Params& p, int64_t units, Sel sel, hipStream_t s) {
  return sel.vfirst ? launch_qdq<K, VB, NT, true, KDA, ADDR, TIn>(p, units, sel.qdq, s)
                    : launch_qdq<K, VB, NT, false, KDA, ADDR, TIn>(p, units, sel.qdq, s);
}

template <int K, int VB, int NT, bool KDA, int ADDR>
hipError_t launch_io(const gdn::Params& p, int64_t units, Sel sel, hipStream_t s) {
  return sel.bf16 ? launch_layout_qdq<K, VB, NT, KDA, ADDR, gdn::bf16_t>(p, units, sel, s)
                  : launch_layout_qdq<K, VB, NT, KDA, ADDR, float>(p, units, sel, s);
}

template <int K, int VB, int NT>
hipError_t launch_kind(Kind kind, const gdn::Params& p, int64_t units, Sel sel, hipStream_t s) {
  switch (kind) {
    case Kind::GdnPooled: return launch_io<K, VB, NT, false, gdn::kPooled>(p, units, sel, s);
    case Kind::GdnPaged: return launch_io<K, VB, NT, false, gdn::kPaged1>(p, units, sel, s);
    case Kind::KdaPooled: return launch_io<K, VB, NT, true, gdn::kPooled>(p, units, sel, s);
    case Kind::KdaPaged: return launch_io<K, VB, NT, true, gdn::kPaged1>(p, units, sel, s);
    case Kind::GdnPagedVar: return launch_io<K, VB, NT, false, gdn::kPagedVar>(p, units, sel, s);
    case Kind::KdaPagedVar: return launch_io<K, VB, NT, true, gdn::kPagedVar>(p, units, sel, s);
  }
  return hipErrorInvalidValue;
}

int vblock_for(int K) {
  for (const auto& h : kHeads)
    if (h.K == K) return h.VB;
  return 0;
}

bool head_supported(int K, int V) {
  const int vb = vblock_for(K);
  return vb > 0 && V % vb == 0;
}

// Shapes used without QDQ only (K=128, one layout): one instantiation per kind and io type.
template <bool VF, int VB, int NT>
hipError_t launch_noqdq(Kind kind, const gdn::Params& p, int64_t units, Sel sel, hipStream_t s) {
  auto go = [&](auto kda, auto addr) -> hipError_t {
    constexpr bool KDA = decltype(kda)::value;
    constexpr int ADDR = decltype(addr)::value;
    return sel.bf16 ? launch_one<128, VB, NT, VF, KDA, gdn::kQdqNone, ADDR, gdn::bf16_t>(p, units, s)
                    : launch_one<128, VB, NT, VF, KDA, gdn::kQdqNone, ADDR, float>(p, units, s);
  };
  using F = std::false_type;
  using Tr = std::true_type;
  using Pool = std::integral_constant<int, gdn::kPooled>;
  using Pg1 = std::integral_constant<int, gdn::kPaged1>;
  using PgV = std::integral_constant<int, gdn::kPagedVar>;
  switch (kind) {
    case Kind::GdnPooled: return go(F{}, Pool{});
    case Kind::GdnPaged: return go(F{}, Pg1{});
    case Kind::KdaPooled: return go(Tr{}, Pool{});
    case Kind::KdaPaged: return go(Tr{}, Pg1{});
    case Kind::GdnPagedVar: return go(F{}, PgV{});
    case Kind::KdaPagedVar: return go(Tr{}, PgV{});
  }
  return hipErrorInvalidValue;
}

// Packed int8_hadamard32 tiles in a narrower shape (single-token calls): one instantiation per kind and io type.
template <int VB, int NT>
hipError_t launch_packed(Kind kind, const gdn::Params& p, int64_t units, Sel sel, hipStream_t s) {
  auto go = [&](auto kda, auto addr) -> hipError_t {
    constexpr bool KDA = decltype(kda)::value;
    constexpr int ADDR = decltype(addr)::value;
    return sel.bf16 ? launch_one<128, VB, NT, false, KDA, gdn::kQdqHadPacked, ADDR, gdn::bf16_t>(p, units, s)
                    : launch_one<128, VB, NT, false, KDA, gdn::kQdqHadPacked, ADDR, float>(p, units, s);
  };
  using F = std::false_type;
  using Tr = std::true_type;
  using Pool = std::integral_constant<int, gdn::kPooled>;
  using Pg1 = std::integral_constant<int, gdn::kPaged1>;
  using PgV = std::integral_constant<int, gdn::kPagedVar>;
  switch (kind) {
    case Kind::GdnPooled: return go(F{}, Pool{});
    case Kind::GdnPaged: return go(F{}, Pg1{});
    case Kind::KdaPooled: return go(Tr{}, Pool{});
    case Kind::KdaPaged: return go(Tr{}, Pg1{});
    case Kind::GdnPagedVar: return go(F{}, PgV{});
    case Kind::KdaPagedVar: return go(Tr{}, PgV{});
  }
  return hipErrorInvalidValue;
}

// Packed fp8 tiles of a V_FIRST pool, GDN, about one token per sequence: the
// 64-column tile over 128 threads (paged B=256: 0.080 against 0.088 ms with
// 256 threads; KDA and K_FIRST pools measured slower or no faster that way).
constexpr int kFp8SmallVB = 64, kFp8SmallNT = 128;

template <int VB, int NT>
hipError_t launch_fp8p_gdn_vfirst(Kind kind, const gdn::Params& p, int64_t units, Sel sel, hipStream_t s) {
  auto go = [&](auto addr) -> hipError_t {
    constexpr int ADDR = decltype(addr)::value;
    return sel.bf16 ? launch_one<128, VB, NT, true, false, gdn::kQdqTilePacked, ADDR, gdn::bf16_t>(p, units, s)
                    : launch_one<128, VB, NT, true, false, gdn::kQdqTilePacked, ADDR, float>(p, units, s);
  };
  switch (kind) {
    case Kind::GdnPooled: return go(std::integral_constant<int, gdn::kPooled>{});
    case Kind::GdnPaged: return go(std::integral_constant<int, gdn::kPaged1>{});
    case Kind::GdnPagedVar: return go(std::integral_constant<int, gdn::kPagedVar>{});
    default: return hipErrorInvalidValue;
  }
}

int check_options(const gdn_options* o, int K, int V, Kind kind) {
  if (!o) return fail(GDN_ERR_INVALID, "options pointer is NULL");
  if (o->io_dtype != GDN_F32 && o->io_dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID, "io_dtype must be GDN_F32 or GDN_BF16 (got %d)", o->io_dtype);
  if (o->out_dtype != GDN_F32 && o->out_dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID, "out_dtype must be GDN_F32 or GDN_BF16 (got %d)", o->out_dtype);
  if (o->state_layout != GDN_K_FIRST && o->state_layout != GDN_V_FIRST)
    return fail(GDN_ERR_INVALID, "state_layout must be GDN_K_FIRST or GDN_V_FIRST (got %d)", o->state_layout);
  if (o->beta_mode != GDN_BETA_LOGITS && o->beta_mode != GDN_BETA_PROBABILITY)
    return fail(GDN_ERR_INVALID, "beta_mode must be LOGITS or PROBABILITY (got %d)", o->beta_mode);
  if (o->gate_mode != GDN_GATE_ORIGINAL && o->gate_mode != GDN_GATE_SAFE)
    return fail(GDN_ERR_INVALID, "gate_mode must be ORIGINAL or SAFE (got %d)", o->gate_mode);
  if (o->gate_mode == GDN_GATE_SAFE)
    return fail(GDN_ERR_UNSUPPORTED, "gate_mode SAFE needs a gate lower bound this library does not define");
  if (o->qdq != GDN_QDQ_NONE && o->qdq != GDN_QDQ_FP8_E4M3_TILE && o->qdq != GDN_QDQ_INT8_HADAMARD32)
    return fail(GDN_ERR_INVALID, "qdq must be NONE, FP8_E4M3_TILE or INT8_HADAMARD32 (got %d)", o->qdq);
  if (o->readout != GDN_READOUT_WORKING && o->readout != GDN_READOUT_STORED)
    return fail(GDN_ERR_INVALID, "readout must be WORKING or STORED (got %d)", o->readout);
  const bool paged = kind == Kind::GdnPaged || kind == Kind::KdaPaged || kind == Kind::GdnPagedVar ||
                     kind == Kind::KdaPagedVar;
  if (paged && o->index_dtype != GDN_I32 && o->index_dtype != GDN_I64)
    return fail(GDN_ERR_INVALID, "index_dtype must be GDN_I32 or GDN_I64 (got %d)", o->index_dtype);
  if (!(o->scale >= 0.0f) || std::isinf(o->scale))
    return fail(GDN_ERR_INVALID, "scale must be finite and >= 0 (0 selects 1/sqrt(K))");
  if (o->qdq == GDN_QDQ_FP8_E4M3_TILE) {
    if (o->block_v <= 0 || V % o->block_v != 0)
      return fail(GDN_ERR_INVALID, "block_v=%d must be positive and divide V=%d", o->block_v, V);
    if (o->block_v != vblock_for(K))
      return fail(GDN_ERR_UNSUPPORTED, "fp8 tile QDQ is compiled for block_v=%d at K=%d (got %d)", vblock_for(K), K,
                  o->block_v);
  }
  if (o->qdq == GDN_QDQ_INT8_HADAMARD32) {
    // block_v is the execution tile width: any multiple of 32 that divides V
    // gives the same result, since no 32-value group crosses a tile
    if (o->block_v <= 0 || V % o->block_v != 0 || o->block_v % 32 != 0)
      return fail(GDN_ERR_INVALID, "block_v=%d must be a positive multiple of 32 dividing V=%d for int8_hadamard32",
                  o->block_v, V);
    if (K != 128) return fail(GDN_ERR_UNSUPPORTED, "the int8_hadamard32 codec is compiled for K=128 (got K=%d)", K);
  }
  if (o->state_storage != GDN_STORAGE_F32 && o->state_storage != GDN_STORAGE_I8H32 &&
      o->state_storage != GDN_STORAGE_FP8_TILE)
    return fail(GDN_ERR_INVALID, "state_storage must be GDN_STORAGE_F32, I8H32 or FP8_TILE (got %d)",
                o->state_storage);
  if (o->state_storage == GDN_STORAGE_FP8_TILE && o->qdq != GDN_QDQ_FP8_E4M3_TILE)
    return fail(GDN_ERR_INVALID, "state_storage FP8_TILE holds fp8 tile codes: qdq must be FP8_E4M3_TILE");
  if (o->state_storage == GDN_STORAGE_I8H32) {
    if (o->qdq != GDN_QDQ_INT8_HADAMARD32)
      return fail(GDN_ERR_INVALID, "state_storage I8H32 holds int8_hadamard32 codes: qdq must be INT8_HADAMARD32");
    if (o->state_layout != GDN_K_FIRST)
      return fail(GDN_ERR_UNSUPPORTED, "packed tiles have one layout ([K][V] codes): state_layout must be K_FIRST");
  }
  return GDN_OK;
}

int check_dims(int32_t B, int32_t HK, int32_t HV, int32_t K, int32_t V) {
  if (B <= 0 || HK <= 0 || HV <= 0 || K <= 0 || V <= 0)
    return fail(GDN_ERR_INVALID, "dimensions must be positive (B=%d HK=%d HV=%d K=%d V=%d)", B, HK, HV, K, V);
  if (HV % HK != 0) return fail(GDN_ERR_INVALID, "HV=%d is not a multiple of HK=%d", HV, HK);
  if (!head_supported(K, V)) return fail(GDN_ERR_UNSUPPORTED, "no kernel for head dims K=%d V=%d", K, V);
  return GDN_OK;
}

// n / d == (n * m) >> s for every 0 <= n < 2^31, with s = 31 + ceil(log2 d)
// and m = floor(2^s / d) + 1 (the error term n (m d - 2^s) / (d 2^s) stays
// below 1/d).
void fast_div_consts(uint32_t d, uint64_t& m, int32_t& s) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  s = 31 + l;
  m = ((1ull << s) / d) + 1;
}

void fill_common(gdn::Params& p, const gdn_options* o, Kind kind, int32_t B, int32_t T, int32_t HK, int32_t HV,
                 int32_t K, int32_t V) {
  p.B = B;
  p.HK = HK;
  p.HV = HV;
  p.V = V;
  const Shape sh = shape_for(K, o->state_layout == GDN_V_FIRST, o->qdq != GDN_QDQ_NONE, T, B, is_kda(kind),
                             o->state_storage == GDN_STORAGE_I8H32);
  p.nvb = V / sh.VB;
  p.xcd_shift = 6;   // 64 consecutive work units per XCD
  fast_div_consts(static_cast<uint32_t>(p.nvb), p.div_nvb_m, p.div_nvb_s);
  fast_div_consts(static_cast<uint32_t>(HV), p.div_hv_m, p.div_hv_s);
  fast_div_consts(static_cast<uint32_t>(HV / HK), p.div_gqa_m, p.div_gqa_s);
  p.gqa = HV / HK;
  p.scale = o->scale > 0.0f ? o->scale : 1.0f / std::sqrt(static_cast<float>(K));
  p.l2norm = o->use_qk_l2norm ? 1 : 0;
  p.out_bf16 = o->out_dtype == GDN_BF16;
  p.beta_prob = o->beta_mode == GDN_BETA_PROBABILITY;
  p.idx64 = o->index_dtype == GDN_I64;
  p.quantize_initial = (o->qdq != GDN_QDQ_NONE && o->quantize_initial) ? 1 : 0;
  p.readout_stored = (o->qdq != GDN_QDQ_NONE && o->readout == GDN_READOUT_STORED) ? 1 : 0;
  p.slots = o->slots;
}

int run(Kind kind, const gdn::Params& p, int K, int32_t T, const gdn_options* o, void* stream) {
  const int64_t units = static_cast<int64_t>(p.B) * p.HV * p.nvb;
  if (units > 0x7fffffffLL) return fail(GDN_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)units);
  const int qdq = o->qdq == GDN_QDQ_FP8_E4M3_TILE
                      ? (o->state_storage == GDN_STORAGE_FP8_TILE ? gdn::kQdqTilePacked : gdn::kQdqTile)
                  : o->qdq == GDN_QDQ_INT8_HADAMARD32
                      ? (o->state_storage == GDN_STORAGE_I8H32 ? gdn::kQdqHadPacked : gdn::kQdqHad)
                      : gdn::kQdqNone;
  const Sel sel{o->state_layout == GDN_V_FIRST, qdq, o->io_dtype == GDN_BF16};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipErrorInvalidValue;
  switch (K) {
    case 16: err = launch_kind<16, 16, 64>(kind, p, units, sel, s); break;
    case 128:
      if (sel.qdq == gdn::kQdqHadPacked && 2 * T <= 3 * p.B) {   // the packed single-token shape
        err = launch_packed<kPackedVB, kPackedNT>(kind, p, units, sel, s);
        break;
      }
      if (sel.qdq == gdn::kQdqTilePacked && sel.vfirst && !is_kda(kind) && 2 * T <= 3 * p.B) {
        err = launch_fp8p_gdn_vfirst<kFp8SmallVB, kFp8SmallNT>(kind, p, units, sel, s);
        break;
      }
      switch (shape_for(K, sel.vfirst, sel.qdq != gdn::kQdqNone, T, p.B, is_kda(kind), false).VB) {
        case 8: err = launch_noqdq<true, 8, 128>(kind, p, units, sel, s); break;
        case 16: err = launch_noqdq<true, 16, 128>(kind, p, units, sel, s); break;
        case 32:
          err = sel.vfirst ? launch_noqdq<true, 32, 256>(kind, p, units, sel, s)
                           : launch_noqdq<false, 32, 256>(kind, p, units, sel, s);
          break;
        default: err = launch_kind<128, 64, 256>(kind, p, units, sel, s);
      }
      break;
    default: return fail(GDN_ERR_UNSUPPORTED, "no kernel for K=%d", K);
  }
  if (err != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return GDN_OK;
}

}  // namespace

extern "C" {

void gdn_options_init(gdn_options* o) {
  if (!o) return;
  o->scale = 0.0f;
  o->use_qk_l2norm = 1;
  o->io_dtype = GDN_BF16;
  o->out_dtype = GDN_BF16;
  o->state_layout = GDN_K_FIRST;
  o->beta_mode = GDN_BETA_LOGITS;
  o->gate_mode = GDN_GATE_ORIGINAL;
  o->index_dtype = GDN_I32;
  o->qdq = GDN_QDQ_NONE;
  o->block_v = 64;
  o->quantize_initial = 0;
  o->readout = GDN_READOUT_WORKING;
  o->slots = nullptr;
  o->state_storage = GDN_STORAGE_F32;
}

int gdn_decode_pooled(const void* q, const void* k, const void* v, const void* a, const void* b,
                      const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                      const int32_t* state_indices, float* state_pool, void* out, int32_t B, int32_t T,
                      int32_t HK, int32_t HV, int32_t K, int32_t V, int64_t num_slots, const gdn_options* opt,
                      void* stream) {
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !state_indices || !state_pool || !out)
    return fail(GDN_ERR_INVALID, "a required pointer is NULL");
  if (int rc = check_dims(B, HK, HV, K, V)) return rc;
  if (T < 0 || num_slots <= 0) return fail(GDN_ERR_INVALID, "T must be >= 0 and num_slots > 0");
  if (!cu_seqlens && T != B)
    return fail(GDN_ERR_SHAPE, "without cu_seqlens each sequence has one token, so T (%d) must equal B (%d)", T, B);
  if (int rc = check_options(opt, K, V, Kind::GdnPooled)) return rc;
  if (opt->slots) return fail(GDN_ERR_INVALID, "slots apply to paged calls only");
  gdn::Params p{};
  p.q = q; p.k = k; p.v = v; p.gate = a; p.beta = b;
  p.a_log = A_log; p.dt_bias = dt_bias;
  p.cu_seqlens = cu_seqlens; p.state_indices = state_indices;
  p.pool = state_pool; p.out = out;
  fill_common(p, opt, Kind::GdnPooled, B, T, HK, HV, K, V);
  if (int rc = checked_pooled(cu_seqlens, state_indices, B, T, num_slots, stream)) return rc;
  if (T == 0) { g_last_error.clear(); return GDN_OK; }
  return run(Kind::GdnPooled, p, K, T, opt, stream);
}

}  // extern "C"

namespace {

// Shared body of the paged entry points.  T == B and cu_seqlens == NULL for
// one token per sequence (P3 semantics), else varlen suffixes with page_size.
int paged_call(Kind kind, const void* q, const void* k, const void* v, const void* gate, const void* beta,
               const float* a_log, const float* dt_bias, const int32_t* cu_seqlens, const void* page_indices,
               const void* page_indptr, const void* last_page_len, int32_t page_size, float* state_pool, void* out,
               int32_t B, int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V, int64_t num_pages, int64_t nnz,
               const gdn_options* opt, void* stream) {
  const bool var = kind == Kind::GdnPagedVar || kind == Kind::KdaPagedVar;
  if (!q || !k || !v || !gate || !beta || !a_log || !dt_bias || !page_indices || !page_indptr || !last_page_len ||
      !state_pool || !out || (var && !cu_seqlens))
    return fail(GDN_ERR_INVALID, "a required pointer is NULL");
  if (int rc = check_dims(B, HK, HV, K, V)) return rc;
  if (num_pages <= 0 || nnz <= 0) return fail(GDN_ERR_INVALID, "num_pages and nnz must be positive");
  if (nnz < B) return fail(GDN_ERR_SHAPE, "nnz (%lld) must be at least B (%d): every sequence owns a page",
                           (long long)nnz, B);
  if (var && page_size <= 0) return fail(GDN_ERR_INVALID, "page_size must be positive (got %d)", page_size);
  if (var && T < 0) return fail(GDN_ERR_INVALID, "T must be >= 0");
  if (int rc = check_options(opt, K, V, kind)) return rc;
  if (var && opt->slots) return fail(GDN_ERR_INVALID, "slots apply to single-token paged calls only");
  gdn::Params p{};
  p.q = q; p.k = k; p.v = v; p.gate = gate; p.beta = beta;
  p.a_log = a_log; p.dt_bias = dt_bias;
  p.cu_seqlens = cu_seqlens;
  p.page_indices = page_indices; p.page_indptr = page_indptr; p.last_page_len = last_page_len;
  p.page_size = page_size;
  p.pool = state_pool; p.out = out;
  fill_common(p, opt, kind, B, T, HK, HV, K, V);
  if (int rc = checked_paged(cu_seqlens, page_indices, page_indptr, last_page_len, p.idx64 != 0, opt->slots, B, T,
                             page_size, num_pages, nnz, stream))
    return rc;
  if (T == 0) { g_last_error.clear(); return GDN_OK; }
  return run(kind, p, K, T, opt, stream);
}

}  // namespace

extern "C" {

int gdn_decode_paged(const void* q, const void* k, const void* v, const void* a, const void* b,
                     const float* A_log, const float* dt_bias, const void* page_indices, const void* page_indptr,
                     const void* last_page_len, float* state_pool, void* out, int32_t B, int32_t HK, int32_t HV,
                     int32_t K, int32_t V, int64_t num_pages, int64_t nnz, const gdn_options* opt, void* stream) {
  return paged_call(Kind::GdnPaged, q, k, v, a, b, A_log, dt_bias, nullptr, page_indices, page_indptr,
                    last_page_len, 0, state_pool, out, B, B, HK, HV, K, V, num_pages, nnz, opt, stream);
}

int kda_decode_paged(const void* q, const void* k, const void* v, const void* raw_gate, const void* beta_logits,
                     const float* a_log, const float* dt_bias, const void* page_indices, const void* page_indptr,
                     const void* last_page_len, float* state_pool, void* out, int32_t B, int32_t HK, int32_t HV,
                     int32_t K, int32_t V, int64_t num_pages, int64_t nnz, const gdn_options* opt, void* stream) {
  return paged_call(Kind::KdaPaged, q, k, v, raw_gate, beta_logits, a_log, dt_bias, nullptr, page_indices,
                    page_indptr, last_page_len, 0, state_pool, out, B, B, HK, HV, K, V, num_pages, nnz, opt, stream);
}

int gdn_decode_paged_varlen(const void* q, const void* k, const void* v, const void* a, const void* b,
                            const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                            const void* page_indices, const void* page_indptr, const void* last_page_len,
                            int32_t page_size, float* state_pool, void* out, int32_t B, int32_t T, int32_t HK,
                            int32_t HV, int32_t K, int32_t V, int64_t num_pages, int64_t nnz,
                            const gdn_options* opt, void* stream) {
  return paged_call(Kind::GdnPagedVar, q, k, v, a, b, A_log, dt_bias, cu_seqlens, page_indices, page_indptr,
                    last_page_len, page_size, state_pool, out, B, T, HK, HV, K, V, num_pages, nnz, opt, stream);
}

int kda_decode_paged_varlen(const void* q, const void* k, const void* v, const void* raw_gate,
                            const void* beta_logits, const float* a_log, const float* dt_bias,
                            const int32_t* cu_seqlens, const void* page_indices, const void* page_indptr,
                            const void* last_page_len, int32_t page_size, float* state_pool, void* out, int32_t B,
                            int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V, int64_t num_pages,
                            int64_t nnz, const gdn_options* opt, void* stream) {
  return paged_call(Kind::KdaPagedVar, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, page_indices,
                    page_indptr, last_page_len, page_size, state_pool, out, B, T, HK, HV, K, V, num_pages, nnz, opt,
                    stream);
}

int gdn_paged_decode_slots(const void* page_indices, const void* page_indptr, const void* last_page_len, int32_t B,
                           int32_t index_dtype, int64_t* slots, void* stream) {
  if (!page_indices || !page_indptr || !last_page_len || !slots) return fail(GDN_ERR_INVALID, "a required pointer is NULL");
  if (B <= 0) return fail(GDN_ERR_INVALID, "B must be positive (got %d)", B);
  if (index_dtype != GDN_I32 && index_dtype != GDN_I64)
    return fail(GDN_ERR_INVALID, "index_dtype must be GDN_I32 or GDN_I64 (got %d)", index_dtype);
  if (kChecked) {
    // no nnz or num_pages here: the table's structure only (the decode call
    // that takes these slots checks them against the whole table)
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool i64 = index_dtype == GDN_I64;
    std::vector<unsigned char> hptr, hlpl;
    if (!fetch(page_indptr, B + 1, i64 ? 8 : 4, hptr, s) || !fetch(last_page_len, B, i64 ? 8 : 4, hlpl, s))
      return fail(GDN_ERR_HIP, "copying the index arrays to the host failed");
    std::string msg;
    if (!gdn_host::check_table(hptr.data(), hlpl.data(), i64, B, 0, -1, msg))
      return fail(GDN_ERR_PRECONDITION, "%s", msg.c_str());
    for (int32_t b = 0; b < B; ++b)
      if (gdn_host::index_at(hlpl.data(), b, i64) == 1 &&
          gdn_host::index_at(hptr.data(), b + 1, i64) - gdn_host::index_at(hptr.data(), b, i64) < 2)
        return fail(GDN_ERR_PRECONDITION, "sequence %d opens a new page but has no previous page", b);
  }
  hipLaunchKernelGGL(gdn::paged_slots_kernel, dim3((B + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     page_indices, page_indptr, last_page_len, B, index_dtype == GDN_I64 ? 1 : 0, slots);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return GDN_OK;
}

}  // extern "C"

namespace {

// Shared body of the chunked prefill entry points (GDN / KDA).
int prefill_call(bool kda, const void* q, const void* k, const void* v, const void* gate, const void* beta,
                 const float* a_log, const float* dt_bias, const int32_t* cu_seqlens, const void* page_indices,
                 const void* page_indptr, const void* last_page_len, int32_t page_size, float* state_pool,
                 void* out, int32_t B, int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V, int64_t num_pages,
                 int64_t nnz, const gdn_options* opt, void* stream) {
  if (!q || !k || !v || !gate || !beta || !a_log || !dt_bias || !cu_seqlens || !page_indices || !page_indptr ||
      !last_page_len || !state_pool || !out)
    return fail(GDN_ERR_INVALID, "a required pointer is NULL");
  if (int rc = check_dims(B, HK, HV, K, V)) return rc;
  if (K != 128 || V % 128 != 0)
    return fail(GDN_ERR_UNSUPPORTED, "the chunked prefill is compiled for K=128 and V a multiple of 128 (K=%d V=%d)", K,
                V);
  if (num_pages <= 0 || nnz <= 0) return fail(GDN_ERR_INVALID, "num_pages and nnz must be positive");
  if (nnz < B) return fail(GDN_ERR_SHAPE, "nnz (%lld) must be at least B (%d): every sequence owns a page",
                           (long long)nnz, B);
  if (page_size <= 0) return fail(GDN_ERR_INVALID, "page_size must be positive (got %d)", page_size);
  if (page_size % gdn::kChunk != 0)
    return fail(GDN_ERR_UNSUPPORTED, "the chunked prefill needs a page size that is a multiple of %d (got %d)",
                gdn::kChunk, page_size);
  if (T < 0) return fail(GDN_ERR_INVALID, "T must be >= 0");
  if (int rc = check_options(opt, K, V, kda ? Kind::KdaPagedVar : Kind::GdnPagedVar)) return rc;
  if (opt->slots) return fail(GDN_ERR_INVALID, "slots apply to single-token paged calls only");
  if (opt->qdq != GDN_QDQ_NONE) return fail(GDN_ERR_UNSUPPORTED, "the chunked prefill has no state quantisation");
  if (int rc = checked_paged(cu_seqlens, page_indices, page_indptr, last_page_len, opt->index_dtype == GDN_I64,
                             nullptr, B, T, page_size, num_pages, nnz, stream))
    return rc;
  if (T == 0) { g_last_error.clear(); return GDN_OK; }
  gdn::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.gate = gate; p.beta = beta;
  p.a_log = a_log; p.dt_bias = dt_bias;
  p.cu_seqlens = cu_seqlens;
  p.page_indices = page_indices; p.page_indptr = page_indptr; p.last_page_len = last_page_len;
  p.page_size = page_size;
  p.pool = state_pool; p.out = out;
  p.B = B; p.HK = HK; p.HV = HV; p.V = V;
  constexpr int VT = 2, NW = 4;     // two 16-column value tiles per wave, 4 waves: 128 columns per workgroup
  p.nvb = V / gdn::kPrefillVBlk<VT, NW>;
  p.gqa = HV / HK;
  // keep the units that share a key head (gqa heads x nvb V-blocks) on one XCD
  p.xcd_shift = 0;
  while ((1 << p.xcd_shift) < p.gqa * p.nvb && p.xcd_shift < 6) ++p.xcd_shift;
  p.scale = opt->scale > 0.0f ? opt->scale : 1.0f / std::sqrt(static_cast<float>(K));
  p.l2norm = opt->use_qk_l2norm ? 1 : 0;
  p.out_bf16 = opt->out_dtype == GDN_BF16;
  p.beta_prob = opt->beta_mode == GDN_BETA_PROBABILITY;
  p.idx64 = opt->index_dtype == GDN_I64;
  const int64_t units = static_cast<int64_t>(B) * HV * p.nvb;
  if (units > 0x7fffffffLL) return fail(GDN_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)units);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(units)), block(NW * 64);
  // prefill_ws_kernel: one workgroup per (sequence, pair of value heads,
  // V-block); the units of one key head's pairs stay on one XCD
  gdn::PrefillParams pw = p;
  constexpr int NH = gdn::kWsHeads;
  const int64_t units_ws = static_cast<int64_t>(B) * ((HV + NH - 1) / NH) * p.nvb;
  if (units_ws > 0x7fffffffLL) return fail(GDN_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)units_ws);
  pw.xcd_shift = 0;
  while ((1 << pw.xcd_shift) < std::max(1, p.gqa / NH) * p.nvb && pw.xcd_shift < 6) ++pw.xcd_shift;
  const dim3 grid_ws(static_cast<uint32_t>(units_ws));
  auto go = [&](auto kda_c, auto vf_c, auto io_c) {
    constexpr bool KDA = decltype(kda_c)::value, VF = decltype(vf_c)::value;
    using TIn = typename decltype(io_c)::type;
    // GDN with 16-bit inputs: prefill_ws_kernel (producer and consumer waves,
    // two value heads per workgroup); KDA, whose A' and P are formed pair by
    // pair on the VALU, and 32-bit inputs keep the four-wave kernel
    if constexpr (KDA || sizeof(TIn) != 2)
      hipLaunchKernelGGL((gdn::prefill_kernel<VT, NW, KDA, VF, TIn>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((gdn::prefill_ws_kernel<VF, TIn>), grid_ws, dim3(gdn::kWsHeads * 6 * 64), 0, s, pw);
  };
  using F = std::false_type;
  using Tr = std::true_type;
  using Bf = std::common_type<gdn::bf16_t>;
  using Fl = std::common_type<float>;
  const bool vf = opt->state_layout == GDN_V_FIRST, bf = opt->io_dtype == GDN_BF16;
  if (kda) {
    if (vf) bf ? go(Tr{}, Tr{}, Bf{}) : go(Tr{}, Tr{}, Fl{});
    else bf ? go(Tr{}, F{}, Bf{}) : go(Tr{}, F{}, Fl{});
  } else {
    if (vf) bf ? go(F{}, Tr{}, Bf{}) : go(F{}, Tr{}, Fl{});
    else bf ? go(F{}, F{}, Bf{}) : go(F{}, F{}, Fl{});
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_prefill_paged(const void* q, const void* k, const void* v, const void* a, const void* b, const float* A_log,
                      const float* dt_bias, const int32_t* cu_seqlens, const void* page_indices,
                      const void* page_indptr, const void* last_page_len, int32_t page_size, float* state_pool,
                      void* out, int32_t B, int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V,
                      int64_t num_pages, int64_t nnz, const gdn_options* opt, void* stream) {
  return prefill_call(false, q, k, v, a, b, A_log, dt_bias, cu_seqlens, page_indices, page_indptr, last_page_len,
                      page_size, state_pool, out, B, T, HK, HV, K, V, num_pages, nnz, opt, stream);
}

int kda_prefill_paged(const void* q, const void* k, const void* v, const void* raw_gate, const void* beta_logits,
                      const float* a_log, const float* dt_bias, const int32_t* cu_seqlens, const void* page_indices,
                      const void* page_indptr, const void* last_page_len, int32_t page_size, float* state_pool,
                      void* out, int32_t B, int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V,
                      int64_t num_pages, int64_t nnz, const gdn_options* opt, void* stream) {
  return prefill_call(true, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, page_indices, page_indptr,
                      last_page_len, page_size, state_pool, out, B, T, HK, HV, K, V, num_pages, nnz, opt, stream);
}

int kda_decode_pooled(const void* q, const void* k, const void* v, const void* raw_gate, const void* beta_logits,
                      const float* a_log, const float* dt_bias, const int32_t* cu_seqlens,
                      const int32_t* state_indices, float* state_pool, void* out, int32_t B, int32_t T, int32_t HK,
                      int32_t HV, int32_t K, int32_t V, int64_t num_slots, const gdn_options* opt, void* stream) {
  if (!q || !k || !v || !raw_gate || !beta_logits || !a_log || !dt_bias || !cu_seqlens || !state_indices ||
      !state_pool || !out)
    return fail(GDN_ERR_INVALID, "a required pointer is NULL (cu_seqlens is required for KDA)");
  if (int rc = check_dims(B, HK, HV, K, V)) return rc;
  if (T < 0 || num_slots <= 0) return fail(GDN_ERR_INVALID, "T must be >= 0 and num_slots > 0");
  if (int rc = check_options(opt, K, V, Kind::KdaPooled)) return rc;
  if (opt->slots) return fail(GDN_ERR_INVALID, "slots apply to paged calls only");
  gdn::Params p{};
  p.q = q; p.k = k; p.v = v; p.gate = raw_gate; p.beta = beta_logits;
  p.a_log = a_log; p.dt_bias = dt_bias;
  p.cu_seqlens = cu_seqlens; p.state_indices = state_indices;
  p.pool = state_pool; p.out = out;
  fill_common(p, opt, Kind::KdaPooled, B, T, HK, HV, K, V);
  if (int rc = checked_pooled(cu_seqlens, state_indices, B, T, num_slots, stream)) return rc;
  if (T == 0) { g_last_error.clear(); return GDN_OK; }
  return run(Kind::KdaPooled, p, K, T, opt, stream);
}

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID: return "GDN_ERR_INVALID";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    case GDN_ERR_PRECONDITION: return "GDN_ERR_PRECONDITION";
  }
  return "unknown status";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_check_pooled(const int32_t* cu_seqlens, const int32_t* state_indices, int32_t B, int32_t T,
                     int64_t num_slots) {
  if (!state_indices) return fail(GDN_ERR_INVALID, "state_indices is NULL");
  if (B <= 0 || T < 0 || num_slots <= 0) return fail(GDN_ERR_INVALID, "B and num_slots must be positive, T >= 0");
  std::string msg;
  if (!gdn_host::check_pooled(cu_seqlens, state_indices, B, T, num_slots, msg))
    return fail(GDN_ERR_PRECONDITION, "%s", msg.c_str());
  g_last_error.clear();
  return GDN_OK;
}

int gdn_check_paged(const void* page_indices, const void* page_indptr, const void* last_page_len, int32_t index_dtype,
                    const int64_t* slots, int32_t B, int32_t page_size, int64_t num_pages, int64_t nnz) {
  if (!page_indices || !page_indptr || !last_page_len) return fail(GDN_ERR_INVALID, "a required pointer is NULL");
  if (index_dtype != GDN_I32 && index_dtype != GDN_I64)
    return fail(GDN_ERR_INVALID, "index_dtype must be GDN_I32 or GDN_I64 (got %d)", index_dtype);
  if (B <= 0 || page_size < 0 || num_pages <= 0 || nnz <= 0)
    return fail(GDN_ERR_INVALID, "B, num_pages and nnz must be positive, page_size >= 0");
  std::string msg;
  if (!gdn_host::check_paged(page_indices, page_indptr, last_page_len, index_dtype == GDN_I64, slots, B, page_size,
                             num_pages, nnz, msg))
    return fail(GDN_ERR_PRECONDITION, "%s", msg.c_str());
  g_last_error.clear();
  return GDN_OK;
}

int gdn_check_paged_varlen(const int32_t* cu_seqlens, const void* page_indices, const void* page_indptr,
                           const void* last_page_len, int32_t index_dtype, int32_t B, int32_t T, int32_t page_size,
                           int64_t num_pages, int64_t nnz) {
  if (!cu_seqlens || !page_indices || !page_indptr || !last_page_len)
    return fail(GDN_ERR_INVALID, "a required pointer is NULL");
  if (index_dtype != GDN_I32 && index_dtype != GDN_I64)
    return fail(GDN_ERR_INVALID, "index_dtype must be GDN_I32 or GDN_I64 (got %d)", index_dtype);
  if (B <= 0 || T < 0 || page_size <= 0 || num_pages <= 0 || nnz <= 0)
    return fail(GDN_ERR_INVALID, "B, page_size, num_pages and nnz must be positive, T >= 0");
  std::string msg;
  if (!gdn_host::check_paged_varlen(cu_seqlens, page_indices, page_indptr, last_page_len, index_dtype == GDN_I64, B, T,
                                    page_size, num_pages, nnz, msg))
    return fail(GDN_ERR_PRECONDITION, "%s", msg.c_str());
  g_last_error.clear();
  return GDN_OK;
}

int gdn_checked_build(void) { return kChecked ? 1 : 0; }

int64_t gdn_packed_tile_bytes(int32_t K, int32_t V) {
  if (K <= 0 || V <= 0 || V % 32 != 0) return -1;
  return static_cast<int64_t>(K) * V + 4 * static_cast<int64_t>(K) * (V / 32);
}

int64_t gdn_fp8_tile_bytes(int32_t K, int32_t V, int32_t block_v) {
  if (K <= 0 || V <= 0 || block_v <= 0 || V % block_v != 0) return -1;
  return 128 * ((static_cast<int64_t>(K) * V + 4 * static_cast<int64_t>(V / block_v) + 127) / 128);
}

int gdn_stream_rows(const float* src_pool, float* dst_pool, const int64_t* slots, int32_t n, int64_t row_floats,
                    void* stream) {
  if (!src_pool || !dst_pool || (n > 0 && !slots)) return fail(GDN_ERR_INVALID, "a required pointer is NULL");
  if (n < 0 || row_floats <= 0 || row_floats % 512 != 0)
    return fail(GDN_ERR_INVALID, "n must be >= 0 and row_floats a positive multiple of 512 (n=%d row_floats=%lld)", n,
                (long long)row_floats);
  if (n == 0) {
    g_last_error.clear();
    return GDN_OK;
  }
  const int64_t chunks = row_floats / 512;
  const int64_t units = chunks * n;
  if (units > 0x7fffffffLL) return fail(GDN_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)units);
  hipLaunchKernelGGL(gdn::stream_rows_kernel, dim3(static_cast<uint32_t>(units)), dim3(64), 0,
                     static_cast<hipStream_t>(stream), src_pool, dst_pool, slots, row_floats,
                     static_cast<int32_t>(chunks), 6);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_last_error.clear();
  return GDN_OK;
}

int gdn_workgroup_order(int32_t grid, int32_t xcd_shift, int32_t* units) {
  if (grid < 0 || xcd_shift < 0 || xcd_shift > 16 || (grid > 0 && !units))
    return fail(GDN_ERR_INVALID, "grid must be >= 0, xcd_shift in [0, 16] and units non-NULL");
  for (int32_t bx = 0; bx < grid; ++bx) units[bx] = gdn::xcd_unit(bx, grid, xcd_shift);
  g_last_error.clear();
  return GDN_OK;
}

int gdn_supported_head_dims(int32_t* pairs, int cap) {
  const int n = static_cast<int>(sizeof(kHeads) / sizeof(kHeads[0]));
  for (int i = 0; i < n && i < cap && pairs; ++i) {
    pairs[2 * i] = kHeads[i].K;
    pairs[2 * i + 1] = kHeads[i].VB;
  }
  return n;
}

}  // extern "C"

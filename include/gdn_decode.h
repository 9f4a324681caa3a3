/*
 * gdn_decode.h -- C ABI of the gated delta-rule recurrent decode library
 * (libgdn_decode.so, HIP kernels for gfx950 / MI355X).
 *
 * One call advances, for every sequence b and value head h, an fp32 state
 * S[K, V] over the sequence's suffix tokens and writes one output row per
 * token.  Per token (decay first, then the delta write, then the readout of
 * the updated state -- Circuit.LLM.Mixer, "Delta rule" and "Gated memory"):
 *
 *   q_hat = l2norm(q) * scale        k_hat = l2norm(k)
 *   g     = -exp(A_log) * softplus(a + dt_bias)     (GDN: one per head;
 *                                                    KDA: one per key channel)
 *   beta  = sigmoid(b)  or  b                       (beta_mode)
 *   S    <- exp(g) * S          (KDA: row c of S scaled by exp(g_c))
 *   u     = beta * (v - k_hat^T S)
 *   S    <- S + k_hat u^T
 *   o     = q_hat^T S
 *
 * with l2norm(x) = x / sqrt(sum(x^2) + 1e-6), softplus(x) =
 * max(x,0) + log1p(exp(-|x|)), value head h reading key head h / (HV/HK),
 * and, when enabled, a quantise/dequantise of S after every token: fp8
 * e4m3 with one amax/448 scale per [K, block_v] tile (OCP E4M3,
 * nearest-even, saturating), or the int8_hadamard32 codec (enum gdn_qdq).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device pointers must be device memory (or memory the
 *   device can access) of the HIP runtime loaded in the process; all arrays
 *   are dense and row-major ("contiguous") in the shapes given.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream).  The library allocates nothing, keeps no state between calls,
 *   and is reentrant; the caller owns every buffer.
 * - `state_pool` is read and written in place; only the rows named below
 *   as written are modified, byte for byte nothing else.  `out` is fully
 *   overwritten for every token of a non-empty suffix and must not alias an
 *   input or the pool.  All other arrays are read only.
 * - Return value: GDN_OK, or an error code from host-side checks made
 *   before anything is launched (nothing is written then), or GDN_ERR_HIP
 *   if the launch itself failed.  gdn_status_string() names the code and
 *   gdn_last_error() gives the calling thread's last error message.
 * - Not checked (undefined behaviour if violated; max.nn.state_space.kda_decode,
 *   Raises, and flashinfer.gdn_paged.gated_delta_rule_decode_paged, slots,
 *   leave these unchecked on the device too): index values inside the pool,
 *   distinct state_indices, distinct write pages, a write page that another
 *   sequence of the same call reads, non-decreasing cu_seqlens, and
 *   last_page_len == 1 with fewer than two pages.  The gdn_check_* calls
 *   check them on host copies, and a GDN_DEVICE_CHECKS build checks them in
 *   every call (see gdn_check_pooled below).
 */
#ifndef GDN_DECODE_H
#define GDN_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  The mapping follows max.nn.state_space.kda_decode, Raises:
 * a type combination with no compiled kernel, or tensor extents that do not
 * fit together, are reported on the host before any launch. */
enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID = 1,      /* null required pointer, dimension <= 0, HV % HK != 0, bad enum */
  GDN_ERR_SHAPE = 2,        /* extents disagree (e.g. T != B without cu_seqlens) */
  GDN_ERR_UNSUPPORTED = 3,  /* valid request with no compiled kernel (head dims, block_v, gate_mode,
                               storage and layout, a grid beyond 2^31 - 1 workgroups) */
  GDN_ERR_HIP = 4,          /* the HIP launch reported an error */
  GDN_ERR_PRECONDITION = 5  /* an index precondition does not hold: gdn_check_* calls, and every
                               call of a library built with GDN_DEVICE_CHECKS */
};

/* Element types of the I/O tensors and of the page table. */
enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1, GDN_I32 = 2, GDN_I64 = 3 };

/* Pool axis order of one (row, head) state (max.nn.state_space.kda_decode,
 * state_layout): K_FIRST stores [K][V] (V contiguous), V_FIRST stores
 * [V][K] (K contiguous; the [num_pages, HV, V, K] pool of
 * flashinfer.gdn_paged.gated_delta_rule_decode_paged). */
enum gdn_layout { GDN_K_FIRST = 0, GDN_V_FIRST = 1 };

/* max.nn.state_space.kda_decode, beta_mode: apply the sigmoid or not. */
enum gdn_beta_mode { GDN_BETA_LOGITS = 0, GDN_BETA_PROBABILITY = 1 };

/* max.nn.state_space.kda_decode, gate_mode.  GDN_GATE_SAFE depends on a
 * lower-bound constant the page does not give and returns
 * GDN_ERR_UNSUPPORTED. */
enum gdn_gate_mode { GDN_GATE_ORIGINAL = 0, GDN_GATE_SAFE = 1 };

/* State quantise/dequantise after every token.  On an fp32 pool
 * (GDN_STORAGE_F32) the state written back is the dequantised value; the
 * packed storages (gdn_storage) hold the codes and scales instead.
 *
 * GDN_QDQ_FP8_E4M3_TILE (modelopt ... linear_attention.config,
 * LinearAttentionConfig, state.block_v: each [K, block_v] tile of a
 * sequence's head state gets its own scale, recomputed every time;
 * ... linear_attention.decode: state_format 'fp8_e4m3'): OCP E4M3,
 * scale = amax / 448 per tile, nearest even, saturating.
 *
 * GDN_QDQ_INT8_HADAMARD32 (LinearAttentionDecodeConfig, state_codec
 * 'int8_hadamard32': one scale per key channel and 32 values;
 * LinearAttentionCarry, value_basis / reconstruct: the codec works in a
 * rotated value basis and the state is returned in the original one):
 * every group of 32 consecutive value columns of a key row is rotated by
 * the orthonormal 32-point Walsh-Hadamard matrix H/sqrt(32) (Sylvester
 * order), rounded to int8 codes in [-127, 127] with scale amax/127 of the
 * group (nearest even), dequantised and rotated back.  block_v stays the
 * execution tile width and does not change the result; it must be a
 * multiple of 32.  K = 128 only. */
enum gdn_qdq { GDN_QDQ_NONE = 0, GDN_QDQ_FP8_E4M3_TILE = 1, GDN_QDQ_INT8_HADAMARD32 = 2 };

/* modelopt ... linear_attention.config, LinearAttentionDecodeConfig,
 * readout: 'working' reads o from the updated state before its rounding,
 * 'stored' from the rounded state. */
enum gdn_readout { GDN_READOUT_WORKING = 0, GDN_READOUT_STORED = 1 };

/* How the pool holds the state.  GDN_STORAGE_F32: fp32 states in the
 * state_layout order (every entry point's default).  GDN_STORAGE_I8H32:
 * the int8_hadamard32 codec's own codes -- this library's format; the
 * pages (modelopt ... linear_attention.config, LinearAttentionConfig)
 * describe the codec as a quantise/dequantise emulation with no
 * compressed-storage claim.  Each (row, value head) tile is
 * gdn_packed_tile_bytes(K, V) bytes: K V int8 codes in [V / 32][K][32]
 * order (one 32-value group of every key row after another), then
 * K V / 32 float32 scales in [V / 32][K] order; codes c[g][k][0..31] and
 * scale s[g][k] stand for the state row S[k][32 g .. 32 g + 31] =
 * (c[g][k] H) * s[g][k] / 32 (H the +-1 Sylvester Hadamard matrix of
 * order 32), so s is amax/127 of the group in the +-1 Hadamard basis.
 * state_pool then points to rows * HV such tiles (4-byte aligned) and is
 * read and written as such.  Requires qdq = GDN_QDQ_INT8_HADAMARD32 (else
 * GDN_ERR_INVALID) and state_layout = GDN_K_FIRST (else
 * GDN_ERR_UNSUPPORTED); results equal those of GDN_STORAGE_F32 with the
 * codec up to float32 rounding, with about 3.6x fewer pool bytes at
 * K = V = 128. */
/* GDN_STORAGE_FP8_TILE: the fp8 tile QDQ's own codes, again this library's
 * format (modelopt ... linear_attention.decode, EncodedLinearAttentionTensor,
 * holds dequantised values beside their scales and claims no compressed
 * storage).  Each (row, value head) tile is
 * gdn_fp8_tile_bytes(K, V, block_v) bytes: the K V OCP E4M3 bytes in the
 * pool's state_layout order (K_FIRST [K][V], V_FIRST [V][K]), then the
 * V / block_v float32 tile scales amax/448 (scale 0 for an all-zero tile),
 * the tile zero-padded to whole 128-byte lines (so that no two tiles share
 * a cache line); element x = e4m3(byte) * scale of
 * its [K, block_v] tile.  Requires qdq = GDN_QDQ_FP8_E4M3_TILE (else
 * GDN_ERR_INVALID); results equal those of GDN_STORAGE_F32 with the fp8
 * tiles up to float32 rounding, with about 4x fewer pool bytes. */
enum gdn_storage { GDN_STORAGE_F32 = 0, GDN_STORAGE_I8H32 = 1, GDN_STORAGE_FP8_TILE = 2 };

/* Options of a call.  Fill with gdn_options_init() and change fields. */
typedef struct gdn_options {
  float scale;              /* query scale; 0 means 1/sqrt(K)                     (default 0) */
  int32_t use_qk_l2norm;    /* 1: L2-normalise q and k inside the call              (default 1) */
  int32_t io_dtype;         /* q, k, v, a, b, raw_gate, beta_logits: F32 or BF16  (default BF16) */
  int32_t out_dtype;        /* out: F32 or BF16                                    (default BF16) */
  int32_t state_layout;     /* gdn_layout                                   (default K_FIRST) */
  int32_t beta_mode;        /* gdn_beta_mode                                 (default LOGITS) */
  int32_t gate_mode;        /* gdn_gate_mode                               (default ORIGINAL) */
  int32_t index_dtype;      /* paged table: I32 or I64                           (default I32) */
  int32_t qdq;              /* gdn_qdq                                           (default NONE) */
  int32_t block_v;          /* QDQ tile width over V; must divide V           (default 64) */
  int32_t quantize_initial; /* 1: also round the state read before the first token (default 0) */
  int32_t readout;          /* gdn_readout                                     (default WORKING) */
  const int64_t* slots;     /* single-token paged calls only: device [B][2] (read row, write row)
                               that gdn_paged_decode_slots() produced from this call's table, or
                               NULL to resolve the rows inside the call (default NULL).  Not
                               checked against the table (flashinfer.gdn_paged, slots). */
  int32_t state_storage;    /* gdn_storage                                      (default F32) */
} gdn_options;

/* Fill `opt` with the defaults listed above.  `opt` must not be NULL. */
void gdn_options_init(gdn_options* opt);

/*
 * gdn_decode_pooled -- GDN decode (one gate per value head) on a slot pool,
 * varlen suffixes.  flashinfer.gdn_paged.gated_delta_rule_decode_paged,
 * parameters q..b and scale/use_qk_l2norm (inherited from the pooled
 * decode), generalised to several tokens per sequence the way
 * max.nn.state_space.kda_decode, cu_seqlens, does.
 *
 *   q, k          [T, HK, K]   io_dtype   device
 *   v             [T, HV, V]   io_dtype   device
 *   a, b          [T, HV]      io_dtype   device
 *   A_log, dt_bias[HV]         f32        device
 *   cu_seqlens    [B+1]        i32        device; exclusive prefix offsets of
 *                                         the suffixes in the token axis, or
 *                                         NULL for exactly one token per
 *                                         sequence (then T must equal B)
 *   state_indices [B]          i32        device; pool slot of each sequence
 *   state_pool    [num_slots, HV, K, V] (K_FIRST) or [num_slots, HV, V, K]
 *                 (V_FIRST)    f32        device; slot state_indices[b] is
 *                                         read and written in place if the
 *                                         suffix of b is non-empty; an empty
 *                                         suffix reads and writes nothing
 *   out           [T, HV, V]   out_dtype  device
 */
int gdn_decode_pooled(const void* q, const void* k, const void* v, const void* a, const void* b,
                      const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                      const int32_t* state_indices, float* state_pool, void* out, int32_t B,
                      int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V, int64_t num_slots,
                      const gdn_options* opt, void* stream);

/*
 * gdn_decode_paged -- GDN decode of one token per sequence on a CSR-paged pool
 * (flashinfer.gdn_paged.gated_delta_rule_decode_paged).  Token b ends
 * sequence b and occupies slot last_page_len[b] of its final page,
 * page_indices[page_indptr[b+1]-1].  With last_page_len[b] == 1 the token
 * starts that page: the starting state comes from the page before it,
 * page_indices[page_indptr[b+1]-2], the result goes to the final page, and
 * the page before (possibly shared with other sequences) keeps every byte.
 * In any other slot the final page is read and rewritten in place.
 *
 *   q, k          [B, HK, K]   io_dtype   device
 *   v             [B, HV, V]   io_dtype   device
 *   a, b          [B, HV]      io_dtype   device
 *   A_log, dt_bias[HV]         f32        device
 *   page_indices  [nnz]        index_dtype device
 *   page_indptr   [B+1]        index_dtype device
 *   last_page_len [B]          index_dtype device, values in [1, page_size]
 *   state_pool    [num_pages, HV, V, K] (V_FIRST) or [num_pages, HV, K, V]
 *                 (K_FIRST)    f32        device, updated in place
 *   out           [B, HV, V]   out_dtype  device (the [B, 1, HV, V] output)
 */
int gdn_decode_paged(const void* q, const void* k, const void* v, const void* a, const void* b,
                     const float* A_log, const float* dt_bias, const void* page_indices,
                     const void* page_indptr, const void* last_page_len, float* state_pool,
                     void* out, int32_t B, int32_t HK, int32_t HV, int32_t K, int32_t V,
                     int64_t num_pages, int64_t nnz, const gdn_options* opt, void* stream);

/*
 * kda_decode_pooled -- KDA decode (one gate per value head and key channel)
 * on a slot pool, varlen suffixes (max.nn.state_space.kda_decode).
 *
 *   q, k          [T, HK, K]   io_dtype   device
 *   v             [T, HV, V]   io_dtype   device
 *   raw_gate      [T, HV, K]   io_dtype   device; gate input, dt_bias not yet added
 *   beta_logits   [T, HV]      io_dtype   device
 *   a_log         [HV]         f32        device
 *   dt_bias       [HV, K]      f32        device
 *   cu_seqlens    [B+1]        i32        device, required
 *   state_indices [B]          i32        device
 *   state_pool    as for gdn_decode_pooled
 *   out           [T, HV, V]   out_dtype  device
 */
int kda_decode_pooled(const void* q, const void* k, const void* v, const void* raw_gate,
                      const void* beta_logits, const float* a_log, const float* dt_bias,
                      const int32_t* cu_seqlens, const int32_t* state_indices, float* state_pool,
                      void* out, int32_t B, int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V,
                      int64_t num_slots, const gdn_options* opt, void* stream);

/*
 * kda_decode_paged -- single-token KDA decode on a CSR-paged pool: the paging
 * of gdn_decode_paged (flashinfer.gdn_paged.gated_delta_rule_decode_paged)
 * with the per-key-channel gate and the inputs of kda_decode_pooled
 * (max.nn.state_space.kda_decode).  q, k [B, HK, K]; v [B, HV, V];
 * raw_gate [B, HV, K]; beta_logits [B, HV]; a_log [HV]; dt_bias [HV, K];
 * table, pool and out as for gdn_decode_paged.
 */
int kda_decode_paged(const void* q, const void* k, const void* v, const void* raw_gate,
                     const void* beta_logits, const float* a_log, const float* dt_bias,
                     const void* page_indices, const void* page_indptr, const void* last_page_len,
                     float* state_pool, void* out, int32_t B, int32_t HK, int32_t HV, int32_t K,
                     int32_t V, int64_t num_pages, int64_t nnz, const gdn_options* opt, void* stream);

/*
 * gdn_decode_paged_varlen / kda_decode_paged_varlen -- several decoded tokens
 * per sequence on a CSR-paged pool (the single-token rule of
 * flashinfer.gdn_paged.gated_delta_rule_decode_paged, applied token by
 * token).  cu_seqlens [B+1] (i32, device) gives each sequence's suffix in
 * the token axis, as in max.nn.state_space.kda_decode.  The page table
 * describes the sequences after the suffix: sequence b holds
 * n_b = (pages_b - 1) * page_size + last_page_len[b] tokens and the suffix is
 * its last T_b tokens; the suffix never starts at token 1.  The starting
 * state comes from the page holding token n_b - T_b; a suffix token at a
 * position that is a multiple of page_size completes its page and stores its
 * state there; the state after the last token goes to the final page.  Pages that hold no
 * suffix token are never written; pages a suffix writes must belong to that
 * sequence alone (not checked).  q, k [T, HK, K], v [T, HV, V], out
 * [T, HV, V]; other inputs as for the single-token calls with T rows.
 * opt->slots must be NULL.
 */
int gdn_decode_paged_varlen(const void* q, const void* k, const void* v, const void* a, const void* b,
                            const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                            const void* page_indices, const void* page_indptr,
                            const void* last_page_len, int32_t page_size, float* state_pool,
                            void* out, int32_t B, int32_t T, int32_t HK, int32_t HV, int32_t K,
                            int32_t V, int64_t num_pages, int64_t nnz, const gdn_options* opt,
                            void* stream);
int kda_decode_paged_varlen(const void* q, const void* k, const void* v, const void* raw_gate,
                            const void* beta_logits, const float* a_log, const float* dt_bias,
                            const int32_t* cu_seqlens, const void* page_indices,
                            const void* page_indptr, const void* last_page_len, int32_t page_size,
                            float* state_pool, void* out, int32_t B, int32_t T, int32_t HK,
                            int32_t HV, int32_t K, int32_t V, int64_t num_pages, int64_t nnz,
                            const gdn_options* opt, void* stream);

/*
 * gdn_prefill_paged -- chunked GDN prefill on a CSR-paged pool: the same
 * arguments and the same result as gdn_decode_paged_varlen (flashinfer names
 * the paged chunked prefill chunk_gated_delta_rule_paged; the chunked form
 * follows the step names of modelopt ... linear_attention.config,
 * LinearAttentionConfig, with the exact solve of LinearAttentionSolveConfig,
 * and Circuit.LLM.Mixer, "Chunked additive linear": chunked equals
 * sequential).  The suffix is processed in chunks of 16 tokens aligned to
 * absolute positions, each as dense products on the matrix cores, so long
 * suffixes (prompts) run chunk-parallel instead of token by token; results
 * agree with the token-by-token call to float32 rounding, not bit for bit.
 * Requirements (else GDN_ERR_UNSUPPORTED): K = 128, V a multiple of 128,
 * page_size a multiple of 16, opt->qdq == GDN_QDQ_NONE.  opt->slots must be
 * NULL.  The chunk's identity padding (positions of a chunk outside the
 * suffix) reads and writes nothing.  kda_prefill_paged is the same for the
 * per-key-channel gate, with kda_decode_paged_varlen's arguments (raw_gate
 * [T, HV, K], beta_logits [T, HV], a_log [HV], dt_bias [HV, K]).
 */
int gdn_prefill_paged(const void* q, const void* k, const void* v, const void* a, const void* b,
                      const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                      const void* page_indices, const void* page_indptr, const void* last_page_len,
                      int32_t page_size, float* state_pool, void* out, int32_t B, int32_t T, int32_t HK,
                      int32_t HV, int32_t K, int32_t V, int64_t num_pages, int64_t nnz,
                      const gdn_options* opt, void* stream);
int kda_prefill_paged(const void* q, const void* k, const void* v, const void* raw_gate,
                      const void* beta_logits, const float* a_log, const float* dt_bias,
                      const int32_t* cu_seqlens, const void* page_indices, const void* page_indptr,
                      const void* last_page_len, int32_t page_size, float* state_pool, void* out,
                      int32_t B, int32_t T, int32_t HK, int32_t HV, int32_t K, int32_t V,
                      int64_t num_pages, int64_t nnz, const gdn_options* opt, void* stream);

/*
 * gdn_paged_decode_slots -- the (read row, write row) pair of every sequence
 * for a single-token paged decode step, written to slots [B][2] (int64,
 * device).  Computed once per step and passed to every layer's call through
 * gdn_options.slots (flashinfer.gdn_paged.gated_delta_rule_decode_paged,
 * slots).  page_indices / page_indptr / last_page_len as for gdn_decode_paged,
 * of type index_dtype (GDN_I32 or GDN_I64).  Asynchronous on stream.
 */
int gdn_paged_decode_slots(const void* page_indices, const void* page_indptr,
                           const void* last_page_len, int32_t B, int32_t index_dtype,
                           int64_t* slots, void* stream);

/* Static name of a status code ("GDN_OK", ...); "unknown status" otherwise. */
const char* gdn_status_string(int status);

/* Message of the calling thread's last failed call ("" if none).  The
 * pointer stays valid until the thread's next call into the library. */
const char* gdn_last_error(void);

/*
 * Host-side checks of the index preconditions the kernels do not check (the
 * "Not checked" list above; flashinfer.gdn_paged,
 * gated_delta_rule_decode_paged, slots, and max.nn.state_space.kda_decode,
 * Raises, leave them to debug builds).  Every pointer here is HOST memory
 * holding a copy of the arrays a call would receive; nothing touches the
 * GPU.  Returns GDN_OK, GDN_ERR_PRECONDITION with gdn_last_error() naming
 * the first violation and the sequence, or GDN_ERR_INVALID for a NULL
 * pointer or a non-positive size.
 *
 * gdn_check_pooled: cu_seqlens (NULL: T == B) has cu[0] == 0, never
 *   decreases and ends at T; the slot of every non-empty suffix is in
 *   [0, num_slots) and no two non-empty suffixes share one.
 * gdn_check_paged (single-token calls): page_indptr[0] >= 0, every sequence
 *   has a page, page_indptr[B] <= nnz, last_page_len in [1, page_size]
 *   (page_size 0: >= 1), a sequence with last_page_len == 1 has a previous
 *   page, read and write pages are in [0, num_pages), no two sequences write
 *   one page, no sequence writes a page another reads, and `slots` (NULL or
 *   [B][2] int64) equals the (read, write) rows of the table.
 * gdn_check_paged_varlen (paged varlen decode and prefill calls): the table
 *   and cu_seqlens as above, last_page_len <= page_size, a token before
 *   every non-empty suffix, the page read and every page written in range,
 *   and no page written by one sequence is read or written by another.
 *
 * A library compiled with GDN_DEVICE_CHECKS (libgdn_decode_checked.so) runs
 * the same checks in every entry point on host copies of its index arrays
 * (synchronising `stream` first) and returns GDN_ERR_PRECONDITION without
 * launching anything when one fails; gdn_paged_decode_slots, which has no
 * nnz or num_pages, checks the table's structure only.  gdn_checked_build()
 * returns 1 in such a build and 0 otherwise.
 */
int gdn_check_pooled(const int32_t* cu_seqlens, const int32_t* state_indices, int32_t B, int32_t T,
                     int64_t num_slots);
int gdn_check_paged(const void* page_indices, const void* page_indptr, const void* last_page_len,
                    int32_t index_dtype, const int64_t* slots, int32_t B, int32_t page_size,
                    int64_t num_pages, int64_t nnz);
int gdn_check_paged_varlen(const int32_t* cu_seqlens, const void* page_indices,
                           const void* page_indptr, const void* last_page_len, int32_t index_dtype,
                           int32_t B, int32_t T, int32_t page_size, int64_t num_pages, int64_t nnz);
int gdn_checked_build(void);

/* Bytes of one packed (row, value head) tile of a GDN_STORAGE_I8H32 pool:
 * K V + 4 K (V / 32); -1 if V is not a positive multiple of 32 or K <= 0. */
int64_t gdn_packed_tile_bytes(int32_t K, int32_t V);

/* Bytes of one (row, value head) tile of a GDN_STORAGE_FP8_TILE pool:
 * K V + 4 (V / block_v) rounded up to a multiple of 128; -1 if block_v does
 * not divide V or a size is not positive. */
int64_t gdn_fp8_tile_bytes(int32_t K, int32_t V, int32_t block_v);

/* Head dims with a compiled kernel: writes up to `cap` (K, VB) pairs as
 * 2*n ints into `pairs` (NULL allowed) and returns the number of pairs
 * available.  A key head dim K is supported with any value head dim V that
 * is a multiple of its VB; fp8 tile QDQ needs block_v == VB; the
 * int8_hadamard32 codec needs VB >= 32. */
int gdn_supported_head_dims(int32_t* pairs, int cap);

/*
 * Measurement and launch-order helpers (not operations of the pages).
 *
 * gdn_stream_rows -- the state traffic of a single-token step with no
 * arithmetic: for each of the n pairs slots[i] = (read row, write row)
 * (int64, device, as gdn_paged_decode_slots writes them; a pooled call's
 * pair is (slot, slot)), copy row_floats consecutive floats from src_pool +
 * read row * row_floats to dst_pool + write row * row_floats, 2 KiB per
 * workgroup with non-temporal 128-bit loads and stores, workgroups ordered
 * on the XCDs as the decode kernels order theirs.  src_pool and dst_pool
 * may be the same pool (the decode's in-place read-modify-write); no read
 * row may be another pair's write row.  A reference for the bandwidth a
 * decode step's state stream reaches: the fastest of the plain stream
 * shapes measured for that row pattern.  row_floats must be a positive
 * multiple of 512 and n >= 0 (else GDN_ERR_INVALID); asynchronous on
 * stream.
 */
int gdn_stream_rows(const float* src_pool, float* dst_pool, const int64_t* slots, int32_t n,
                    int64_t row_floats, void* stream);

/*
 * gdn_workgroup_order -- host only: units[bx] = the work unit that workgroup
 * bx of a grid of `grid` workgroups runs when the kernels keep runs of
 * 2^xcd_shift consecutive units on one XCD (the same function the kernels
 * call).  grid >= 0 and 0 <= xcd_shift <= 16, else GDN_ERR_INVALID.
 */
int gdn_workgroup_order(int32_t grid, int32_t xcd_shift, int32_t* units);

#ifdef __cplusplus
}
#endif

#endif /* GDN_DECODE_H */

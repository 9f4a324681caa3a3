// Host-side validation of the index preconditions of a decode call.
//
// The pages leave these unchecked on the device (flashinfer.gdn_paged,
// gated_delta_rule_decode_paged, slots: rows are not checked against the
// table; max.nn.state_space.kda_decode, Raises: device guards are debug
// assertions only).  Here they are plain C++ over host copies of the index
// arrays, used by the exported gdn_check_* calls and, in builds compiled
// with GDN_DEVICE_CHECKS, by every entry point before it launches anything.
//
// What is checked (every function returns true, or false with `msg` naming
// the first violation found):
//   cu_seqlens     cu[0] == 0, non-decreasing, cu[B] == T
//   pooled         the slot of every non-empty suffix is in [0, rows) and no
//                  two non-empty suffixes share a slot
//   page table     page_indptr[0] >= 0, at least one page per sequence,
//                  page_indptr[B] <= nnz, last_page_len in [1, page_size]
//                  (>= 1 when page_size is 0, i.e. unknown)
//   one token      last_page_len == 1 needs a previous page; the read and
//                  write pages are in [0, rows); write pages are distinct;
//                  no sequence writes a page another sequence reads; given
//                  slots equal the table's (read, write) pairs
//   suffixes       at least one token precedes every non-empty suffix; the
//                  page read and every page written are in [0, rows); a
//                  page written by one sequence is neither read nor written
//                  by another
#pragma once

#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>
#include <unordered_map>

namespace gdn_host {

inline int64_t index_at(const void* p, int64_t i, bool i64) {
  return i64 ? static_cast<const int64_t*>(p)[i] : static_cast<const int32_t*>(p)[i];
}

__attribute__((format(printf, 2, 3))) inline bool violation(std::string& msg, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  msg = buf;
  return false;
}

// Suffix length of sequence b (one token each without cu_seqlens).
inline int64_t suffix_len(const int32_t* cu, int64_t b) { return cu ? int64_t(cu[b + 1]) - cu[b] : 1; }

inline bool check_cu(const int32_t* cu, int32_t B, int32_t T, std::string& msg) {
  if (!cu) {
    if (T != B) return violation(msg, "without cu_seqlens T (%d) must equal B (%d)", T, B);
    return true;
  }
  if (cu[0] != 0) return violation(msg, "cu_seqlens[0] is %d, not 0", cu[0]);
  for (int32_t b = 0; b < B; ++b)
    if (cu[b + 1] < cu[b]) return violation(msg, "cu_seqlens decreases at sequence %d (%d -> %d)", b, cu[b], cu[b + 1]);
  if (cu[B] != T) return violation(msg, "cu_seqlens[B] is %d, not T = %d", cu[B], T);
  return true;
}

inline bool check_pooled(const int32_t* cu, const int32_t* slots, int32_t B, int32_t T, int64_t rows,
                         std::string& msg) {
  if (!check_cu(cu, B, T, msg)) return false;
  std::unordered_map<int64_t, int32_t> owner;
  for (int32_t b = 0; b < B; ++b) {
    if (suffix_len(cu, b) == 0) continue;            // an empty suffix touches no slot
    const int64_t r = slots[b];
    if (r < 0 || r >= rows) return violation(msg, "state_indices[%d] = %lld is outside [0, %lld)", b, (long long)r,
                                             (long long)rows);
    const auto it = owner.emplace(r, b);
    if (!it.second) return violation(msg, "sequences %d and %d share slot %lld", it.first->second, b, (long long)r);
  }
  return true;
}

inline bool check_table(const void* ptr, const void* lpl, bool i64, int32_t B, int32_t page_size, int64_t nnz,
                        std::string& msg) {
  if (index_at(ptr, 0, i64) < 0) return violation(msg, "page_indptr[0] is negative");
  for (int32_t b = 0; b < B; ++b) {
    const int64_t s = index_at(ptr, b, i64), e = index_at(ptr, b + 1, i64);
    if (e <= s) return violation(msg, "sequence %d has no page (page_indptr %lld -> %lld)", b, (long long)s,
                                 (long long)e);
    const int64_t l = index_at(lpl, b, i64);
    if (l < 1) return violation(msg, "last_page_len[%d] = %lld is below 1", b, (long long)l);
    if (page_size > 0 && l > page_size)
      return violation(msg, "last_page_len[%d] = %lld exceeds page_size %d", b, (long long)l, page_size);
  }
  if (nnz >= 0 && index_at(ptr, B, i64) > nnz)
    return violation(msg, "page_indptr[B] = %lld exceeds nnz = %lld", (long long)index_at(ptr, B, i64), (long long)nnz);
  return true;
}

inline bool page_in_range(int64_t row, int64_t rows, int32_t b, const char* what, std::string& msg) {
  if (row < 0 || row >= rows)
    return violation(msg, "sequence %d: %s page %lld is outside [0, %lld)", b, what, (long long)row, (long long)rows);
  return true;
}

// One decoded token per sequence: (read, write) pairs from the table, or
// the caller's slots checked against them.
inline bool check_paged(const void* pi, const void* ptr, const void* lpl, bool i64, const int64_t* slots, int32_t B,
                        int32_t page_size, int64_t rows, int64_t nnz, std::string& msg) {
  if (!check_table(ptr, lpl, i64, B, page_size, nnz, msg)) return false;
  std::unordered_map<int64_t, int32_t> writer, reader;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t s = index_at(ptr, b, i64), e = index_at(ptr, b + 1, i64);
    const int64_t l = index_at(lpl, b, i64);
    if (l == 1 && e - s < 2) return violation(msg, "sequence %d opens a new page but has no previous page", b);
    const int64_t w = index_at(pi, e - 1, i64);
    const int64_t r = l == 1 ? index_at(pi, e - 2, i64) : w;
    if (!page_in_range(r, rows, b, "read", msg) || !page_in_range(w, rows, b, "write", msg)) return false;
    if (slots && (slots[2 * b] != r || slots[2 * b + 1] != w))
      return violation(msg, "slots of sequence %d are (%lld, %lld), the table gives (%lld, %lld)", b,
                       (long long)slots[2 * b], (long long)slots[2 * b + 1], (long long)r, (long long)w);
    const auto it = writer.emplace(w, b);
    if (!it.second) return violation(msg, "sequences %d and %d write page %lld", it.first->second, b, (long long)w);
    if (r != w) reader.emplace(r, b);
  }
  for (const auto& rw : reader) {
    const auto it = writer.find(rw.first);
    if (it != writer.end() && it->second != rw.second)
      return violation(msg, "sequence %d writes page %lld, which sequence %d reads", it->second, (long long)rw.first,
                       rw.second);
  }
  return true;
}

// Suffixes of several tokens: the page holding the token before the suffix
// is read, every page a suffix token fills and the last page are written.
inline bool check_paged_varlen(const int32_t* cu, const void* pi, const void* ptr, const void* lpl, bool i64, int32_t B,
                               int32_t T, int32_t page_size, int64_t rows, int64_t nnz, std::string& msg) {
  if (!cu) return violation(msg, "cu_seqlens is required");
  if (page_size <= 0) return violation(msg, "page_size must be positive");
  if (!check_cu(cu, B, T, msg) || !check_table(ptr, lpl, i64, B, page_size, nnz, msg)) return false;
  std::unordered_map<int64_t, int32_t> writer;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = suffix_len(cu, b);
    if (n == 0) continue;
    const int64_t s = index_at(ptr, b, i64), e = index_at(ptr, b + 1, i64);
    const int64_t pos_last = (e - s - 1) * page_size + index_at(lpl, b, i64);
    const int64_t pos0 = pos_last - n + 1;
    if (pos0 < 2)
      return violation(msg, "sequence %d: its %lld suffix tokens leave no earlier token in its %lld", b, (long long)n,
                       (long long)pos_last);
    for (int64_t pos = pos0; pos <= pos_last; ++pos) {
      if (pos % page_size != 0 && pos != pos_last) continue;
      const int64_t w = index_at(pi, s + (pos - 1) / page_size, i64);
      if (!page_in_range(w, rows, b, "written", msg)) return false;
      const auto it = writer.emplace(w, b);
      if (!it.second && it.first->second != b)
        return violation(msg, "sequences %d and %d write page %lld", it.first->second, b, (long long)w);
    }
  }
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = suffix_len(cu, b);
    if (n == 0) continue;
    const int64_t s = index_at(ptr, b, i64), e = index_at(ptr, b + 1, i64);
    const int64_t pos0 = (e - s - 1) * page_size + index_at(lpl, b, i64) - n + 1;
    const int64_t r = index_at(pi, s + (pos0 - 2) / page_size, i64);
    if (!page_in_range(r, rows, b, "read", msg)) return false;
    const auto it = writer.find(r);
    if (it != writer.end() && it->second != b)
      return violation(msg, "sequence %d writes page %lld, which sequence %d reads", it->second, (long long)r, b);
  }
  return true;
}

}  // namespace gdn_host

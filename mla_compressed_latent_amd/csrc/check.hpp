// Checks of the arguments that live in device memory -- sequence offsets,
// lengths and page ids -- for one sequence of an append, decode or extend
// call.  The same functions run on the GPU (check.hip, in the checking build
// of the library) and on the host (a CPU test compiles them for the host
// under the address and undefined-behaviour sanitizers).
//
// Each function reads only the entries the call itself would read for
// sequence b, and reads a page-table entry only after showing that its index
// lies inside row b of the table, so it is safe on any values.  It returns 0
// when the sequence is valid, else a CheckCode; *detail receives the bad
// value or page index.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MLA_CHECK_FN __host__ __device__ inline
#else
#define MLA_CHECK_FN inline
#endif

namespace mla_check {

enum CheckCode : uint32_t {
  kOk = 0,
  kBadOffsets = 1,    // cu[b], cu[b+1] not nondecreasing inside [0, total], or cu[0] != 0, cu[batch] != total
  kBadQueryLen = 2,   // decode/extend: query count outside [1, max_q_len]
  kBadSeqLen = 3,     // decode/extend: seq_len outside [q_len, max_seq_len]
  kBadPrefix = 4,     // append: prefix < 0, or prefix + new tokens beyond the page-table row
  kBadPage = 5,       // a page the sequence touches has an id outside [0, num_pages)
};

// Word that orders failures by sequence: the minimum over all sequences of
// encode(b, code) names the first failing sequence; kNone means none failed.
constexpr uint32_t kNone = 0xFFFFFFFFu;
MLA_CHECK_FN uint32_t encode(int b, uint32_t code) { return ((uint32_t)b << 4) | code; }
MLA_CHECK_FN int failed_sequence(uint32_t word) { return (int)(word >> 4); }
MLA_CHECK_FN uint32_t failed_code(uint32_t word) { return word & 15u; }

MLA_CHECK_FN uint32_t check_offsets(int b, const int32_t* cu, int batch, int total, int32_t* detail) {
  const int32_t lo = cu[b], hi = cu[b + 1];
  if (lo < 0 || hi < lo || hi > total || (b == 0 && lo != 0) || (b == batch - 1 && hi != total)) {
    *detail = lo < 0 || (b == 0 && lo != 0) ? lo : hi;
    return kBadOffsets;
  }
  return kOk;
}

// Pages [first, last] of row b of the table must hold ids in [0, num_pages).
MLA_CHECK_FN uint32_t check_pages(int b, const int32_t* page_table, int max_pages, int64_t first, int64_t last,
                                  int64_t num_pages, int32_t* detail) {
  for (int64_t p = first; p <= last; ++p) {
    const int32_t id = page_table[(int64_t)b * max_pages + p];
    if (id < 0 || (int64_t)id >= num_pages) {
      *detail = (int32_t)p;
      return kBadPage;
    }
  }
  return kOk;
}

// Decode and extend: queries cu_q[b] .. cu_q[b+1]-1 at the last positions of
// seq_lens[b] cached tokens, which occupy pages 0 .. ceil(seq_len/page_size)-1
// (a length needing more pages than the table row holds fails as a length).
MLA_CHECK_FN uint32_t check_decode_sequence(int b, const int32_t* cu_q, const int32_t* seq_lens,
                                            const int32_t* page_table, int max_pages, int batch, int total_q,
                                            int max_q_len, int max_seq_len, int page_size, int64_t num_pages,
                                            int32_t* detail) {
  uint32_t code = check_offsets(b, cu_q, batch, total_q, detail);
  if (code) return code;
  const int q_len = cu_q[b + 1] - cu_q[b];
  if (q_len < 1 || q_len > max_q_len) {
    *detail = q_len;
    return kBadQueryLen;
  }
  const int32_t len = seq_lens[b];
  const int64_t pages = ((int64_t)len + page_size - 1) / page_size;
  if (len < q_len || len > max_seq_len || pages > max_pages) {
    *detail = len;
    return kBadSeqLen;
  }
  return check_pages(b, page_table, max_pages, 0, pages - 1, num_pages, detail);
}

// Append: new tokens cu_new[b] .. cu_new[b+1]-1 go to positions prefix_lens[b]
// onwards; only the pages those positions fall in are touched.
MLA_CHECK_FN uint32_t check_append_sequence(int b, const int32_t* cu_new, const int32_t* prefix_lens,
                                            const int32_t* page_table, int max_pages, int batch, int total_new,
                                            int page_size, int64_t num_pages, int32_t* detail) {
  uint32_t code = check_offsets(b, cu_new, batch, total_new, detail);
  if (code) return code;
  const int n = cu_new[b + 1] - cu_new[b];
  const int64_t prefix = prefix_lens[b];
  if (prefix < 0 || prefix + n > (int64_t)max_pages * page_size) {
    *detail = (int32_t)prefix;
    return kBadPrefix;
  }
  if (n == 0) return kOk;
  return check_pages(b, page_table, max_pages, prefix / page_size, (prefix + n - 1) / page_size, num_pages,
                     detail);
}

}  // namespace mla_check

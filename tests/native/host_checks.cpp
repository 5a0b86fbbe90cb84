// Host-side tests of the library's C++ code, built with the address and
// undefined-behaviour sanitizers (tests/test_host_sanitized.py builds and
// runs this program; no GPU is used):
//   * the checks of device-resident arguments (check.hpp) on valid inputs
//     and on every kind of bad offset, length and page id;
//   * the page pool and the capacity planner (pool.cpp) through the C ABI;
//   * the host validation of the C ABI's GPU calls (api.hip), on a layer
//     handle made here with stand-in device pointers: every call below must
//     be refused by a host check before anything would be enqueued.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/mla.h"
#include "../../mla_compressed_latent_amd/csrc/check.hpp"
#include "../../mla_compressed_latent_amd/csrc/layer.hpp"

static int g_cases = 0, g_failed = 0;

#define EXPECT(cond)                                                          \
  do {                                                                        \
    ++g_cases;                                                                \
    if (!(cond)) {                                                            \
      ++g_failed;                                                             \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, \
              #cond);                                                         \
    }                                                                         \
  } while (0)

using namespace mla_check;

// ---------------------------------------------------------------------------
// check.hpp

namespace {

struct DecodeArgs {
  std::vector<int32_t> cu_q{0, 1, 3, 4};
  std::vector<int32_t> seq_lens{5, 130, 64};
  int max_pages = 3, batch = 3, total_q = 4, max_q_len = 2, max_seq_len = 130, page_size = 64;
  int64_t num_pages = 10;
  // row b: the pages of sequence b; entries past a sequence's last page are
  // never read (left as garbage on purpose)
  std::vector<int32_t> table{7, -5, 1234, 2, 3, 9, 0, -1, -1};

  uint32_t check(int b, int32_t* detail) const {
    return check_decode_sequence(b, cu_q.data(), seq_lens.data(), table.data(), max_pages, batch, total_q,
                                 max_q_len, max_seq_len, page_size, num_pages, detail);
  }
  uint32_t first(int32_t* detail) const {
    uint32_t w = kNone;
    for (int b = 0; b < batch; ++b) {
      int32_t d = 0;
      const uint32_t c = check(b, &d);
      if (c != kOk && encode(b, c) < w) {
        w = encode(b, c);
        *detail = d;
      }
    }
    return w;
  }
};

void test_decode_checks() {
  int32_t d = 0;
  {
    DecodeArgs a;
    EXPECT(a.first(&d) == kNone);
  }
  {  // a page the sequence reads holds -1
    DecodeArgs a;
    a.table[3 + 2] = -1;
    EXPECT(a.check(1, &d) == kBadPage && d == 2);
    EXPECT(a.first(&d) == encode(1, kBadPage) && d == 2);
  }
  {  // a page id equal to num_pages
    DecodeArgs a;
    a.table[6] = 10;
    EXPECT(a.check(2, &d) == kBadPage && d == 0);
  }
  {  // the last page that 64 tokens use is page 0: page 1 of row 2 is not read
    DecodeArgs a;
    a.table[7] = 1 << 30;
    EXPECT(a.first(&d) == kNone);
    a.seq_lens[2] = 65;  // now it is
    EXPECT(a.check(2, &d) == kBadPage && d == 1);
  }
  {  // length beyond max_seq_len, and shorter than the query count
    DecodeArgs a;
    a.seq_lens[0] = 131;
    EXPECT(a.check(0, &d) == kBadSeqLen && d == 131);
    a.seq_lens[0] = 5;
    a.seq_lens[1] = 1;
    EXPECT(a.check(1, &d) == kBadSeqLen && d == 1);
  }
  {  // a length that needs more pages than the table row holds, even if
     // max_seq_len claims otherwise
    DecodeArgs a;
    a.max_seq_len = 300;
    a.seq_lens[0] = 193;
    EXPECT(a.check(0, &d) == kBadSeqLen && d == 193);
  }
  {  // offsets: not starting at 0, decreasing, not ending at total_q
    DecodeArgs a;
    a.cu_q[0] = 1;
    EXPECT(a.check(0, &d) == kBadOffsets);
    a.cu_q = {0, 3, 1, 4};
    EXPECT(a.check(1, &d) == kBadOffsets);
    a.cu_q = {0, 1, 3, 5};
    EXPECT(a.check(2, &d) == kBadOffsets && d == 5);
  }
  {  // query counts 0 and above max_q_len
    DecodeArgs a;
    a.cu_q = {0, 1, 1, 4};
    EXPECT(a.check(1, &d) == kBadQueryLen && d == 0);
    EXPECT(a.check(2, &d) == kBadQueryLen && d == 3);
  }
  {  // the lowest failing sequence wins
    DecodeArgs a;
    a.table[6] = -3;
    a.seq_lens[1] = 500;
    EXPECT(a.first(&d) == encode(1, kBadSeqLen) && d == 500);
    EXPECT(failed_sequence(encode(1, kBadSeqLen)) == 1 && failed_code(encode(1, kBadSeqLen)) == kBadSeqLen);
  }
}

void test_append_checks() {
  const int max_pages = 3, batch = 3, total_new = 3, page_size = 64;
  const int64_t num_pages = 10;
  std::vector<int32_t> cu_new{0, 1, 3, 3};
  std::vector<int32_t> prefix{4, 126, 0};
  std::vector<int32_t> table{7, -5, -5, 2, 3, -5, -9, -9, -9};
  auto check = [&](int b, int32_t* d) {
    return check_append_sequence(b, cu_new.data(), prefix.data(), table.data(), max_pages, batch, total_new,
                                 page_size, num_pages, d);
  };
  int32_t d = 0;
  // sequence 0 writes position 4 (page 0), sequence 1 positions 126..127
  // (page 1), sequence 2 nothing: the garbage entries are never read
  EXPECT(check(0, &d) == kOk && check(1, &d) == kOk && check(2, &d) == kOk);
  prefix[1] = 127;  // positions 127..128 now reach page 2
  EXPECT(check(1, &d) == kBadPage && d == 2);
  prefix[1] = 126;
  table[4] = 10;
  EXPECT(check(1, &d) == kBadPage && d == 1);
  table[4] = 3;
  prefix[0] = -1;
  EXPECT(check(0, &d) == kBadPrefix && d == -1);
  prefix[0] = 3 * 64;  // one token past the table row
  EXPECT(check(0, &d) == kBadPrefix);
  prefix[0] = 4;
  cu_new = {0, 2, 1, 3};
  EXPECT(check(1, &d) == kBadOffsets);
  cu_new = {0, 1, 3, 2};
  EXPECT(check(2, &d) == kBadOffsets && d == 2);
}

// ---------------------------------------------------------------------------
// pool.cpp

void test_pool() {
  mla_page_pool* pool = nullptr;
  EXPECT(mla_pool_create(0, 64, 4, 3, &pool) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_pool_create(10, 64, 4, 3, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_pool_create(10, 64, 4, 3, &pool) == MLA_OK && pool);
  EXPECT(mla_pool_free_pages(pool) == 10);
  EXPECT(mla_pool_reserve(pool, 0, 100) == MLA_OK);   // 2 pages
  EXPECT(mla_pool_reserve(pool, 1, 192) == MLA_OK);   // 3 pages
  EXPECT(mla_pool_free_pages(pool) == 5);
  EXPECT(mla_pool_length(pool, 0) == 100 && mla_pool_length(pool, 1) == 192);
  EXPECT(mla_pool_reserve(pool, 2, 193) == MLA_ERR_INVALID_ARG);   // beyond 3 pages of 64
  EXPECT(mla_pool_reserve(pool, -1, 1) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_pool_reserve(pool, 4, 1) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_pool_reserve(pool, 2, 192) == MLA_OK && mla_pool_free_pages(pool) == 2);
  EXPECT(mla_pool_reserve(pool, 3, 192) == MLA_ERR_INSUFFICIENT_WORKSPACE);
  EXPECT(mla_pool_free_pages(pool) == 2 && mla_pool_length(pool, 3) == 0);   // unchanged
  std::vector<int32_t> table(2 * 3, 77);
  const int32_t seqs[2] = {1, 0};
  EXPECT(mla_pool_page_table(pool, seqs, 2, table.data()) == MLA_OK);
  EXPECT(table[0] == 2 && table[1] == 3 && table[2] == 4);   // ascending hand-out
  EXPECT(table[3] == 0 && table[4] == 1 && table[5] == -1);
  const int32_t bad[1] = {9};
  EXPECT(mla_pool_page_table(pool, bad, 1, table.data()) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_pool_release(pool, 0) == MLA_OK && mla_pool_free_pages(pool) == 4);
  EXPECT(mla_pool_reserve(pool, 3, 128) == MLA_OK);   // reuses sequence 0's pages
  EXPECT(mla_pool_page_table(pool, seqs + 0, 1, table.data()) == MLA_OK);
  const int32_t three[1] = {3};
  EXPECT(mla_pool_page_table(pool, three, 1, table.data()) == MLA_OK);
  EXPECT(table[0] == 0 && table[1] == 1 && table[2] == -1);
  EXPECT(mla_pool_release(pool, 7) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_pool_length(pool, 7) == -1);
  mla_pool_destroy(pool);
  mla_pool_destroy(nullptr);
}

mla_config dsv2_config() {
  mla_config c;
  memset(&c, 0, sizeof c);
  c.d_model = 5120;
  c.num_attention_heads = 128;
  c.qk_nope_head_dim = 128;
  c.qk_rope_head_dim = 64;
  c.v_head_dim = 128;
  c.kv_lora_rank = 512;
  c.page_size = 64;
  c.rope_base = 10000.f;
  c.softmax_scale = 0.f;
  c.dtype = MLA_DTYPE_BF16;
  c.cache_format = MLA_CACHE_DTYPE;
  return c;
}

void test_planner() {
  mla_config c = dsv2_config();
  mla_cache_plan plan;
  EXPECT(mla_plan_cache(&c, 60, (size_t)1 << 30, &plan) == MLA_OK);
  EXPECT(plan.bytes_per_token == 1152 * 60 && plan.page_bytes == 64 * 1152);
  EXPECT(plan.num_pages == (int64_t)(((size_t)1 << 30) / (60 * plan.page_bytes)));
  EXPECT(mla_plan_cache(&c, 0, (size_t)1 << 30, &plan) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_plan_cache(nullptr, 1, 1, &plan) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_plan_max_sequences(&c, 60, (size_t)1 << 30, 0) == -1);
  EXPECT(mla_plan_max_sequences(&c, 1, 64 * 1152 * 5, 64 * 2) == 2);
}

// ---------------------------------------------------------------------------
// api.hip host validation

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

void test_api_validation() {
  mla_config c = dsv2_config();
  EXPECT(mla_folded_bytes(nullptr) == 0);
  EXPECT(mla_cache_bytes_per_token(&c) == 1152);
  mla_config odd = c;
  odd.qk_rope_head_dim = 63;
  EXPECT(mla_folded_bytes(&odd) == 0);
  mla_config wide = c;
  wide.kv_lora_rank = 256;   // bf16 kernels are built for d_c = 512
  mla_layer* out = nullptr;
  EXPECT(mla_fold_weights(&wide, fake(0x1000), fake(0x1000), fake(0x1000), fake(0x1000), 1 << 30, nullptr,
                          &out) == MLA_ERR_UNSUPPORTED && out == nullptr);
  EXPECT(strlen(mla_last_error()) > 0);
  EXPECT(mla_fold_weights(nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, &out) == MLA_ERR_INVALID_ARG);
  EXPECT(strcmp(mla_status_string(MLA_ERR_HIP), "MLA_ERR_HIP") == 0);

  // a layer handle with stand-in device pointers (never dereferenced here)
  mla_layer* L = new mla_layer();
  L->cfg = c;
  L->elem = 2;
  L->scale = 0.0721687836f;
  L->wdkv_t = L->wuk_p = L->wuv_p = L->wukt_p = fake(0x10000);
  L->num_cus = 256;
  const int32_t* dev_i = static_cast<const int32_t*>(fake(0x20000));
  void* dev = fake(0x30000);

  // split plans on 256 compute units
  EXPECT(mla_decode_kv_chunk(L, 32, 1, 4096, 0) == 1024);
  EXPECT(mla_decode_kv_chunk(L, 8, 1, 131072, 0) == 4096);
  EXPECT(mla_decode_kv_chunk(L, 256, 2, 32770, 0) == 8192);
  EXPECT(mla_decode_kv_chunk(L, 32, 1, 4096, 100) == -1);
  EXPECT(mla_decode_kv_chunk(L, 0, 1, 4096, 0) == -1);
  EXPECT(mla_layer_set_attention_rows(L, 128) == MLA_OK);
  EXPECT(mla_decode_kv_chunk(L, 32, 1, 4096, 0) == 512);
  EXPECT(mla_layer_set_attention_rows(L, 96) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_layer_set_attention_rows(nullptr, 0) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_layer_set_attention_rows(L, 0) == MLA_OK);

  const size_t ws = mla_decode_workspace_bytes(L, 32, 32, 1, 4096, 0);
  EXPECT(ws > 0 && mla_decode_workspace_bytes(L, 32, 32, 1, 0, 0) == 0);
  // every call below fails a host check, so nothing is enqueued
  EXPECT(mla_decode(L, nullptr, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, 0, dev, 2048, dev, dev, ws, nullptr) ==
         MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode(L, dev, dev_i, dev_i, dev_i, 64, 0, 32, 1, 4096, 0, dev, 2048, dev, dev, ws, nullptr) ==
         MLA_ERR_INVALID_ARG);
  EXPECT(mla_decode(L, dev, dev_i, dev_i, dev_i, 64, 32, 31, 1, 4096, 0, dev, 2048, dev, dev, ws, nullptr) ==
         MLA_ERR_INVALID_ARG);                                  // total_q < batch
  EXPECT(mla_decode(L, dev, dev_i, dev_i, dev_i, 63, 32, 32, 1, 4096, 0, dev, 2048, dev, dev, ws, nullptr) ==
         MLA_ERR_INVALID_ARG);                                  // table row shorter than max_seq_len
  EXPECT(mla_decode(L, dev, dev_i, dev_i, dev_i, 64, 32, 33, 1, 4096, 0, dev, 2048, dev, dev, ws, nullptr) ==
         MLA_ERR_INVALID_ARG);                                  // total_q > batch * max_q_len
  EXPECT(mla_decode(L, dev, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, 96, dev, 2048, dev, dev, ws, nullptr) ==
         MLA_ERR_INVALID_ARG);                                  // kv_chunk not a multiple of 64
  EXPECT(mla_decode(L, dev, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, 0, dev, 2048, dev, dev, ws - 1, nullptr) ==
         MLA_ERR_INSUFFICIENT_WORKSPACE);
  EXPECT(mla_decode(L, dev, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, 0, dev, 2048, dev, fake(0x30001), ws,
                    nullptr) == MLA_ERR_INVALID_ARG);           // unaligned workspace
  EXPECT(mla_decode_phases(L, dev, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, 0, dev, 2048, dev, dev, ws, nullptr,
                           8) == MLA_ERR_INVALID_ARG);          // unknown phase bit
  // more splits than the no-allocation scratch holds
  EXPECT(mla_decode_no_alloc(L, dev, dev_i, dev_i, dev_i, 128, 32, 32, 1, 8192, 64, dev, 4096, dev, nullptr) ==
         MLA_ERR_INSUFFICIENT_WORKSPACE);
  EXPECT(strstr(mla_last_error(), "scratch") != nullptr);
  EXPECT(mla_decode_step(L, dev, dev_i, dev_i, -1, dev, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, 0, dev, 2048,
                         dev, dev, ws, nullptr) == MLA_ERR_INVALID_ARG);
  EXPECT(mla_append_latent(L, dev, dev_i, dev_i, dev_i, 64, 32, 32, dev, 2048, dev, 0, nullptr) ==
         MLA_ERR_INSUFFICIENT_WORKSPACE);
  EXPECT(mla_append_latent(L, nullptr, dev_i, dev_i, dev_i, 64, 32, 32, dev, 2048, dev, 1 << 30, nullptr) ==
         MLA_ERR_INVALID_ARG);
  EXPECT(mla_append_latent(L, dev, dev_i, dev_i, dev_i, 64, 32, 0, dev, 2048, dev, 0, nullptr) == MLA_OK);
  EXPECT(mla_extend(L, dev, dev_i, dev_i, dev_i, 64, 4, 4096, 1024, 4096, 9, dev, 2048, dev, dev, 1 << 30,
                    nullptr) == MLA_ERR_INVALID_ARG);           // unknown path
  EXPECT(mla_extend(L, dev, dev_i, dev_i, dev_i, 64, 4, 3, 1024, 4096, MLA_EXTEND_EXPANDED, dev, 2048, dev, dev,
                    1 << 30, nullptr) == MLA_ERR_INVALID_ARG);  // total_q < batch
  EXPECT(mla_decode_project(L, dev, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, dev, 2048, dev, dev, 1 << 30,
                            nullptr) == MLA_ERR_INVALID_ARG);   // no output projection folded
  EXPECT(mla_decode_hidden(L, dev, dev_i, dev_i, dev_i, 64, 32, 32, 1, 4096, dev, 2048, dev, dev, 1 << 30,
                           nullptr) == MLA_ERR_INVALID_ARG);    // no query projection folded
  EXPECT(mla_extend_choose_path(&c, 4, 4096, 1024, 4096) == MLA_EXTEND_EXPANDED ||
         mla_extend_choose_path(&c, 4, 4096, 1024, 4096) == MLA_EXTEND_ABSORBED);
  EXPECT(mla_output_choose_form(nullptr, 1) == -1);
  EXPECT(mla_query_choose_form(&odd, 1) == -1);
  mla_layer_free(L);
  mla_layer_free(nullptr);
}

}  // namespace

int main() {
  test_decode_checks();
  test_append_checks();
  test_pool();
  test_planner();
  test_api_validation();
  printf("host checks: %d of %d expectations held\n", g_cases - g_failed, g_cases);
  return g_failed ? 1 : 0;
}

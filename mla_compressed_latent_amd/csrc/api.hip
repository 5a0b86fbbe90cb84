// Host side of the C ABI declared in include/mla.h: argument validation,
// buffer carving, the split plan, and kernel launches.  No device memory is
// allocated here; every buffer comes from the caller.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>
#include <string>

#include "../../include/mla.h"
#include "check.hpp"
#include "kernels.hpp"
#include "layer.hpp"

// The checking build compiles this file with -DMLA_DEBUG_CHECKS=1.
#ifndef MLA_DEBUG_CHECKS
#define MLA_DEBUG_CHECKS 0
#endif

namespace {

thread_local std::string g_err;

mla_status fail(mla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Checks a config; returns MLA_OK or the failing status (message in g_err).
mla_status check_config(const mla_config* c) {
  if (!c) return fail(MLA_ERR_INVALID_ARG, "config is null");
  if (c->d_model <= 0 || c->num_attention_heads <= 0 || c->qk_nope_head_dim <= 0 ||
      c->qk_rope_head_dim <= 0 || c->v_head_dim <= 0 || c->kv_lora_rank <= 0 || c->page_size <= 0)
    return fail(MLA_ERR_INVALID_ARG, "every dimension must be positive");
  if (c->qk_rope_head_dim % 2) return fail(MLA_ERR_INVALID_ARG, "qk_rope_head_dim must be even");
  if (c->kv_lora_rank % 2) return fail(MLA_ERR_INVALID_ARG, "kv_lora_rank must be even");
  if (c->page_size % 64) return fail(MLA_ERR_INVALID_ARG, "page_size must be a multiple of 64");
  if (!(c->rope_base > 1.f) || !isfinite(c->rope_base))
    return fail(MLA_ERR_INVALID_ARG, "rope_base must be a finite value > 1");
  if (!isfinite(c->softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (c->dtype == MLA_DTYPE_BF16) {
    if (c->kv_lora_rank != 512 || c->qk_rope_head_dim != 64)
      return fail(MLA_ERR_UNSUPPORTED, "bf16 layers need kv_lora_rank 512 and qk_rope_head_dim 64");
    if (c->qk_nope_head_dim % 32 || c->v_head_dim % 32 || c->qk_nope_head_dim > 256)
      return fail(MLA_ERR_UNSUPPORTED,
                  "bf16 layers need qk_nope_head_dim (<= 256) and v_head_dim multiples of 32");
    if (c->d_model % 256)
      return fail(MLA_ERR_UNSUPPORTED, "bf16 layers need d_model to be a multiple of 256");
  } else if (c->dtype == MLA_DTYPE_F32) {
    if (c->kv_lora_rank > 1024 || c->kv_lora_rank % 4)
      return fail(MLA_ERR_UNSUPPORTED, "fp32 layers need kv_lora_rank <= 1024 and a multiple of 4");
  } else {
    return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", (int)c->dtype);
  }
  if (c->cache_format != MLA_CACHE_DTYPE && c->cache_format != MLA_CACHE_FP8)
    return fail(MLA_ERR_INVALID_ARG, "unknown cache_format %d", (int)c->cache_format);
  if (c->cache_format == MLA_CACHE_FP8 && c->dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "the FP8 cache format needs a bf16 layer");
  return MLA_OK;
}

// Bytes of one cached token (row plus, for FP8, its scale).
size_t token_bytes(const mla_config* c) {
  if (c->cache_format == MLA_CACHE_FP8) return mla::kFp8RowBytes + 4;
  return (size_t)(c->kv_lora_rank + c->qk_rope_head_dim) * (c->dtype == MLA_DTYPE_BF16 ? 2 : 4);
}

int elem_of(const mla_config* c) { return c->dtype == MLA_DTYPE_BF16 ? 2 : 4; }

struct FoldLayout {
  size_t off_wdkv, off_wuk, off_wuv, off_wukt, total;
};

FoldLayout fold_layout(const mla_config* c) {
  const size_t e = elem_of(c);
  const size_t D = (size_t)c->kv_lora_rank + c->qk_rope_head_dim;
  FoldLayout f;
  f.off_wdkv = 0;
  f.off_wuk = align256(D * c->d_model * e);
  f.off_wuv = f.off_wuk + align256((size_t)c->num_attention_heads * c->kv_lora_rank * c->qk_nope_head_dim * e);
  f.off_wukt = f.off_wuv + align256((size_t)c->num_attention_heads * c->v_head_dim * c->kv_lora_rank * e);
  // the transposed key weights of the expanded path (bf16 layers only)
  f.total = f.off_wukt + (c->dtype == MLA_DTYPE_BF16
                              ? align256((size_t)c->num_attention_heads * c->qk_nope_head_dim *
                                         c->kv_lora_rank * e)
                              : 0);
  return f;
}

mla_status hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

// Split plan for a decode call (depends on host arguments only).
bool make_plan(const mla_layer* L, int batch, int max_q_len, int max_seq_len, int kv_chunk,
               mla::SplitPlan* p) {
  const int H = L->cfg.num_attention_heads;
  const int rows = max_q_len * H;
  if (kv_chunk > 0 && (kv_chunk % 64 || kv_chunk > 8192)) return false;
  // One resident workgroup per compute unit: cover the longest sequences
  // with about one wave of workgroups, up to the kernels' largest split (a
  // batch of 256 ragged sequences of up to 32k tokens measured 2.55 ms per
  // step at 8192-token splits, 2.65 at 4096, 2.9 at 2048: fewer splits to
  // merge outweigh the coarser balance).
  auto chunk_for = [&](int rq) {
    if (kv_chunk > 0) return kv_chunk;
    const double work = (double)batch * rq * max_seq_len;
    long c = (long)ceil(work / (double)L->num_cus);
    c = ((c + 63) / 64) * 64;
    if (c < 256) c = 256;
    if (c > 8192) c = 8192;
    return (int)c;
  };
  p->NB = 1;
  p->RQ = 1;
  if (L->elem == 2 && rows > 32) {
    // more than 32 rows: 64-row workgroups of eight waves, or (bf16 pages,
    // more than 64 rows) 128-row workgroups of four waves.  The 128-row
    // kernel's loop is the faster one per row, but its start (query rows and
    // first tiles) and its write-out are longer, it takes twice the splits
    // of the 64-row kernel, and its long workgroups balance worse when there
    // are more of them than compute units: by shape it is taken for splits
    // of 1024 tokens or more when the batch's 128-row groups number at most
    // one per compute unit (measured, DeepSeek-V2 shape: B32 x 4096, 512-token
    // splits, 60 vs 52 us; B8 x 128k, 4096-token splits, 345 vs 375 us;
    // 256 ragged sequences of up to 32k with one or two queries, 8192-token
    // splits, 3.35 vs 2.47 ms).
    const bool r128_ok = rows > 64 && L->cfg.cache_format == MLA_CACHE_DTYPE;
    const int rq128 = (rows + 127) / 128;
    bool use128 = r128_ok && (int64_t)batch * rq128 <= L->num_cus && chunk_for(rq128) >= 1024;
    if (L->attn_rows == 128) use128 = r128_ok;
    if (L->attn_rows == 64) use128 = false;
    if (use128) {
      p->NB = 128;
      p->RQ = (rows + 127) / 128;
    } else {
      p->NB = 8;
      p->RQ = (rows + 63) / 64;
    }
  }
  p->chunk = chunk_for(p->RQ);
  p->S_max = (max_seq_len + p->chunk - 1) / p->chunk;
  // More workgroups than compute units: launch from a device-built list of
  // the items that have rows and tokens (ragged batches otherwise launch
  // many that exit at once, interleaved with the busy ones).
  p->list = (p->NB == 8 || p->NB == 128) && p->RQ <= 4096 &&
            (int64_t)batch * p->S_max * p->RQ > L->num_cus;
  // the launch grid (at most twice the full grid with a work list) stays an int
  const int64_t grid = (int64_t)batch * p->S_max * p->RQ;
  if (2 * grid + (int64_t)16 * p->RQ > INT32_MAX) return false;
  return p->S_max <= 1024;   // split weights of one row are staged on chip
}

struct DecodeLayout {
  size_t off_abuf, off_opart, off_lse, off_olat, off_work, total;
};

DecodeLayout decode_layout(const mla_layer* L, int batch, int total_q, const mla::SplitPlan& p) {
  const mla_config& c = L->cfg;
  const size_t rows = (size_t)total_q * c.num_attention_heads;
  const size_t D = (size_t)c.kv_lora_rank + c.qk_rope_head_dim;
  DecodeLayout d;
  d.off_abuf = 0;
  d.off_opart = align256(rows * D * L->elem);
  const size_t part_elem = L->elem == 2 ? 2 : 4;   // bf16 layers' split-KV kernels write bf16 partials
  d.off_lse = d.off_opart + align256((size_t)p.S_max * rows * c.kv_lora_rank * part_elem);
  d.off_olat = d.off_lse + align256((size_t)p.S_max * rows * 4);
  d.off_work = d.off_olat + align256(rows * c.kv_lora_rank * L->elem);
  d.total = d.off_work + (p.list ? align256(mla::work_list_bytes(batch, p)) : 0);
  return d;
}

// Expanded-path workspace: per-head content keys [batch][H][lmax][d_nope] and
// values [batch][H][lmax/64][d_v][64], lmax = max_seq_len rounded up to 256
// (the expansion kernel's token block).
struct ExtendLayout {
  int lmax;
  size_t off_k, off_v, total;
};

ExtendLayout extend_layout(const mla_config& c, int batch, int max_seq_len) {
  ExtendLayout e;
  e.lmax = (max_seq_len + 255) / 256 * 256;
  const size_t per = (size_t)batch * c.num_attention_heads * e.lmax * 2;
  e.off_k = 0;
  e.off_v = align256(per * c.qk_nope_head_dim);
  e.total = e.off_v + align256(per * c.v_head_dim);
  return e;
}

bool expanded_available(const mla_config& c) {
  return c.dtype == MLA_DTYPE_BF16 && c.cache_format == MLA_CACHE_DTYPE &&
         mla::extend_expanded_supported(c.qk_nope_head_dim, c.v_head_dim);
}

// Matrix-core work of the two forms for these host bounds (average keys per
// query taken as max_seq_len - max_q_len / 2, the causal mean of a chunk that
// ends the sequence).  Absorbed: every query is folded into latent space and
// back (2 d_c (d_nope + d_v) per query and head) and scored at width
// 2 d_c + d_rope per key.  Expanded: every cached token is expanded once per
// head (2 d_c (d_nope + d_v)) and scored at width d_nope + d_rope + d_v.
// The expanded count is weighted by kExpandedWeight, the ratio of the two
// paths' measured matrix-core efficiencies.
constexpr double kExpandedWeight = 1.0;

int choose_extend_path(const mla_config& c, int batch, int total_q, int max_q_len, int max_seq_len) {
  if (!expanded_available(c)) return MLA_EXTEND_ABSORBED;
  const double H = c.num_attention_heads, dc = c.kv_lora_rank, dr = c.qk_rope_head_dim;
  const double dn = c.qk_nope_head_dim, dv = c.v_head_dim;
  const double keys = (double)max_seq_len - 0.5 * (double)max_q_len;
  const double absorbed = (double)total_q * H * (2.0 * dc * (dn + dv) + 2.0 * (2.0 * dc + dr) * keys);
  const double expanded = (double)batch * max_seq_len * H * 2.0 * dc * (dn + dv) +
                          (double)total_q * H * 2.0 * (dn + dr + dv) * keys;
  return expanded * kExpandedWeight < absorbed ? MLA_EXTEND_EXPANDED : MLA_EXTEND_ABSORBED;
}

}  // namespace

namespace {

// Host checks of a decode call; fills the split plan and the workspace layout.
mla_status decode_prepare(const mla_layer* L, const void* q, const int32_t* cu_q,
                          const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                          int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                          int32_t kv_chunk, const void* cache, int64_t num_pages, const void* out,
                          const void* workspace, size_t workspace_bytes, mla::SplitPlan* p,
                          DecodeLayout* d) {
  if (!q || !cu_q || !seq_lens || !page_table || !cache || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode: null pointer argument");
  if (batch <= 0 || total_q < batch || max_q_len <= 0 || max_seq_len < max_q_len || max_pages <= 0 ||
      num_pages <= 0 || (int64_t)max_pages * L->cfg.page_size < max_seq_len)
    return fail(MLA_ERR_INVALID_ARG,
                "mla_decode: bad sizes (batch %d, total_q %d, max_q_len %d, max_seq_len %d, max_pages %d)",
                batch, total_q, max_q_len, max_seq_len, max_pages);
  if ((int64_t)total_q > (int64_t)batch * max_q_len)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode: total_q exceeds batch * max_q_len");
  if (kv_chunk < 0 || kv_chunk % 64 || kv_chunk > 8192)
    return fail(MLA_ERR_INVALID_ARG, "mla_decode: kv_chunk must be 0 or a multiple of 64 up to 8192");
  if (!make_plan(L, batch, max_q_len, max_seq_len, kv_chunk, p))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode: cannot plan the split");
  *d = decode_layout(L, batch, total_q, *p);
  if (workspace_bytes < d->total)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "decode workspace holds %zu bytes, %zu needed",
                workspace_bytes, d->total);
  if ((uintptr_t)workspace % 256) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return MLA_OK;
}

// Enqueues the given phases of a decode call that passed decode_prepare.
void decode_launch(const mla_layer* L, const void* q, const int32_t* cu_q, const int32_t* seq_lens,
                   const int32_t* page_table, int32_t max_pages, int32_t batch, int32_t total_q,
                   int32_t max_q_len, const void* cache, void* out, char* ws, const mla::SplitPlan& p,
                   const DecodeLayout& d, uint32_t phases, hipStream_t st) {
  const mla_config& c = L->cfg;
  void* abuf = ws + d.off_abuf;
  float* opart = (float*)(ws + d.off_opart);
  float* lse = (float*)(ws + d.off_lse);
  void* olat = ws + d.off_olat;
  const int H = c.num_attention_heads;
  if (phases & MLA_PHASE_ABSORB)
    mla::launch_absorb(L->elem, q, L->wuk_p, abuf, cu_q, seq_lens, batch, total_q, max_q_len, H,
                       c.qk_nope_head_dim, c.qk_rope_head_dim, c.kv_lora_rank, c.rope_base, L->freq,
                       L->scale * 1.4426950408889634f, st);
  if (phases & MLA_PHASE_ATTEND)
    mla::launch_splitkv(L->elem, p, abuf, cache, cu_q, seq_lens, page_table, max_pages, batch, total_q, H,
                        c.kv_lora_rank, c.qk_rope_head_dim, c.page_size, L->scale, opart, lse,
                        c.cache_format == MLA_CACHE_FP8, ws + d.off_work, st);
  if (phases & MLA_PHASE_OUTPUT) {
    const bool part_bf16 = L->elem == 2;   // bf16 layers' split-KV kernels write bf16 partials
    if (L->elem == 2 && p.S_max <= mla::kCombineMaxSplits) {
      mla::launch_combine_out(p, opart, lse, cu_q, seq_lens, L->wuv_p, out, batch, total_q, H,
                              c.v_head_dim, L->num_cus, st);
    } else {
      mla::launch_combine(L->elem, p, opart, part_bf16, lse, cu_q, seq_lens, batch, total_q, H,
                          c.kv_lora_rank, olat, st);
      mla::launch_out_proj(L->elem, olat, L->wuv_p, out, total_q, H, c.kv_lora_rank, c.v_head_dim,
                           st);
    }
  }
}

// The append's rows from its GEMM partials (part): sum, rotate, round and
// scatter into the pages (or quantize, for FP8 pages).
void append_finish(const mla_layer* L, const float* part, const int32_t* cu_new,
                   const int32_t* prefix_lens, const int32_t* page_table, int32_t max_pages,
                   int32_t batch, int32_t total_new, void* cache, hipStream_t st) {
  const mla_config& c = L->cfg;
  const int ks = L->elem == 2 ? mla::append_ksplits_bf16(c.d_model) : 1;
  if (c.cache_format == MLA_CACHE_FP8)
    mla::launch_append_finish_fp8(part, ks, total_new, cu_new, prefix_lens, page_table, max_pages, batch,
                                  cache, c.page_size, L->freq, st);
  else
    mla::launch_append_finish(L->elem, part, ks, total_new, cu_new, prefix_lens, page_table, max_pages,
                              batch, cache, c.page_size, c.kv_lora_rank, c.qk_rope_head_dim, c.rope_base,
                              L->freq, st);
}

}  // namespace

// Scratch of mla_decode_no_alloc: its decode workspace, one copy per GPU,
// resident from the library's load on that GPU to the process end.  Host
// code never passes this name to a kernel (on the host it is only a
// stand-in); it uses the device address looked up once per device.
static __device__ __align__(256) char scratch[MLA_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (nullptr + g_err on error).
char* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    fail(MLA_ERR_HIP, "mla_decode_no_alloc: no usable current device (%d)", dev);
    return nullptr;
  }
  char* ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_dev[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !addr) {
    (void)hipGetLastError();
    fail(MLA_ERR_HIP, "mla_decode_no_alloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
         hipGetErrorString(e));
    return nullptr;
  }
  ptr = (char*)addr;
  g_scratch_dev[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

// Result words of the checking build's argument check (launch_check_args).
static __device__ uint32_t check_result[2];

namespace {

constexpr bool kDebugChecks = MLA_DEBUG_CHECKS != 0;
std::mutex g_check_mu;

const char* check_code_name(uint32_t code) {
  switch (code) {
    case mla_check::kBadOffsets: return "sequence offsets out of order or range";
    case mla_check::kBadQueryLen: return "query count outside [1, max_q_len]";
    case mla_check::kBadSeqLen: return "sequence length outside [query count, max_seq_len]";
    case mla_check::kBadPrefix: return "prefix length negative or beyond the page-table row";
    case mla_check::kBadPage: return "page id outside [0, num_pages) at page index";
  }
  return "unknown check failure";
}

// Checking build only: run the device check of this call's offsets,
// lengths and page ids, wait for it, and fail the call if it found a bad
// sequence.  Not under stream capture (it cannot wait there).  One check at
// a time per process: the result words are shared.
mla_status device_check(const char* what, bool append, const int32_t* cu, const int32_t* lens,
                        const int32_t* page_table, int max_pages, int batch, int total, int max_q_len,
                        int max_seq_len, int page_size, int64_t num_pages, hipStream_t st) {
  if (!kDebugChecks) return MLA_OK;
  auto hip_fail = [&](hipError_t e) {
    (void)hipGetLastError();
    return fail(MLA_ERR_HIP, "%s: device argument check: %s", what, hipGetErrorString(e));
  };
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return hip_fail(e);
  if (cs != hipStreamCaptureStatusNone) return MLA_OK;
  std::lock_guard<std::mutex> lock(g_check_mu);
  void* addr = nullptr;
  e = hipGetSymbolAddress(&addr, HIP_SYMBOL(check_result));
  if (e != hipSuccess || !addr) return hip_fail(e);
  mla::launch_check_args(append, cu, lens, page_table, max_pages, batch, total, max_q_len, max_seq_len,
                         page_size, num_pages, (uint32_t*)addr, st);
  uint32_t res[2] = {0, 0};
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(res, addr, sizeof res, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  if (res[0] == mla_check::kNone) return MLA_OK;
  return fail(MLA_ERR_INVALID_ARG, "%s: device argument check: sequence %d: %s %d", what,
              mla_check::failed_sequence(res[0]), check_code_name(mla_check::failed_code(res[0])),
              (int32_t)res[1]);
}

mla_status device_check_decode(const mla_layer* L, const char* what, const int32_t* cu_q, const int32_t* seq_lens,
                               const int32_t* page_table, int max_pages, int batch, int total_q, int max_q_len,
                               int max_seq_len, int64_t num_pages, hipStream_t st) {
  return device_check(what, false, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                      max_seq_len, L->cfg.page_size, num_pages, st);
}

mla_status device_check_append(const mla_layer* L, const char* what, const int32_t* cu_new,
                               const int32_t* prefix_lens, const int32_t* page_table, int max_pages, int batch,
                               int total_new, int64_t num_pages, hipStream_t st) {
  return device_check(what, true, cu_new, prefix_lens, page_table, max_pages, batch, total_new, 0, 0,
                      L->cfg.page_size, num_pages, st);
}

}  // namespace

// Shared with the host-only parts of the library (pool.cpp).
namespace mla_api {
mla_status fail_msg(mla_status s, const char* msg) { return fail(s, "%s", msg); }
size_t row_bytes(const mla_config* cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return token_bytes(cfg);
}
}  // namespace mla_api

#pragma GCC visibility push(default)
extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_INSUFFICIENT_WORKSPACE: return "MLA_ERR_INSUFFICIENT_WORKSPACE";
  }
  return "unknown mla_status";
}

const char* mla_last_error(void) { return g_err.c_str(); }

size_t mla_folded_bytes(const mla_config* cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return fold_layout(cfg).total;
}

size_t mla_cache_bytes_per_token(const mla_config* cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return token_bytes(cfg);
}

mla_status mla_fold_weights(const mla_config* cfg, const void* w_dkv, const void* w_uk,
                            const void* w_uv, void* folded, size_t folded_bytes, void* hip_stream,
                            mla_layer** out) {
  mla_status st = check_config(cfg);
  if (st != MLA_OK) return st;
  if (!w_dkv || !w_uk || !w_uv || !folded || !out)
    return fail(MLA_ERR_INVALID_ARG, "mla_fold_weights: null pointer argument");
  if ((uintptr_t)folded % 256) return fail(MLA_ERR_INVALID_ARG, "folded buffer must be 256-byte aligned");
  const FoldLayout f = fold_layout(cfg);
  if (folded_bytes < f.total)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "folded buffer holds %zu bytes, %zu needed", folded_bytes,
                f.total);
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return fail(MLA_ERR_HIP, "cannot query the current device");
  mla_layer* L = new (std::nothrow) mla_layer;
  if (!L) return fail(MLA_ERR_INVALID_ARG, "mla_fold_weights: out of host memory");
  L->cfg = *cfg;
  L->elem = elem_of(cfg);
  L->scale = cfg->softmax_scale > 0.f
                 ? cfg->softmax_scale
                 : (float)(1.0 / sqrt((double)(cfg->qk_nope_head_dim + cfg->qk_rope_head_dim)));
  L->wdkv_t = (char*)folded + f.off_wdkv;
  L->wuk_p = (char*)folded + f.off_wuk;
  L->wuv_p = (char*)folded + f.off_wuv;
  L->wukt_p = L->elem == 2 ? (char*)folded + f.off_wukt : nullptr;
  L->num_cus = ncu;
  for (int i = 0; i < mla::kRopePairs; ++i)
    L->freq.theta[i] = pow((double)cfg->rope_base, -2.0 * i / (double)cfg->qk_rope_head_dim);
  mla::launch_pack(L->elem, w_dkv, w_uk, w_uv, L->wdkv_t, L->wuk_p, L->wuv_p, L->wukt_p,
                   cfg->d_model, cfg->num_attention_heads, cfg->qk_nope_head_dim, cfg->v_head_dim,
                   cfg->kv_lora_rank, cfg->qk_rope_head_dim, (hipStream_t)hip_stream);
  st = hip_check("fold launch");
  if (st != MLA_OK) {
    delete L;
    return st;
  }
  *out = L;
  return MLA_OK;
}

void mla_layer_free(mla_layer* layer) { delete layer; }

mla_status mla_layer_set_attention_rows(mla_layer* L, int32_t rows) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  if (rows != 0 && rows != 64 && rows != 128)
    return fail(MLA_ERR_INVALID_ARG, "mla_layer_set_attention_rows: rows must be 0, 64 or 128 (got %d)", rows);
  L->attn_rows = rows;
  return MLA_OK;
}

size_t mla_append_workspace_bytes(const mla_layer* L, int32_t total_new) {
  if (!L || total_new < 0) return 0;
  const size_t D = (size_t)L->cfg.kv_lora_rank + L->cfg.qk_rope_head_dim;
  const size_t ks = L->elem == 2 ? (size_t)mla::append_ksplits_bf16(L->cfg.d_model) : 1;
  return align256(ks * (size_t)total_new * D * 4);
}

mla_status mla_append_latent(const mla_layer* L, const void* x, const int32_t* cu_new,
                             const int32_t* prefix_lens, const int32_t* page_table, int32_t max_pages,
                             int32_t batch, int32_t total_new, void* cache, int64_t num_pages,
                             void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  if (total_new < 0 || batch <= 0 || max_pages <= 0 || num_pages <= 0)
    return fail(MLA_ERR_INVALID_ARG, "mla_append_latent: bad sizes (batch %d, total_new %d, max_pages %d)",
                batch, total_new, max_pages);
  if (total_new == 0) return MLA_OK;
  if (!x || !cu_new || !prefix_lens || !page_table || !cache || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "mla_append_latent: null pointer argument");
  const size_t need = mla_append_workspace_bytes(L, total_new);
  if (workspace_bytes < need)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "append workspace holds %zu bytes, %zu needed",
                workspace_bytes, need);
  const mla_config& c = L->cfg;
  const int D = c.kv_lora_rank + c.qk_rope_head_dim;
  hipStream_t st = (hipStream_t)hip_stream;
  float* part = (float*)workspace;
  const mla_status chk = device_check_append(L, "mla_append_latent", cu_new, prefix_lens, page_table, max_pages,
                                             batch, total_new, num_pages, st);
  if (chk != MLA_OK) return chk;
  if (L->elem == 2)
    mla::launch_append_gemm_bf16(x, L->wdkv_t, part, total_new, D, c.d_model, st);
  else
    mla::launch_append_gemm_f32(x, L->wdkv_t, part, total_new, D, c.d_model, st);
  append_finish(L, part, cu_new, prefix_lens, page_table, max_pages, batch, total_new, cache, st);
  return hip_check("append launch");
}

int32_t mla_decode_kv_chunk(const mla_layer* L, int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                            int32_t kv_chunk) {
  if (!L || batch <= 0 || max_q_len <= 0 || max_seq_len < max_q_len || kv_chunk < 0) return -1;
  mla::SplitPlan p;
  if (!make_plan(L, batch, max_q_len, max_seq_len, kv_chunk, &p)) return -1;
  return p.chunk;
}

size_t mla_decode_workspace_bytes(const mla_layer* L, int32_t batch, int32_t total_q, int32_t max_q_len,
                                  int32_t max_seq_len, int32_t kv_chunk) {
  if (!L || batch <= 0 || total_q <= 0 || max_q_len <= 0 || max_seq_len < max_q_len || kv_chunk < 0)
    return 0;
  mla::SplitPlan p;
  if (!make_plan(L, batch, max_q_len, max_seq_len, kv_chunk, &p)) return 0;
  return decode_layout(L, batch, total_q, p).total;
}

mla_status mla_decode_phases(const mla_layer* L, const void* q, const int32_t* cu_q,
                             const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                             int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                             int32_t kv_chunk, const void* cache, int64_t num_pages, void* out,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             uint32_t phases) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  if (phases == 0 || (phases & ~(uint32_t)MLA_PHASE_ALL))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_phases: bad phase mask 0x%x", phases);
  mla::SplitPlan p;
  DecodeLayout d;
  const mla_status s = decode_prepare(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                                      max_seq_len, kv_chunk, cache, num_pages, out, workspace, workspace_bytes,
                                      &p, &d);
  if (s != MLA_OK) return s;
  const mla_status chk = device_check_decode(L, "mla_decode", cu_q, seq_lens, page_table, max_pages, batch,
                                             total_q, max_q_len, max_seq_len, num_pages, (hipStream_t)hip_stream);
  if (chk != MLA_OK) return chk;
  decode_launch(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len, cache, out,
                (char*)workspace, p, d, phases, (hipStream_t)hip_stream);
  return hip_check("decode launch");
}

mla_status mla_decode(const mla_layer* L, const void* q, const int32_t* cu_q, const int32_t* seq_lens,
                      const int32_t* page_table, int32_t max_pages, int32_t batch, int32_t total_q,
                      int32_t max_q_len, int32_t max_seq_len, int32_t kv_chunk, const void* cache,
                      int64_t num_pages, void* out, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  return mla_decode_phases(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                           max_seq_len, kv_chunk, cache, num_pages, out, workspace, workspace_bytes,
                           hip_stream, MLA_PHASE_ALL);
}

mla_status mla_decode_no_alloc(const mla_layer* L, const void* q, const int32_t* cu_q,
                               const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                               int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                               int32_t kv_chunk, const void* cache, int64_t num_pages, void* out,
                               void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  const size_t need = mla_decode_workspace_bytes(L, batch, total_q, max_q_len, max_seq_len, kv_chunk);
  if (need > MLA_NO_ALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE,
                "mla_decode_no_alloc: this call needs %zu bytes of scratch, the static buffer holds %zu; "
                "use mla_decode with a workspace",
                need, (size_t)MLA_NO_ALLOC_SCRATCH_BYTES);
  char* ws = scratch_address();
  if (!ws) return MLA_ERR_HIP;
  mla::SplitPlan p;
  DecodeLayout d;
  const mla_status s = decode_prepare(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                                      max_seq_len, kv_chunk, cache, num_pages, out, ws,
                                      MLA_NO_ALLOC_SCRATCH_BYTES, &p, &d);
  if (s != MLA_OK) return s;
  const mla_status chk = device_check_decode(L, "mla_decode_no_alloc", cu_q, seq_lens, page_table, max_pages,
                                             batch, total_q, max_q_len, max_seq_len, num_pages,
                                             (hipStream_t)hip_stream);
  if (chk != MLA_OK) return chk;
  decode_launch(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len, cache, out, ws, p, d,
                MLA_PHASE_ALL, (hipStream_t)hip_stream);
  return hip_check("decode launch");
}

size_t mla_decode_step_workspace_bytes(const mla_layer* L, int32_t batch, int32_t total_new,
                                       int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                                       int32_t kv_chunk) {
  if (!L || total_new < 0) return 0;
  const size_t dec = mla_decode_workspace_bytes(L, batch, total_q, max_q_len, max_seq_len, kv_chunk);
  if (dec == 0) return 0;
  return align256(dec) + mla_append_workspace_bytes(L, total_new);
}

mla_status mla_decode_step(const mla_layer* L, const void* x, const int32_t* cu_new,
                           const int32_t* prefix_lens, int32_t total_new, const void* q,
                           const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                           int32_t max_pages, int32_t batch, int32_t total_q, int32_t max_q_len,
                           int32_t max_seq_len, int32_t kv_chunk, void* cache, int64_t num_pages,
                           void* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  if (total_new < 0) return fail(MLA_ERR_INVALID_ARG, "mla_decode_step: total_new %d < 0", total_new);
  if (total_new > 0 && (!x || !cu_new || !prefix_lens))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_step: null pointer argument");
  mla::SplitPlan p;
  DecodeLayout d;
  mla_status s = decode_prepare(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                                max_seq_len, kv_chunk, cache, num_pages, out, workspace, workspace_bytes, &p,
                                &d);
  if (s != MLA_OK) return s;
  const size_t off_app = align256(d.total);
  const size_t need = off_app + mla_append_workspace_bytes(L, total_new);
  if (workspace_bytes < need)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "decode step workspace holds %zu bytes, %zu needed",
                workspace_bytes, need);
  const mla_config& c = L->cfg;
  hipStream_t st = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  float* part = (float*)(ws + off_app);
  const int D = c.kv_lora_rank + c.qk_rope_head_dim;
  if (total_new > 0) {
    s = device_check_append(L, "mla_decode_step", cu_new, prefix_lens, page_table, max_pages, batch, total_new,
                            num_pages, st);
    if (s != MLA_OK) return s;
  }
  s = device_check_decode(L, "mla_decode_step", cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                          max_seq_len, num_pages, st);
  if (s != MLA_OK) return s;
  uint32_t phases = MLA_PHASE_ALL;
  if (total_new > 0 && L->elem == 2 && c.cache_format == MLA_CACHE_DTYPE) {
    // the append GEMM, then the query absorb with the append finish
    mla::launch_append_gemm_bf16(x, L->wdkv_t, part, total_new, D, c.d_model, st);
    mla::launch_absorb_finish(q, L->wuk_p, ws + d.off_abuf, cu_q, seq_lens, batch, total_q, max_q_len,
                              c.num_attention_heads, c.qk_nope_head_dim, c.qk_rope_head_dim, c.kv_lora_rank,
                              L->freq, L->scale * 1.4426950408889634f, part,
                              mla::append_ksplits_bf16(c.d_model), total_new, cu_new, prefix_lens, page_table,
                              max_pages, cache, c.page_size, st);
    phases = MLA_PHASE_ATTEND | MLA_PHASE_OUTPUT;
  } else if (total_new > 0) {
    if (L->elem == 2) {
      // FP8 pages: the append GEMM with the query absorb, then the quantizing finish
      mla::launch_absorb_append(q, L->wuk_p, ws + d.off_abuf, cu_q, seq_lens, batch, total_q, max_q_len,
                                c.num_attention_heads, c.qk_nope_head_dim, c.qk_rope_head_dim,
                                c.kv_lora_rank, L->freq, L->scale * 1.4426950408889634f, x, L->wdkv_t, part,
                                total_new, D, c.d_model, st);
      phases = MLA_PHASE_ATTEND | MLA_PHASE_OUTPUT;
    } else {
      mla::launch_append_gemm_f32(x, L->wdkv_t, part, total_new, D, c.d_model, st);
    }
    append_finish(L, part, cu_new, prefix_lens, page_table, max_pages, batch, total_new, cache, st);
  }
  decode_launch(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len, cache, out, ws, p, d,
                phases, st);
  return hip_check("decode step launch");
}

int32_t mla_extend_choose_path(const mla_config* cfg, int32_t batch, int32_t total_q, int32_t max_q_len,
                               int32_t max_seq_len) {
  if (check_config(cfg) != MLA_OK) return -1;
  if (batch <= 0 || total_q < batch || max_q_len <= 0 || max_seq_len < max_q_len ||
      (int64_t)total_q > (int64_t)batch * max_q_len)
    return -1;
  return choose_extend_path(*cfg, batch, total_q, max_q_len, max_seq_len);
}

size_t mla_extend_workspace_bytes(const mla_layer* L, int32_t batch, int32_t total_q, int32_t max_q_len,
                                  int32_t max_seq_len, int32_t path) {
  if (!L) return 0;
  if (path == MLA_EXTEND_AUTO) path = mla_extend_choose_path(&L->cfg, batch, total_q, max_q_len, max_seq_len);
  if (path == MLA_EXTEND_ABSORBED)
    return mla_decode_workspace_bytes(L, batch, total_q, max_q_len, max_seq_len, 0);
  if (path != MLA_EXTEND_EXPANDED || !expanded_available(L->cfg)) return 0;
  if (batch <= 0 || total_q < batch || max_q_len <= 0 || max_seq_len < max_q_len) return 0;
  return extend_layout(L->cfg, batch, max_seq_len).total;
}

mla_status mla_extend(const mla_layer* L, const void* q, const int32_t* cu_q, const int32_t* seq_lens,
                      const int32_t* page_table, int32_t max_pages, int32_t batch, int32_t total_q,
                      int32_t max_q_len, int32_t max_seq_len, int32_t path, const void* cache,
                      int64_t num_pages, void* out, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  if (path != MLA_EXTEND_AUTO && path != MLA_EXTEND_ABSORBED && path != MLA_EXTEND_EXPANDED)
    return fail(MLA_ERR_INVALID_ARG, "mla_extend: unknown path %d", path);
  if (!q || !cu_q || !seq_lens || !page_table || !cache || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "mla_extend: null pointer argument");
  if (batch <= 0 || total_q < batch || max_q_len <= 0 || max_seq_len < max_q_len || max_pages <= 0 ||
      num_pages <= 0 || (int64_t)max_pages * L->cfg.page_size < max_seq_len ||
      (int64_t)total_q > (int64_t)batch * max_q_len)
    return fail(MLA_ERR_INVALID_ARG,
                "mla_extend: bad sizes (batch %d, total_q %d, max_q_len %d, max_seq_len %d, max_pages %d)",
                batch, total_q, max_q_len, max_seq_len, max_pages);
  if (path == MLA_EXTEND_AUTO) path = choose_extend_path(L->cfg, batch, total_q, max_q_len, max_seq_len);
  if (path == MLA_EXTEND_ABSORBED)
    return mla_decode_phases(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                             max_seq_len, 0, cache, num_pages, out, workspace, workspace_bytes, hip_stream,
                             MLA_PHASE_ALL);
  const mla_config& c = L->cfg;
  if (!expanded_available(c))
    return fail(MLA_ERR_UNSUPPORTED,
                "mla_extend: the expanded path needs a bf16 layer with a bf16 cache and "
                "qk_nope_head_dim and v_head_dim each 64 or 128");
  const ExtendLayout e = extend_layout(c, batch, max_seq_len);
  if (workspace_bytes < e.total)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "extend workspace holds %zu bytes, %zu needed",
                workspace_bytes, e.total);
  if ((uintptr_t)workspace % 256) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t st = (hipStream_t)hip_stream;
  const mla_status chk = device_check_decode(L, "mla_extend", cu_q, seq_lens, page_table, max_pages, batch,
                                             total_q, max_q_len, max_seq_len, num_pages, st);
  if (chk != MLA_OK) return chk;
  char* ws = (char*)workspace;
  const int H = c.num_attention_heads;
  mla::launch_expand_kv(cache, seq_lens, page_table, max_pages, batch, H, c.qk_nope_head_dim, c.v_head_dim,
                        c.page_size, e.lmax, L->wukt_p, L->wuv_p, ws + e.off_k, ws + e.off_v, st);
  mla::launch_extend_attn(q, ws + e.off_k, ws + e.off_v, cache, cu_q, seq_lens, page_table, max_pages, batch,
                          max_q_len, H, c.qk_nope_head_dim, c.v_head_dim, c.page_size, e.lmax, L->freq,
                          L->scale, out, st);
  return hip_check("extend launch");
}

int32_t mla_output_choose_form(const mla_config* cfg, int32_t total_q) {
  if (check_config(cfg) != MLA_OK || total_q < 1) return -1;
  // weight bytes streamed and matrix-core flops of the two forms; the time of
  // each is the larger of bytes / 8 TB/s and flops / 2.5 PFLOP/s
  const double H = cfg->num_attention_heads, dc = cfg->kv_lora_rank, dv = cfg->v_head_dim;
  const double dm = cfg->d_model, e = cfg->dtype == MLA_DTYPE_BF16 ? 2.0 : 4.0, T = total_q;
  const double unf = fmax(e * H * dv * (dc + dm) / 8e12, 2.0 * T * H * dv * (dc + dm) / 2.5e15);
  const double fol = fmax(e * H * dc * dm / 8e12, 2.0 * T * H * dc * dm / 2.5e15);
  return fol < unf ? MLA_OUTPUT_FOLDED : MLA_OUTPUT_UNFOLDED;
}

size_t mla_output_folded_bytes(const mla_config* cfg, int32_t form) {
  if (check_config(cfg) != MLA_OK || cfg->dtype != MLA_DTYPE_BF16) return 0;
  const size_t H = cfg->num_attention_heads, dm = cfg->d_model;
  if (form == MLA_OUTPUT_UNFOLDED) return align256(H * cfg->v_head_dim * dm * 2);
  if (form == MLA_OUTPUT_FOLDED) return align256(H * cfg->kv_lora_rank * dm * 2);
  return 0;
}

mla_status mla_fold_output(mla_layer* L, const void* w_uv, const void* w_o, int32_t form, void* folded,
                           size_t folded_bytes, void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  const mla_config& c = L->cfg;
  if (form == MLA_OUTPUT_AUTO) form = mla_output_choose_form(&c, 1);
  if (form != MLA_OUTPUT_UNFOLDED && form != MLA_OUTPUT_FOLDED)
    return fail(MLA_ERR_INVALID_ARG, "mla_fold_output: unknown form %d", form);
  if (c.dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "mla_fold_output: the projection kernels need a bf16 layer");
  // contraction width of the projection GEMM (its k-split is 256 wide)
  const int64_t K = (int64_t)c.num_attention_heads *
                    (form == MLA_OUTPUT_FOLDED ? c.kv_lora_rank : c.v_head_dim);
  if (K % 256)
    return fail(MLA_ERR_UNSUPPORTED,
                "mla_fold_output: num_attention_heads * %s must be a multiple of 256",
                form == MLA_OUTPUT_FOLDED ? "kv_lora_rank" : "v_head_dim");
  if (!w_o || !folded || (form == MLA_OUTPUT_FOLDED && !w_uv))
    return fail(MLA_ERR_INVALID_ARG, "mla_fold_output: null pointer argument");
  if ((uintptr_t)folded % 256) return fail(MLA_ERR_INVALID_ARG, "folded buffer must be 256-byte aligned");
  const size_t need = mla_output_folded_bytes(&c, form);
  if (folded_bytes < need)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "output fold buffer holds %zu bytes, %zu needed", folded_bytes,
                need);
  mla::launch_fold_output(form, w_uv, w_o, folded, c.num_attention_heads, c.kv_lora_rank, c.v_head_dim,
                          c.d_model, (hipStream_t)hip_stream);
  const mla_status st = hip_check("output fold launch");
  if (st != MLA_OK) return st;
  L->wo_p = folded;
  L->out_form = form;
  return MLA_OK;
}

namespace {
struct ProjectLayout {
  size_t off_dec, off_act, off_part, total;
  int K;
};
bool project_layout(const mla_layer* L, int batch, int total_q, int max_q_len, int max_seq_len,
                    ProjectLayout* pl) {
  const mla_config& c = L->cfg;
  const size_t dec = mla_decode_workspace_bytes(L, batch, total_q, max_q_len, max_seq_len, 0);
  if (dec == 0 || !L->wo_p) return false;
  pl->K = L->out_form == MLA_OUTPUT_FOLDED ? c.num_attention_heads * c.kv_lora_rank
                                           : c.num_attention_heads * c.v_head_dim;
  pl->off_dec = 0;
  pl->off_act = align256(dec);
  // unfolded: the per-head outputs [Tq][H*dv]; folded: o_lat sits in the
  // decode workspace already
  const size_t act = L->out_form == MLA_OUTPUT_FOLDED ? 0 : (size_t)total_q * pl->K * 2;
  pl->off_part = pl->off_act + align256(act);
  pl->total = pl->off_part + align256((size_t)(pl->K / 256) * total_q * c.d_model * 4);
  return true;
}
}  // namespace

size_t mla_decode_project_workspace_bytes(const mla_layer* L, int32_t batch, int32_t total_q,
                                          int32_t max_q_len, int32_t max_seq_len) {
  if (!L) return 0;
  ProjectLayout pl;
  if (!project_layout(L, batch, total_q, max_q_len, max_seq_len, &pl)) return 0;
  return pl.total;
}

mla_status mla_decode_project(const mla_layer* L, const void* q, const int32_t* cu_q, const int32_t* seq_lens,
                              const int32_t* page_table, int32_t max_pages, int32_t batch, int32_t total_q,
                              int32_t max_q_len, int32_t max_seq_len, const void* cache, int64_t num_pages,
                              void* y, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  if (!L->wo_p) return fail(MLA_ERR_INVALID_ARG, "mla_decode_project: no output projection folded (mla_fold_output)");
  if (!y || !workspace) return fail(MLA_ERR_INVALID_ARG, "mla_decode_project: null pointer argument");
  ProjectLayout pl;
  if (batch <= 0 || total_q < batch || max_q_len <= 0 || max_seq_len < max_q_len ||
      !project_layout(L, batch, total_q, max_q_len, max_seq_len, &pl))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_project: bad sizes");
  if (workspace_bytes < pl.total)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "project workspace holds %zu bytes, %zu needed",
                workspace_bytes, pl.total);
  if ((uintptr_t)workspace % 256) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const mla_config& c = L->cfg;
  hipStream_t st = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  const size_t dec_bytes = pl.off_act;
  const void* act;
  mla_status s;
  if (L->out_form == MLA_OUTPUT_UNFOLDED) {
    s = mla_decode_phases(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len, max_seq_len, 0,
                          cache, num_pages, ws + pl.off_act, ws, dec_bytes, hip_stream, MLA_PHASE_ALL);
    act = ws + pl.off_act;
  } else {
    // absorb and attend as in decode, then the split merge into o_lat (no W_uv)
    s = mla_decode_phases(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len, max_seq_len, 0,
                          cache, num_pages, y, ws, dec_bytes, hip_stream, MLA_PHASE_ABSORB | MLA_PHASE_ATTEND);
    if (s != MLA_OK) return s;
    mla::SplitPlan p;
    make_plan(L, batch, max_q_len, max_seq_len, 0, &p);
    const DecodeLayout d = decode_layout(L, batch, total_q, p);
    mla::launch_combine(L->elem, p, ws + d.off_opart, L->elem == 2, (const float*)(ws + d.off_lse), cu_q,
                        seq_lens, batch, total_q, c.num_attention_heads, c.kv_lora_rank, ws + d.off_olat, st);
    act = ws + d.off_olat;
  }
  if (s != MLA_OK) return s;
  mla::launch_project(act, L->wo_p, (float*)(ws + pl.off_part), y, total_q, c.d_model, pl.K, st);
  return hip_check("project launch");
}

int32_t mla_query_choose_form(const mla_config* cfg, int32_t total_q) {
  if (check_config(cfg) != MLA_OK || total_q < 1) return -1;
  // weight bytes streamed and matrix-core flops of the two forms (the
  // unfolded form also runs the per-head absorb through W_uk)
  const double H = cfg->num_attention_heads, dc = cfg->kv_lora_rank, dn = cfg->qk_nope_head_dim;
  const double dr = cfg->qk_rope_head_dim, dm = cfg->d_model;
  const double e = cfg->dtype == MLA_DTYPE_BF16 ? 2.0 : 4.0, T = total_q;
  const double wu = H * ((dn + dr) * dm + dn * dc), wf = H * (dc + dr) * dm;
  const double unf = fmax(e * wu / 8e12, 2.0 * T * wu / 2.5e15);
  const double fol = fmax(e * wf / 8e12, 2.0 * T * wf / 2.5e15);
  return fol < unf ? MLA_QUERY_FOLDED : MLA_QUERY_UNFOLDED;
}

size_t mla_query_folded_bytes(const mla_config* cfg, int32_t form) {
  if (check_config(cfg) != MLA_OK || cfg->dtype != MLA_DTYPE_BF16) return 0;
  const size_t H = cfg->num_attention_heads, dm = cfg->d_model;
  if (form == MLA_QUERY_UNFOLDED) return align256(H * (cfg->qk_nope_head_dim + cfg->qk_rope_head_dim) * dm * 2);
  if (form == MLA_QUERY_FOLDED) return align256(H * (cfg->kv_lora_rank + cfg->qk_rope_head_dim) * dm * 2);
  return 0;
}

mla_status mla_fold_query(mla_layer* L, const void* w_q, const void* w_uk, int32_t form, void* folded,
                          size_t folded_bytes, void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  const mla_config& c = L->cfg;
  if (form == MLA_QUERY_AUTO) form = mla_query_choose_form(&c, 1);
  if (form != MLA_QUERY_UNFOLDED && form != MLA_QUERY_FOLDED)
    return fail(MLA_ERR_INVALID_ARG, "mla_fold_query: unknown form %d", form);
  if (c.dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "mla_fold_query: the projection kernels need a bf16 layer");
  if (!w_q || !folded || (form == MLA_QUERY_FOLDED && !w_uk))
    return fail(MLA_ERR_INVALID_ARG, "mla_fold_query: null pointer argument");
  if ((uintptr_t)folded % 256) return fail(MLA_ERR_INVALID_ARG, "folded buffer must be 256-byte aligned");
  const size_t need = mla_query_folded_bytes(&c, form);
  if (folded_bytes < need)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "query fold buffer holds %zu bytes, %zu needed", folded_bytes,
                need);
  mla::launch_fold_query(form, w_q, w_uk, folded, c.num_attention_heads, c.qk_nope_head_dim,
                         c.qk_rope_head_dim, c.kv_lora_rank, c.d_model, (hipStream_t)hip_stream);
  const mla_status st = hip_check("query fold launch");
  if (st != MLA_OK) return st;
  L->wq_p = folded;
  L->q_form = form;
  return MLA_OK;
}

}  // extern "C"

namespace {
// Workspace of mla_decode_hidden: the decode's own, then (unfolded form) the
// projected queries [Tq][H*dq], then the projection's split-K partials.
struct HiddenLayout {
  size_t off_q, off_part, total;
  int N;
};
bool hidden_layout(const mla_layer* L, int batch, int total_q, int max_q_len, int max_seq_len,
                   HiddenLayout* hl) {
  const mla_config& c = L->cfg;
  const size_t dec = mla_decode_workspace_bytes(L, batch, total_q, max_q_len, max_seq_len, 0);
  if (dec == 0 || !L->wq_p) return false;
  const bool folded = L->q_form == MLA_QUERY_FOLDED;
  hl->N = c.num_attention_heads *
          ((folded ? c.kv_lora_rank : c.qk_nope_head_dim) + c.qk_rope_head_dim);
  hl->off_q = align256(dec);
  hl->off_part = hl->off_q + (folded ? 0 : align256((size_t)total_q * hl->N * 2));
  hl->total = hl->off_part +
              align256((size_t)mla::append_ksplits_bf16(c.d_model) * total_q * hl->N * 4);
  return true;
}
}  // namespace

extern "C" {

size_t mla_decode_hidden_workspace_bytes(const mla_layer* L, int32_t batch, int32_t total_q,
                                         int32_t max_q_len, int32_t max_seq_len) {
  if (!L) return 0;
  HiddenLayout hl;
  if (!hidden_layout(L, batch, total_q, max_q_len, max_seq_len, &hl)) return 0;
  return hl.total;
}

mla_status mla_decode_hidden(const mla_layer* L, const void* x, const int32_t* cu_q, const int32_t* seq_lens,
                             const int32_t* page_table, int32_t max_pages, int32_t batch, int32_t total_q,
                             int32_t max_q_len, int32_t max_seq_len, const void* cache, int64_t num_pages,
                             void* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!L) return fail(MLA_ERR_INVALID_ARG, "layer is null");
  if (!L->wq_p) return fail(MLA_ERR_INVALID_ARG, "mla_decode_hidden: no query projection folded (mla_fold_query)");
  HiddenLayout hl;
  if (batch <= 0 || total_q < batch || max_q_len <= 0 || max_seq_len < max_q_len ||
      !hidden_layout(L, batch, total_q, max_q_len, max_seq_len, &hl))
    return fail(MLA_ERR_INVALID_ARG, "mla_decode_hidden: bad sizes");
  if (!workspace) return fail(MLA_ERR_INVALID_ARG, "mla_decode_hidden: null pointer argument");
  if (workspace_bytes < hl.total)
    return fail(MLA_ERR_INSUFFICIENT_WORKSPACE, "hidden-input decode workspace holds %zu bytes, %zu needed",
                workspace_bytes, hl.total);
  const mla_config& c = L->cfg;
  hipStream_t st = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  float* part = (float*)(ws + hl.off_part);
  mla::SplitPlan p;
  DecodeLayout d;
  const mla_status s = decode_prepare(L, x, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len,
                                      max_seq_len, 0, cache, num_pages, out, ws, hl.off_q, &p, &d);
  if (s != MLA_OK) return s;
  const mla_status chk = device_check_decode(L, "mla_decode_hidden", cu_q, seq_lens, page_table, max_pages, batch,
                                             total_q, max_q_len, max_seq_len, num_pages, st);
  if (chk != MLA_OK) return chk;
  if (L->q_form == MLA_QUERY_UNFOLDED) {
    // q = x . W_q, then the whole decode from q (its own absorb)
    void* q = ws + hl.off_q;
    mla::launch_project(x, L->wq_p, part, q, total_q, hl.N, c.d_model, st);
    decode_launch(L, q, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len, cache, out, ws, p, d,
                  MLA_PHASE_ALL, st);
  } else {
    // folded: the projection writes the attention's query rows directly
    const int ks = mla::launch_project_gemm(x, L->wq_p, part, total_q, hl.N, c.d_model, st);
    mla::launch_query_finish(part, ks, total_q, c.num_attention_heads,
                             c.kv_lora_rank, c.qk_rope_head_dim, cu_q, seq_lens, batch, L->freq,
                             L->scale * 1.4426950408889634f, ws + d.off_abuf, st);
    decode_launch(L, x, cu_q, seq_lens, page_table, max_pages, batch, total_q, max_q_len, cache, out, ws, p,
                  d, MLA_PHASE_ATTEND | MLA_PHASE_OUTPUT, st);
  }
  return hip_check("hidden-input decode launch");
}

}  // extern "C"
#pragma GCC visibility pop

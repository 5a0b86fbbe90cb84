// Internal launchers of the MLA decode library (host side, not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mla {

// FP8 cache pages (MLA_CACHE_FP8): page_size rows of kFp8RowBytes (512 E4M3
// latent codes, then the 64 bf16 of the rotated rope key), then page_size
// fp32 row scales.
constexpr int kFp8RowBytes = 640;

// ---- checking build ---------------------------------------------------------
// One workgroup checks every sequence's device-resident offsets, lengths and
// page ids (check.hpp; append: cu = cu_new, lens = prefix_lens, total =
// total_new; else cu = cu_q, lens = seq_lens, total = total_q) and writes
// result[0] = the first failure's word (mla_check::kNone if none) and
// result[1] = its detail.
void launch_check_args(bool append, const int32_t* cu, const int32_t* lens, const int32_t* page_table,
                       int max_pages, int batch, int total, int max_q_len, int max_seq_len, int page_size,
                       int64_t num_pages, uint32_t* result, hipStream_t st);

// ---- fold (pack) ---------------------------------------------------------
// bf16 (elem 2): fragment-tiled wdkv (rows n, k = d), wuk[h] (rows j, k = i),
// wuv[h] (rows v, k = j), wukt[h] (rows i, k = j).  fp32 (elem 4):
// wdkv_t[n][d] = w_dkv[d][n]; wuk_p[h][j][i] = w_uk[j][h*dn+i];
// wuv_p[h][v][j] = w_uv[j][h*dv+v]; wukt unused (may be null).
void launch_pack(int elem, const void* w_dkv, const void* w_uk, const void* w_uv, void* wdkv_t,
                 void* wuk_p, void* wuv_p, void* wukt, int d_model, int H, int dn, int dv, int dc,
                 int dr, hipStream_t st);

// ---- append --------------------------------------------------------------
// part[ks][m][n] = sum over the ks-th k chunk of x[m][k] * wt[n][k].
int append_ksplits_bf16(int K);
void launch_append_gemm_bf16(const void* x, const void* wt, float* part, int M, int N, int K,
                             hipStream_t st);
void launch_append_gemm_f32(const void* x, const void* wt, float* part, int M, int N, int K,
                            hipStream_t st);
// Sum the k partials, rotate the rope block, round and scatter into pages.
void launch_append_finish(int elem, const float* part, int ksplits, int T, const int32_t* cu_new,
                          const int32_t* prefix_lens, const int32_t* page_table, int max_pages,
                          int batch, void* cache, int page_size, int dc, int dr, float base,
                          const RopeFreq& freq, hipStream_t st);

// FP8 cache rows (bf16 layers, d_c 512, d_rope 64): quantize each new row's
// latent with its power-of-two scale, rotate and round its rope key.
void launch_append_finish_fp8(const float* part, int ksplits, int T, const int32_t* cu_new,
                              const int32_t* prefix_lens, const int32_t* page_table, int max_pages,
                              int batch, void* cache, int page_size, const RopeFreq& freq,
                              hipStream_t st);

// ---- per-head GEMMs --------------------------------------------------------
// abuf[t][h][0:dc] = W_uk_h q_nope[t][h]; abuf[t][h][dc:] = rot(q_rope, pos_t);
// bf16 layers store both parts multiplied by qscale (softmax scale * log2 e).
void launch_absorb(int elem, const void* q, const void* wuk, void* abuf, const int32_t* cu_q,
                   const int32_t* seq_lens, int batch, int Tq, int max_q_len, int H, int dn, int dr,
                   int dc, float base, const RopeFreq& freq, float qscale, hipStream_t st);
// bf16 layers: launch_absorb's work and launch_append_gemm_bf16's (part,
// M = new tokens, N = row width, K = d_model) as one launch of one-wave blocks.
void launch_absorb_append(const void* q, const void* wuk, void* abuf, const int32_t* cu_q,
                          const int32_t* seq_lens, int batch, int Tq, int max_q_len, int H, int dn,
                          int dr, int dc, const RopeFreq& freq, float qscale, const void* x,
                          const void* wdkv, float* part, int M, int N, int K, hipStream_t st);
// bf16 layers with bf16 pages: launch_absorb's work and the append finish of
// launch_append_gemm_bf16's partials (part, ksplits, T_new new tokens) as one
// launch of one-wave blocks.
void launch_absorb_finish(const void* q, const void* wuk, void* abuf, const int32_t* cu_q,
                          const int32_t* seq_lens, int batch, int Tq, int max_q_len, int H, int dn,
                          int dr, int dc, const RopeFreq& freq, float qscale, const float* part,
                          int ksplits, int T_new, const int32_t* cu_new, const int32_t* prefix_lens,
                          const int32_t* page_table, int max_pages, void* cache, int page_size,
                          hipStream_t st);
// out[t][h][v] = sum_j olat[t][h][j] * wuv_p[h][v][j]
void launch_out_proj(int elem, const void* olat, const void* wuv_p, void* out, int Tq, int H, int dc,
                     int dv, hipStream_t st);

// ---- split-KV attention over the latent cache --------------------------------
struct SplitPlan {
  int chunk;    // tokens per work item (multiple of 64)
  int S_max;    // splits of the longest sequence
  int RQ;       // row groups per sequence (bf16 path)
  int NB;       // bf16 path: 1 = one 32-row block per workgroup, 8 = 64-row eight-wave kernel,
                // 128 = 128-row four-wave kernel (bf16 pages)
  bool list;    // NB 8 / 128: launch from a device-built list of busy work items
};
// Work list of a plan (bytes at its work pointer): a header of
// kListHeaderInts ints ([0] busy items, [1 + x] items of XCD x, [9 + x] where
// they start), the items (an int2 per possible item), then scratch for the
// ranked splits (an int2 per possible split).
constexpr int kListHeaderInts = 32;
inline size_t work_list_bytes(int batch, const SplitPlan& p) {
  return kListHeaderInts * 4 + ((size_t)batch * p.S_max * p.RQ + (size_t)batch * p.S_max) * 8;
}
// Workgroups of a launch from the work list: block id % 8 picks an XCD's
// items, id / 8 the item.  An XCD holds at most 2 ceil(batch S_max / 16)
// splits of at most RQ row groups each.
inline int work_list_grid(int batch, const SplitPlan& p) {
  return 8 * p.RQ * 2 * ((batch * p.S_max + 15) / 16);
}
// fp8: the cache holds MLA_CACHE_FP8 pages (bf16 layers).
void launch_splitkv(int elem, const SplitPlan& plan, const void* abuf, const void* cache,
                    const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                    int max_pages, int batch, int Tq, int H, int dc, int dr, int page_size,
                    float scale, float* opart, float* lse, bool fp8, void* work, hipStream_t st);
// out[t][h][:] = (LSE-weighted merge of the split partials) . W_uv_h, one
// workgroup per (32 query tokens, head); bf16 layers, at most kCombineMaxSplits.
constexpr int kCombineMaxSplits = 64;
// The partials are bf16 (every bf16 layer's split-KV kernel writes them so).
void launch_combine_out(const SplitPlan& plan, const void* opart, const float* lse,
                        const int32_t* cu_q, const int32_t* seq_lens, const void* wuv, void* out,
                        int batch, int Tq, int H, int dv, int num_cus, hipStream_t st);
// 64 query rows per workgroup, eight waves (bf16 layers, plan.NB == 8);
// bf16 partials.
void launch_splitkv_x8(const SplitPlan& plan, const void* abuf, const void* cache,
                       const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                       int max_pages, int batch, int Tq, int H, int page_size, void* opart,
                       float* lse, bool fp8, const int2* items, const int* list_hdr, hipStream_t st);
// 128 query rows per workgroup, four waves (bf16 layers with bf16 pages,
// plan.NB == 128); bf16 partials.
void launch_splitkv_r128(const SplitPlan& plan, const void* abuf, const void* cache,
                         const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                         int max_pages, int batch, int Tq, int H, int page_size, void* opart,
                         float* lse, const int2* items, const int* list_hdr, hipStream_t st);
// olat[t][h][:] = LSE-weighted merge of the split partials
void launch_combine(int elem, const SplitPlan& plan, const void* opart, bool part_bf16, const float* lse,
                    const int32_t* cu_q, const int32_t* seq_lens, int batch, int Tq, int H, int dc,
                    void* olat, hipStream_t st);

// ---- expanded prefill / chunked extend (bf16 layers) ------------------------
// Whether the expanded kernels are built for these head widths.
bool extend_expanded_supported(int dn, int dv);
// Per head, materialise the content keys and the values of every cached token
// of every sequence from its latent row, K_h[t][i] = sum_j c_t[j] W_uk[j][h*dn+i]
// and V_h[t][v] = sum_j c_t[j] W_uv[j][h*dv+v], for t < round_up(seq_len_b,
// 256) (rows past seq_len_b repeat the last row).  Both are stored per
// (sequence, head, 64-token tile) as 1 KB matrix-core operand fragments
// (64 lanes x 8 bf16):
//   kexp: fragment (tb, s), tb < 2, s < dn/16: lane l holds K[32 tb + l%32]
//         [16 s + 8 (l/32) .. + 7];
//   vexp: fragment (vb, k), vb < dv/32, k < 4: lane l holds V[t][32 vb + l%32]
//         for the eight tokens t = 16 k + 8 (e/4) + 4 (l/32) + e%4, e = 0..7.
// lmax (a multiple of 256) is the token stride of one (sequence, head).
void launch_expand_kv(const void* cache, const int32_t* seq_lens, const int32_t* page_table,
                      int max_pages, int batch, int H, int dn, int dv, int page_size, int lmax,
                      const void* wukt, const void* wuv, void* kexp, void* vexp, hipStream_t st);
// Causal flash attention of every query over its sequence's expanded keys
// and values: out[t][h][:] = softmax(scale * q_t . k) V.
void launch_extend_attn(const void* q, const void* kexp, const void* vexp, const void* cache,
                        const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                        int max_pages, int batch, int max_q_len, int H, int dn, int dv,
                        int page_size, int lmax, const RopeFreq& freq, float scale, void* out,
                        hipStream_t st);

// ---- output projection (bf16 layers) ----------------------------------------
// form 1: W_o [H*dv][dm] -> tiled (rows j < dm, k < H*dv); form 2: the fold
// W_uvo[j][h*dc + c] = sum_v W_uv[c][h*dv + v] W_o[h*dv + v][j], tiled (K = H*dc).
void launch_fold_output(int form, const void* w_uv, const void* w_o, void* out, int H, int dc, int dv,
                        int dm, hipStream_t st);
// ---- queries from the layer input (bf16 layers) -------------------------------
// form 1: W_q [dm][H*dq] -> tiled (rows H*dq, k < dm); form 2: the fold
// W_qa[h*D + j] = [W_q_h^nope W_uk_h^T | W_q_h^rope] (D = dc + dr), tiled (k < dm).
void launch_fold_query(int form, const void* w_q, const void* w_uk, void* out, int H, int dn, int dr,
                       int dc, int dm, hipStream_t st);
// abuf[t][h][:] (the attention's query rows, times qscale, rope part rotated at
// the token's position) from the split-K partials part[ks][Tq][H*(dc + dr)].
void launch_query_finish(const float* part, int ks, int Tq, int H, int dc, int dr, const int32_t* cu_q,
                         const int32_t* seq_lens, int batch, const RopeFreq& freq, float qscale, void* abuf,
                         hipStream_t st);
// part[s][M][N] (fp32) = the s-th split of a[M][K] . W^T for a tiled W (rows N,
// contraction K, K a multiple of 256, N of 32); returns the number of splits
// (at most K/256).
int launch_project_gemm(const void* a, const void* w_tiled, float* part, int M, int N, int K, hipStream_t st);
// y[M][N] (bf16) = a[M][K] . W^T for a tiled W (rows N, contraction K), via
// launch_project_gemm's partials summed in split order.
void launch_project(const void* a, const void* w_tiled, float* part, void* y, int M, int N, int K,
                    hipStream_t st);

}  // namespace mla

// The host handle behind the opaque mla_layer of include/mla.h (internal:
// shared by the C ABI's implementation and its native host tests).
#pragma once

#include "../../include/mla.h"
#include "common.hpp"

struct mla_layer {
  mla_config cfg;
  int elem;        // bytes per stored element
  float scale;     // softmax scale actually used
  // folded weights: fragment-tiled for bf16, transposed row-major for fp32
  void* wdkv_t;    // rows n < D, k = d < d_model
  void* wuk_p;     // per head: rows j < d_c, k = i < d_nope
  void* wuv_p;     // per head: rows v < d_v, k = j < d_c
  void* wukt_p;    // bf16: per head, rows i < d_nope, k = j < d_c (expanded path)
  mla::RopeFreq freq;   // rotary frequencies (bf16 layers)
  int num_cus;
  void* wo_p = nullptr;  // output projection, tiled (mla_fold_output)
  int out_form = 0;      // MLA_OUTPUT_UNFOLDED or MLA_OUTPUT_FOLDED once folded
  void* wq_p = nullptr;  // query projection, tiled (mla_fold_query)
  int q_form = 0;        // MLA_QUERY_UNFOLDED or MLA_QUERY_FOLDED once folded
  int attn_rows = 0;     // split-KV rows per workgroup: 0 = by shape, 64 or 128
};


// The append path's one-wave blocks, shared by the append launches and the
// fused launches of a decode step: the GEMM block (bf16 layers) and the
// finish block (sum, rotate, round, scatter).
#pragma once

#include "common.hpp"

namespace mla {

constexpr int kAppendKChunk = 256;   // d_model elements per split

// u^T block (32 row elements x 32 tokens) over one k chunk: token block bx,
// row-element block by, k chunk bz.  The folded W_dkv is the A operand
// (contiguous fragments), the hidden states the B operand; each lane stores 4
// consecutive row elements of one token into part[bz][t][:].
__device__ __forceinline__ void append_gemm_block(const bf16* __restrict__ x,
                                                  const bf16* __restrict__ wdkv,
                                                  float* __restrict__ part, int M, int N, int K,
                                                  int bx, int by, int bz) {
  constexpr int NS = kAppendKChunk / 16;
  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
  const int m0 = bx * 32, nb = by, ks = bz;
  const int t = m0 + l32;
  const bf16* xr = x + (int64_t)min(t, M - 1) * K + ks * kAppendKChunk + 8 * g;
  bf16x8 a[NS], b[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    a[s] = load_fragment(wdkv, nb, ks * NS + s, K, lane);
    b[s] = load_bf16x8(xr + 16 * s);
  }
  f32x16 acc = zero_f32x16();
#pragma unroll
  for (int s = 0; s < NS; ++s) acc = mfma32(a[s], b[s], acc);
  if (t < M) {
    float* out = part + ((int64_t)ks * M + t) * N + nb * 32 + 4 * g;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v = {acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
      *reinterpret_cast<f32x4*>(out + 8 * r4) = v;
    }
  }
}

// The append finish's one-wave block: one lane per element pair (pairs
// 64 py .. 64 py + 63) of new token t's row: sum the k-split partials in a
// fixed order, rotate rope pairs, round, store into the token's page slot.
template <typename T>
__device__ __forceinline__ void append_finish_block(
    const float* __restrict__ part, int ksplits, int T_new, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, T* __restrict__ cache, int page_size, int dc, int dr, float base,
    const RopeFreq& freq, int t, int py) {
  const int D = dc + dr;
  const int p = py * 64 + (threadIdx.x & 63);
  const int n = 2 * p;
  const int64_t stride = (int64_t)T_new * D;
  // the k-split partials first (they depend on nothing), so that their
  // latency overlaps the chain of lookups that finds the token's page slot;
  // up to 32 splits in flight, summed in split order
  const float* src = part + (int64_t)t * D + min(n, D - 2);
  float2 v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j)
    v[j] = j < ksplits ? *reinterpret_cast<const float2*>(src + j * stride) : float2{0.f, 0.f};
  __shared__ CuStage cu_st;
  const int32_t* cu = stage_cu(cu_st, cu_new, batch);
  if (p >= D / 2) return;
  const int b = seq_of_token(cu, batch, t);
  const int pos = prefix_lens[b] + (t - cu[b]);
  const int page = page_table[(int64_t)b * max_pages + pos / page_size];
  T* dst = cache + ((int64_t)page * page_size + pos % page_size) * D;
  float u0 = 0.f, u1 = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    if (j < ksplits) {
      u0 += v[j].x;
      u1 += v[j].y;
    }
  }
  for (int ks = 32; ks < ksplits; ++ks) {
    const float2 w = *reinterpret_cast<const float2*>(src + ks * stride);
    u0 += w.x;
    u1 += w.y;
  }
  if (n >= dc) {
    float c, s;
    if constexpr (sizeof(T) == 2)
      rope_cos_sin_reduced(pos, freq.theta[(n - dc) >> 1], &c, &s);   // bf16: d_rope = 64
    else
      rope_cos_sin(pos, (n - dc) >> 1, dr, base, &c, &s);
    const float r0 = u0 * c - u1 * s;
    const float r1 = u0 * s + u1 * c;
    u0 = r0;
    u1 = r1;
  }
  dst[n] = from_f32<T>(u0);
  dst[n + 1] = from_f32<T>(u1);
}

}  // namespace mla

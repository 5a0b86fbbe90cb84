// The append GEMM's one-wave block (bf16 layers), shared by the append launch
// and the fused append + query-absorb launch of a decode step.
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

}  // namespace mla

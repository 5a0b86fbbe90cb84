// Output projection of the layer, with the value up-projection either kept
// apart or folded into it ("Multi-head Latent Attention and KV Cache
// Compression" (jongkwan.dev), section "The absorption trick and decoupled
// RoPE": the value-side up-projection is absorbed into the output projection
// the same way the key side is absorbed into the query).
//
//   unfolded:  y = concat_h (o_lat_h W_uv_h) . W_o          K = H * d_v
//   folded:    y = concat_h o_lat_h . W_uvo,  W_uvo_h = W_uv_h W_o_h   K = H * d_c
//
// Both are one plain matrix product of the query rows with a weight matrix
// stored fragment-tiled at load (rows = the d_model outputs, contraction
// index k), run by the split-K matrix-core GEMM of the append path and a
// fixed-order reduction of its fp32 partials.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

// W_o [H*dv][dm] -> tiled rows j < dm, k = h*dv + v.  One thread per element.
__global__ void pack_wo_kernel(const bf16* __restrict__ w_o, bf16* __restrict__ out, int K, int dm) {
  const int64_t n = (int64_t)K * dm;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(o % dm), k = (int)(o / dm);   // consecutive threads: consecutive j
    out[tiled_index(j, k, K)] = w_o[(int64_t)k * dm + j];
  }
}

// W_uvo[j][h*dc + c] = sum_v W_uv[c][h*dv + v] W_o[h*dv + v][j], fp32
// accumulation in v order, rounded to bf16, stored tiled (rows j, K = H*dc).
// One thread per element; a one-time fold at load.
__global__ void fold_wuvo_kernel(const bf16* __restrict__ w_uv, const bf16* __restrict__ w_o,
                                 bf16* __restrict__ out, int H, int dc, int dv, int dm) {
  const int K = H * dc;
  const int64_t n = (int64_t)K * dm;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(o % dm), k = (int)(o / dm);   // consecutive threads: consecutive j
    const int h = k / dc, c = k % dc;
    const bf16* a = w_uv + (int64_t)c * H * dv + (int64_t)h * dv;
    const bf16* b = w_o + (int64_t)h * dv * dm + j;
    float acc = 0.f;
    for (int v = 0; v < dv; ++v) acc = fmaf(to_f32(a[v]), to_f32(b[(int64_t)v * dm]), acc);
    out[tiled_index(j, k, K)] = from_f32<bf16>(acc);
  }
}

// y[m][n] = sum over splits s (in order) of part[s][m][n], rounded to bf16.
__global__ void sum_splits_kernel(const float* __restrict__ part, int ks, int M, int N,
                                  bf16* __restrict__ y) {
  const int64_t n = (int64_t)M * N;
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= n) return;
  float acc = 0.f;
  for (int s = 0; s < ks; ++s) acc += part[(int64_t)s * n + o];
  y[o] = from_f32<bf16>(acc);
}

}  // namespace

void launch_fold_output(int form, const void* w_uv, const void* w_o, void* out, int H, int dc, int dv,
                        int dm, hipStream_t st) {
  if (form == 1)
    pack_wo_kernel<<<4096, 256, 0, st>>>((const bf16*)w_o, (bf16*)out, H * dv, dm);
  else
    fold_wuvo_kernel<<<8192, 256, 0, st>>>((const bf16*)w_uv, (const bf16*)w_o, (bf16*)out, H, dc, dv, dm);
}

void launch_project(const void* a, const void* w_tiled, float* part, void* y, int M, int N, int K,
                    hipStream_t st) {
  launch_append_gemm_bf16(a, w_tiled, part, M, N, K, st);
  const int64_t n = (int64_t)M * N;
  sum_splits_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(part, append_ksplits_bf16(K), M, N,
                                                                 (bf16*)y);
}

}  // namespace mla

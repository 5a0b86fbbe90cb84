// Fold: repack the layer's weights once at load into the layouts the decode
// kernels stream ("Multi-head Latent Attention: the KV cache, compressed",
// section "Absorption: the part that makes it free" -- the fold is done once,
// not per step).  Each packed matrix keeps the contraction index contiguous
// so one 16-byte load per lane feeds one matrix-core operand.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

template <typename T>
__global__ void pack_kernel(const T* __restrict__ w_dkv, const T* __restrict__ w_uk,
                            const T* __restrict__ w_uv, T* __restrict__ wdkv_t,
                            T* __restrict__ wuk_p, T* __restrict__ wuv_p, int d_model, int H,
                            int dn, int dv, int dc, int dr) {
  const int64_t D = dc + dr;
  const int64_t n1 = D * d_model;               // wdkv_t
  const int64_t n2 = (int64_t)H * dc * dn;      // wuk_p
  const int64_t n3 = (int64_t)H * dv * dc;      // wuv_p
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n1 + n2 + n3;
       o += (int64_t)gridDim.x * blockDim.x) {
    if (o < n1) {                                // wdkv_t[n][d] = w_dkv[d][n]
      int64_t n = o / d_model, d = o % d_model;
      wdkv_t[o] = w_dkv[d * D + n];
    } else if (o < n1 + n2) {                    // wuk_p[h][j][i] = w_uk[j][h*dn + i]
      int64_t p = o - n1;
      int64_t i = p % dn, j = (p / dn) % dc, h = p / ((int64_t)dn * dc);
      wuk_p[p] = w_uk[j * ((int64_t)H * dn) + h * dn + i];
    } else {                                     // wuv_p[h][v][j] = w_uv[j][h*dv + v]
      int64_t p = o - n1 - n2;
      int64_t j = p % dc, v = (p / dc) % dv, h = p / ((int64_t)dc * dv);
      wuv_p[p] = w_uv[j * ((int64_t)H * dv) + h * dv + v];
    }
  }
}

}  // namespace

void launch_pack(int elem, const void* w_dkv, const void* w_uk, const void* w_uv, void* wdkv_t,
                 void* wuk_p, void* wuv_p, int d_model, int H, int dn, int dv, int dc, int dr,
                 hipStream_t st) {
  const int threads = 256, blocks = 2048;
  if (elem == 2) {
    pack_kernel<bf16><<<blocks, threads, 0, st>>>(
        (const bf16*)w_dkv, (const bf16*)w_uk, (const bf16*)w_uv, (bf16*)wdkv_t, (bf16*)wuk_p,
        (bf16*)wuv_p, d_model, H, dn, dv, dc, dr);
  } else {
    pack_kernel<float><<<blocks, threads, 0, st>>>(
        (const float*)w_dkv, (const float*)w_uk, (const float*)w_uv, (float*)wdkv_t, (float*)wuk_p,
        (float*)wuv_p, d_model, H, dn, dv, dc, dr);
  }
}

}  // namespace mla

// Fold: repack the layer's weights once at load into the layouts the decode
// kernels stream ("Multi-head Latent Attention: the KV cache, compressed",
// section "Absorption: the part that makes it free" -- the fold is done once,
// not per step).
//
// bf16 layers: every matrix is stored fragment-tiled (tiled_index), with the
// contraction index as k:
//   wdkv[n][d]      rows n < d_c + d_rope, k = d < d_model     (append)
//   wuk[h][j][i]    per head, rows j < d_c, k = i < d_nope      (absorb)
//   wuv[h][v][j]    per head, rows v < d_v, k = j < d_c         (output, and
//                   the value expansion of the expanded prefill path)
//   wukt[h][i][j]   per head, rows i < d_nope, k = j < d_c      (key expansion
//                   of the expanded prefill path)
// fp32 layers keep plain row-major transposes with the contraction index
// contiguous (the fp32 kernels read them one element at a time).
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

// One thread per destination element; source reads are scattered, which is
// fine for a one-time repack.
__global__ void pack_bf16_kernel(const bf16* __restrict__ w_dkv, const bf16* __restrict__ w_uk,
                                 const bf16* __restrict__ w_uv, bf16* __restrict__ wdkv,
                                 bf16* __restrict__ wuk, bf16* __restrict__ wuv,
                                 bf16* __restrict__ wukt, int d_model, int H, int dn, int dv, int dc,
                                 int dr) {
  const int D = dc + dr;
  const int64_t n1 = (int64_t)D * d_model;
  const int64_t n2 = (int64_t)H * dc * dn;
  const int64_t n3 = (int64_t)H * dv * dc;
  const int64_t n4 = (int64_t)H * dn * dc;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n1 + n2 + n3 + n4;
       o += (int64_t)gridDim.x * blockDim.x) {
    // invert tiled_index within one matrix of K columns
    auto untile = [](int64_t p, int K, int* row, int* k) {
      const int i = (int)(p & 7), lane = (int)((p >> 3) & 63);
      const int64_t frag = p >> 9;
      const int s = (int)(frag % (K >> 4)), rb = (int)(frag / (K >> 4));
      *row = 32 * rb + (lane & 31);
      *k = 16 * s + 8 * (lane >> 5) + i;
    };
    int row, k;
    if (o < n1) {
      untile(o, d_model, &row, &k);                       // row = n, k = d
      wdkv[o] = w_dkv[(int64_t)k * D + row];
    } else if (o < n1 + n2) {
      const int64_t p = o - n1, per = (int64_t)dc * dn;
      const int h = (int)(p / per);
      untile(p % per, dn, &row, &k);                      // row = j, k = i
      wuk[p] = w_uk[(int64_t)row * H * dn + (int64_t)h * dn + k];
    } else if (o < n1 + n2 + n3) {
      const int64_t p = o - n1 - n2, per = (int64_t)dv * dc;
      const int h = (int)(p / per);
      untile(p % per, dc, &row, &k);                      // row = v, k = j
      wuv[p] = w_uv[(int64_t)k * H * dv + (int64_t)h * dv + row];
    } else {
      const int64_t p = o - n1 - n2 - n3, per = (int64_t)dn * dc;
      const int h = (int)(p / per);
      untile(p % per, dc, &row, &k);                      // row = i, k = j
      wukt[p] = w_uk[(int64_t)k * H * dn + (int64_t)h * dn + row];
    }
  }
}

__global__ void pack_f32_kernel(const float* __restrict__ w_dkv, const float* __restrict__ w_uk,
                                const float* __restrict__ w_uv, float* __restrict__ wdkv_t,
                                float* __restrict__ wuk_p, float* __restrict__ wuv_p, int d_model,
                                int H, int dn, int dv, int dc, int dr) {
  const int64_t D = dc + dr;
  const int64_t n1 = D * d_model;               // wdkv_t[n][d] = w_dkv[d][n]
  const int64_t n2 = (int64_t)H * dc * dn;      // wuk_p[h][j][i] = w_uk[j][h*dn + i]
  const int64_t n3 = (int64_t)H * dv * dc;      // wuv_p[h][v][j] = w_uv[j][h*dv + v]
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n1 + n2 + n3;
       o += (int64_t)gridDim.x * blockDim.x) {
    if (o < n1) {
      int64_t n = o / d_model, d = o % d_model;
      wdkv_t[o] = w_dkv[d * D + n];
    } else if (o < n1 + n2) {
      int64_t p = o - n1;
      int64_t i = p % dn, j = (p / dn) % dc, h = p / ((int64_t)dn * dc);
      wuk_p[p] = w_uk[j * ((int64_t)H * dn) + h * dn + i];
    } else {
      int64_t p = o - n1 - n2;
      int64_t j = p % dc, v = (p / dc) % dv, h = p / ((int64_t)dc * dv);
      wuv_p[p] = w_uv[j * ((int64_t)H * dv) + h * dv + v];
    }
  }
}

}  // namespace

void launch_pack(int elem, const void* w_dkv, const void* w_uk, const void* w_uv, void* wdkv,
                 void* wuk, void* wuv, void* wukt, int d_model, int H, int dn, int dv, int dc,
                 int dr, hipStream_t st) {
  const int threads = 256, blocks = 2048;
  if (elem == 2) {
    pack_bf16_kernel<<<blocks, threads, 0, st>>>(
        (const bf16*)w_dkv, (const bf16*)w_uk, (const bf16*)w_uv, (bf16*)wdkv, (bf16*)wuk,
        (bf16*)wuv, (bf16*)wukt, d_model, H, dn, dv, dc, dr);
  } else {
    pack_f32_kernel<<<blocks, threads, 0, st>>>(
        (const float*)w_dkv, (const float*)w_uk, (const float*)w_uv, (float*)wdkv, (float*)wuk,
        (float*)wuv, d_model, H, dn, dv, dc, dr);
  }
}

}  // namespace mla

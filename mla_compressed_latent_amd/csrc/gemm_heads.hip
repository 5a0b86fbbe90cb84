// Batched per-head GEMMs on either side of the attention: fold each query into
// latent space, and project each head's latent output back out.
//
// "Multi-head Latent Attention and KV Cache Compression" (jongkwan.dev),
// section "The absorption trick and decoupled RoPE": a score q . (W_u c)
// equals (W_u^T q) . c, so the key up-projection moves onto the query, and
// the value up-projection moves onto the output in the same way.  Per head h
// with W_uk_h = W_uk[:, h*d_nope : (h+1)*d_nope]:
//     q_lat[t][h] = W_uk_h q_nope[t][h]              (d_nope -> d_c)
//     out[t][h]   = o_lat[t][h] W_uv_h               (d_c -> d_v)
// The query's rope part is rotated at the token's own position ("Multi-head
// Latent Attention: the KV cache, compressed", section "The code",
// decoupled_score) and appended, giving one d_c + d_rope row per (token, head)
// that is scored against whole cached rows.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

__device__ __forceinline__ int query_position(const int32_t* __restrict__ cu_q,
                                              const int32_t* __restrict__ seq_lens, int batch,
                                              int t) {
  const int b = seq_of_token(cu_q, batch, t);
  return seq_lens[b] - (cu_q[b + 1] - cu_q[b]) + (t - cu_q[b]);
}

// One wave: 32 tokens x 32 latent columns of one head, or (last column block)
// the rotated rope part of 32 tokens of that head.
__global__ __launch_bounds__(64) void absorb_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ wuk_p, bf16* __restrict__ abuf,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int batch, int Tq,
    int H, int dn, int dr, int dc, float base) {
  const int lane = threadIdx.x;
  const int m0 = blockIdx.x * 32, jb = blockIdx.y, h = blockIdx.z;
  const int dq = dn + dr, D = dc + dr;
  if (jb >= dc / 32) {
    // rope part: each extra column block rotates 64 (token, pair) elements
    __shared__ CuStage cu_st;
    const int32_t* cu = stage_cu(cu_st, cu_q, batch);
    const int npair = dr / 2;
    const int idx = (jb - dc / 32) * 64 + lane;
    const int t = m0 + idx / npair, p = idx % npair;
    if (t >= Tq || idx >= 32 * npair) return;
    const int pos = query_position(cu, seq_lens, batch, t);
    const bf16* src = q + ((int64_t)t * H + h) * dq + dn + 2 * p;
    float c, s;
    rope_cos_sin(pos, p, dr, base, &c, &s);
    const float x0 = to_f32(src[0]), x1 = to_f32(src[1]);
    bf16* dst = abuf + ((int64_t)t * H + h) * D + dc + 2 * p;
    dst[0] = from_f32<bf16>(x0 * c - x1 * s);
    dst[1] = from_f32<bf16>(x0 * s + x1 * c);
    return;
  }
  const int j0 = jb * 32;
  const int trow = min(m0 + (lane & 31), Tq - 1);
  const bf16* qa = q + ((int64_t)trow * H + h) * dq + 8 * (lane >> 5);
  const bf16* wb = wuk_p + ((int64_t)h * dc + j0 + (lane & 31)) * dn + 8 * (lane >> 5);
  f32x16 acc = zero_f32x16();
  for (int k = 0; k < dn; k += 64) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool in = k + 16 * s < dn;
      a[s] = in ? load_bf16x8(qa + k + 16 * s) : zero_bf16x8();
      b[s] = in ? load_bf16x8(wb + k + 16 * s) : zero_bf16x8();
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma32(a[s], b[s], acc);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = m0 + acc_row32(r, lane);
    if (t < Tq) abuf[((int64_t)t * H + h) * D + j0 + (lane & 31)] = from_f32<bf16>(acc[r]);
  }
}

__global__ __launch_bounds__(64) void out_proj_bf16_kernel(const bf16* __restrict__ olat,
                                                           const bf16* __restrict__ wuv_p,
                                                           bf16* __restrict__ out, int Tq, int H,
                                                           int dc, int dv) {
  const int lane = threadIdx.x;
  const int m0 = blockIdx.x * 32, v0 = blockIdx.y * 32, h = blockIdx.z;
  const int trow = min(m0 + (lane & 31), Tq - 1);
  const bf16* oa = olat + ((int64_t)trow * H + h) * dc + 8 * (lane >> 5);
  const bf16* wb = wuv_p + ((int64_t)h * dv + v0 + (lane & 31)) * dc + 8 * (lane >> 5);
  f32x16 acc = zero_f32x16();
  for (int k = 0; k < dc; k += 128) {
    bf16x8 a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      a[s] = load_bf16x8(oa + k + 16 * s);
      b[s] = load_bf16x8(wb + k + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma32(a[s], b[s], acc);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = m0 + acc_row32(r, lane);
    if (t < Tq) out[((int64_t)t * H + h) * dv + v0 + (lane & 31)] = from_f32<bf16>(acc[r]);
  }
}

// fp32 layers: one thread per output element.
__global__ void absorb_f32_kernel(const float* __restrict__ q, const float* __restrict__ wuk_p,
                                  float* __restrict__ abuf, const int32_t* __restrict__ cu_q,
                                  const int32_t* __restrict__ seq_lens, int batch, int Tq, int H,
                                  int dn, int dr, int dc, float base) {
  const int per = dc + dr / 2;   // content columns, then rope pairs
  int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= (int64_t)Tq * H * per) return;
  const int j = (int)(o % per);
  const int64_t th = o / per;
  const int h = (int)(th % H), t = (int)(th / H);
  const int dq = dn + dr, D = dc + dr;
  const float* qr = q + th * dq;
  float* dst = abuf + th * D;
  if (j < dc) {
    const float* w = wuk_p + ((int64_t)h * dc + j) * dn;
    float acc = 0.f;
    for (int i = 0; i < dn; ++i) acc = fmaf(qr[i], w[i], acc);
    dst[j] = acc;
  } else {
    const int p = j - dc;
    const int pos = query_position(cu_q, seq_lens, batch, t);
    float c, s;
    rope_cos_sin(pos, p, dr, base, &c, &s);
    const float x0 = qr[dn + 2 * p], x1 = qr[dn + 2 * p + 1];
    dst[dc + 2 * p] = x0 * c - x1 * s;
    dst[dc + 2 * p + 1] = x0 * s + x1 * c;
  }
}

__global__ void out_proj_f32_kernel(const float* __restrict__ olat, const float* __restrict__ wuv_p,
                                    float* __restrict__ out, int Tq, int H, int dc, int dv) {
  int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= (int64_t)Tq * H * dv) return;
  const int v = (int)(o % dv);
  const int64_t th = o / dv;
  const int h = (int)(th % H);
  const float* a = olat + th * dc;
  const float* w = wuv_p + ((int64_t)h * dv + v) * dc;
  float acc = 0.f;
  for (int j = 0; j < dc; ++j) acc = fmaf(a[j], w[j], acc);
  out[o] = acc;
}

}  // namespace

void launch_absorb(int elem, const void* q, const void* wuk_p, void* abuf, const int32_t* cu_q,
                   const int32_t* seq_lens, int batch, int Tq, int H, int dn, int dr, int dc,
                   float base, hipStream_t st) {
  if (elem == 2) {
    dim3 grid((Tq + 31) / 32, dc / 32 + (32 * (dr / 2) + 63) / 64, H);
    absorb_bf16_kernel<<<grid, 64, 0, st>>>((const bf16*)q, (const bf16*)wuk_p, (bf16*)abuf, cu_q,
                                            seq_lens, batch, Tq, H, dn, dr, dc, base);
  } else {
    int64_t n = (int64_t)Tq * H * (dc + dr / 2);
    absorb_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        (const float*)q, (const float*)wuk_p, (float*)abuf, cu_q, seq_lens, batch, Tq, H, dn, dr,
        dc, base);
  }
}

void launch_out_proj(int elem, const void* olat, const void* wuv_p, void* out, int Tq, int H, int dc,
                     int dv, hipStream_t st) {
  if (elem == 2) {
    dim3 grid((Tq + 31) / 32, dv / 32, H);
    out_proj_bf16_kernel<<<grid, 64, 0, st>>>((const bf16*)olat, (const bf16*)wuv_p, (bf16*)out,
                                               Tq, H, dc, dv);
  } else {
    int64_t n = (int64_t)Tq * H * dv;
    out_proj_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        (const float*)olat, (const float*)wuv_p, (float*)out, Tq, H, dc, dv);
  }
}

}  // namespace mla

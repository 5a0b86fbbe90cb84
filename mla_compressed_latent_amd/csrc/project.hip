// Output projection of the layer, with the value up-projection either kept
// apart or folded into it ("Multi-head Latent Attention and KV Cache
// Compression" (jongkwan.dev), section "The absorption trick and decoupled
// RoPE": W_uv can be pre-multiplied into W_o just as W_uk is pre-multiplied
// into the query side).
//
//   unfolded:  y = concat_h (o_lat_h W_uv_h) . W_o          K = H * d_v
//   folded:    y = concat_h o_lat_h . W_uvo,  W_uvo_h = W_uv_h W_o_h   K = H * d_c
//
// Both are one plain matrix product of the query rows with a weight matrix
// stored fragment-tiled at load (rows = the d_model outputs, contraction
// index k), run by a split-K matrix-core GEMM and a fixed-order reduction of
// its fp32 partials.
//
// The queries themselves can come from the layer input the same way, with
// the key up-projection kept apart or folded into the query projection
// ("Multi-head Latent Attention: the KV cache, compressed", section "Store
// the archive, not the files": (x W_q)(c W_uk)^T = x (W_q W_uk^T) c^T, so
// W_abs = W_q W_uk^T is formed once at load):
//
//   unfolded:  q = x . W_q, then the decode's own absorb      N = H * (d_nope + d_rope)
//   folded:    [q_lat | q_rope]_h = x . [W_q_h^nope W_uk_h^T | W_q_h^rope]
//              straight into the attention's query rows         N = H * (d_c + d_rope)
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

// Row-major W [K][N] -> tiled rows j < N, contraction k < K (W_o with K =
// H*dv, N = dm; W_q with K = dm, N = H*(dn + dr)).  One thread per element.
__global__ void pack_tiled_kernel(const bf16* __restrict__ w, bf16* __restrict__ out, int K, int N) {
  const int64_t n = (int64_t)K * N;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(o % N), k = (int)(o / N);   // consecutive threads: consecutive j
    out[tiled_index(j, k, K)] = w[(int64_t)k * N + j];
  }
}

// W_qa rows r = h*D + j (D = dc + dr), contraction k < dm, stored tiled:
//   j <  dc: sum_i W_q[k][h*dq + i] W_uk[j][h*dn + i]  (fp32 in i order, rounded to bf16)
//   j >= dc: W_q[k][h*dq + dn + j - dc]                (the rope columns, copied)
// with dq = dn + dr.  One thread per element; a one-time fold at load.
__global__ void fold_wqa_kernel(const bf16* __restrict__ w_q, const bf16* __restrict__ w_uk,
                                bf16* __restrict__ out, int H, int dn, int dr, int dc, int dm) {
  const int D = dc + dr, dq = dn + dr;
  const int64_t n = (int64_t)H * D * dm;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(o % dm), r = (int)(o / dm);   // consecutive threads: consecutive k
    const int h = r / D, j = r % D;
    const bf16* a = w_q + (int64_t)k * H * dq + (int64_t)h * dq;
    bf16 v;
    if (j < dc) {
      const bf16* b = w_uk + (int64_t)j * H * dn + (int64_t)h * dn;
      float acc = 0.f;
      for (int i = 0; i < dn; ++i) acc = fmaf(to_f32(a[i]), to_f32(b[i]), acc);
      v = from_f32<bf16>(acc);
    } else {
      v = a[dn + j - dc];
    }
    out[tiled_index(r, k, dm)] = v;
  }
}

// The attention's query rows abuf[t][h][0 : D] from the split-K partials of
// x . W_qa (part[s][t][h*D + j]): the splits summed in order, the content
// part multiplied by qscale, each rope pair (2p, 2p+1) rotated by the
// token's position times theta_p and then multiplied by qscale -- the same
// rows the absorb kernel writes from an unfolded query.  One thread per
// (token, head, element pair).
__global__ void query_finish_kernel(const float* __restrict__ part, int ks, int Tq, int H, int dc,
                                    int dr, const int32_t* __restrict__ cu_q,
                                    const int32_t* __restrict__ seq_lens, int batch, RopeFreq freq,
                                    float qscale, bf16* __restrict__ abuf) {
  const int D = dc + dr, P = D / 2;
  const int64_t n = (int64_t)Tq * H * P;
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= n) return;
  const int p = (int)(o % P);
  const int64_t th = o / P;   // t * H + h
  const int t = (int)(th / H);
  const int64_t e = th * D + 2 * p;
  const int64_t stride = (int64_t)Tq * H * D;
  float x0 = 0.f, x1 = 0.f;
  for (int s = 0; s < ks; ++s) {
    const float2 v = *reinterpret_cast<const float2*>(part + s * stride + e);
    x0 += v.x;
    x1 += v.y;
  }
  float y0, y1;
  if (2 * p < dc) {
    y0 = x0 * qscale;
    y1 = x1 * qscale;
  } else {
    const int b = seq_of_token(cu_q, batch, t);
    const int pos = seq_lens[b] - (cu_q[b + 1] - cu_q[b]) + (t - cu_q[b]);
    float c, sn;
    rope_cos_sin_reduced(pos, freq.theta[p - dc / 2], &c, &sn);
    y0 = (x0 * c - x1 * sn) * qscale;
    y1 = (x0 * sn + x1 * c) * qscale;
  }
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r = {from_f32<bf16>(y0), from_f32<bf16>(y1)};
  *reinterpret_cast<bf16x2*>(abuf + e) = r;
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

// part[ks][m][n] = sum over k in the ks-th run of KR consecutive 256-wide k
// chunks of a[m][k] w[n][k]: one wave per (32 rows m, 32 outputs n, run),
// the tiled weight as the A operand (contiguous fragments), a as the B
// operand, one fp32 accumulator carried through the run -- the append GEMM's
// block with KR times fewer split partials to write and sum, for the skinny
// (few query rows) projections whose partials would otherwise rival the
// weight bytes.
template <int KR>
__global__ __launch_bounds__(64) void project_gemm_kernel(const bf16* __restrict__ a, const bf16* __restrict__ w,
                                                          float* __restrict__ part, int M, int N, int K) {
  constexpr int NS = 16;   // fragments per 256-wide chunk
  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
  const int t = blockIdx.x * 32 + l32, nb = blockIdx.y, ks = blockIdx.z;
  const bf16* ar = a + (int64_t)min(t, M - 1) * K + 8 * g;
  f32x16 acc = zero_f32x16();
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    const int kc = ks * KR + r;
    bf16x8 wa[NS], xb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      wa[s] = load_fragment(w, nb, kc * NS + s, K, lane);
      xb[s] = load_bf16x8(ar + kc * 256 + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = mfma32(wa[s], xb[s], acc);
  }
  if (t < M) {
    float* out = part + ((int64_t)ks * M + t) * N + nb * 32 + 4 * g;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v = {acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
      *reinterpret_cast<f32x4*>(out + 8 * r4) = v;
    }
  }
}

// The same product with the activation chunk shared through LDS: four waves
// per workgroup take four consecutive 32-output blocks; per 256-wide k chunk
// the workgroup copies the 32 x 256 activation tile once (coalesced 16-byte
// pieces; rows padded by 16 bytes so the 32 rows of an operand read start 4
// banks apart) and each wave reads its B operands from there, instead of
// every wave fetching the tile through its own 32-row strided loads.  The
// next chunk's weight fragments and activation pieces are loaded while the
// current chunk's products run.  N must be a multiple of 128.
constexpr int kXRow = 256 + 8;   // padded LDS row (elements)

template <int KR>
__global__ __launch_bounds__(256) void project_gemm_lds_kernel(const bf16* __restrict__ a,
                                                               const bf16* __restrict__ w,
                                                               float* __restrict__ part, int M, int N,
                                                               int K) {
  constexpr int NS = 16;
  __shared__ __attribute__((aligned(16))) bf16 xs[32 * kXRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.x * 32, nb = blockIdx.y * 4 + wave, ks = blockIdx.z;
  // activation pieces of this thread: rows (tid + 256 j) / 32, 16-byte column (tid % 32)
  const int prow = tid >> 5, pcol = (tid & 31) * 8;
  auto load_x = [&](int kc, bf16x8 (&dst)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j] = load_bf16x8(a + (int64_t)min(m0 + prow + 8 * j, M - 1) * K + kc * 256 + pcol);
  };
  auto load_w = [&](int kc, bf16x8 (&dst)[NS]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) dst[s] = load_fragment(w, nb, kc * NS + s, K, lane);
  };
  bf16x8 xg[4], wa[NS];
  load_x(ks * KR, xg);
  load_w(ks * KR, wa);
  f32x16 acc = zero_f32x16();
#pragma unroll
  for (int r = 0; r < KR; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<bf16x8*>(&xs[(prow + 8 * j) * kXRow + pcol]) = xg[j];
    __syncthreads();
    bf16x8 wn[NS];
    if (r + 1 < KR) {
      load_x(ks * KR + r + 1, xg);
      load_w(ks * KR + r + 1, wn);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 xb = *reinterpret_cast<const bf16x8*>(&xs[l32 * kXRow + 16 * s + 8 * g]);
      acc = mfma32(wa[s], xb, acc);
    }
    if (r + 1 < KR) {
#pragma unroll
      for (int s = 0; s < NS; ++s) wa[s] = wn[s];
      __syncthreads();
    }
  }
  const int t = m0 + l32;
  if (t < M) {
    float* out = part + ((int64_t)ks * M + t) * N + nb * 32 + 4 * g;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v = {acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
      *reinterpret_cast<f32x4*>(out + 8 * r4) = v;
    }
  }
}

// y[m][n] = sum over splits s (in order) of part[s][m][n], rounded to bf16.
// Four consecutive outputs per thread (N is a multiple of 32): 16-byte loads
// of every split, eight in flight.
__global__ void sum_splits_kernel(const float* __restrict__ part, int ks, int M, int N,
                                  bf16* __restrict__ y) {
  const int64_t n = (int64_t)M * N;
  const int64_t o = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (o >= n) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
  for (int s = 0; s < ks; ++s) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + s * n + o);
    a0 += v[0];
    a1 += v[1];
    a2 += v[2];
    a3 += v[3];
  }
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 r = {from_f32<bf16>(a0), from_f32<bf16>(a1), from_f32<bf16>(a2), from_f32<bf16>(a3)};
  *reinterpret_cast<bf16x4*>(y + o) = r;
}

}  // namespace

void launch_fold_output(int form, const void* w_uv, const void* w_o, void* out, int H, int dc, int dv,
                        int dm, hipStream_t st) {
  if (form == 1)
    pack_tiled_kernel<<<4096, 256, 0, st>>>((const bf16*)w_o, (bf16*)out, H * dv, dm);
  else
    fold_wuvo_kernel<<<8192, 256, 0, st>>>((const bf16*)w_uv, (const bf16*)w_o, (bf16*)out, H, dc, dv, dm);
}

void launch_fold_query(int form, const void* w_q, const void* w_uk, void* out, int H, int dn, int dr,
                       int dc, int dm, hipStream_t st) {
  if (form == 1)
    pack_tiled_kernel<<<4096, 256, 0, st>>>((const bf16*)w_q, (bf16*)out, dm, H * (dn + dr));
  else
    fold_wqa_kernel<<<8192, 256, 0, st>>>((const bf16*)w_q, (const bf16*)w_uk, (bf16*)out, H, dn, dr, dc,
                                          dm);
}

void launch_query_finish(const float* part, int ks, int Tq, int H, int dc, int dr, const int32_t* cu_q,
                         const int32_t* seq_lens, int batch, const RopeFreq& freq, float qscale, void* abuf,
                         hipStream_t st) {
  const int64_t n = (int64_t)Tq * H * ((dc + dr) / 2);
  query_finish_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(part, ks, Tq, H, dc, dr, cu_q, seq_lens,
                                                                   batch, freq, qscale, (bf16*)abuf);
}

int launch_project_gemm(const void* a, const void* w_tiled, float* part, int M, int N, int K, hipStream_t st) {
  // the longest run of k chunks that still leaves about eight waves per
  // compute unit
  const int chunks = K / 256, mb = (M + 31) / 32, nb = N / 32;
  int kr = 1;
  for (int c = 8; c > 1; c /= 2)
    if (chunks % c == 0 && (int64_t)mb * nb * (chunks / c) >= 2048) {
      kr = c;
      break;
    }
  if (nb % 4 == 0) {
    const dim3 grid(mb, nb / 4, chunks / kr);
    switch (kr) {
      case 8: project_gemm_lds_kernel<8><<<grid, 256, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K); break;
      case 4: project_gemm_lds_kernel<4><<<grid, 256, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K); break;
      case 2: project_gemm_lds_kernel<2><<<grid, 256, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K); break;
      default: project_gemm_lds_kernel<1><<<grid, 256, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K);
    }
    return chunks / kr;
  }
  const dim3 grid(mb, nb, chunks / kr);
  switch (kr) {
    case 8: project_gemm_kernel<8><<<grid, 64, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K); break;
    case 4: project_gemm_kernel<4><<<grid, 64, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K); break;
    case 2: project_gemm_kernel<2><<<grid, 64, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K); break;
    default: project_gemm_kernel<1><<<grid, 64, 0, st>>>((const bf16*)a, (const bf16*)w_tiled, part, M, N, K);
  }
  return chunks / kr;
}

void launch_project(const void* a, const void* w_tiled, float* part, void* y, int M, int N, int K,
                    hipStream_t st) {
  const int ks = launch_project_gemm(a, w_tiled, part, M, N, K, st);
  const int64_t n4 = (int64_t)M * N / 4;
  sum_splits_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(part, ks, M, N, (bf16*)y);
}

}  // namespace mla

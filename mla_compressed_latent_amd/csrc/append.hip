// Append: compute the cached row of each new token and write it into its page.
//
// Row of token x at position p ("Multi-head Latent Attention: the KV cache,
// compressed", sections "The one formula" and "The code": the latent
// x W_dkv is the only thing cached; the decoupled rope key is cached already
// rotated, one copy shared by all heads):
//     u = x W_dkv                    (d_c + d_rope wide, fp32 accumulation)
//     row = [ u[:d_c] | rot(u[d_c:], p) ]   rounded to the cache dtype
//
// The GEMM is split along d_model so that a handful of new tokens still
// spreads over the whole chip; the split partials are summed in a fixed
// order by the finishing kernel, so the cache contents are deterministic.
#include "append_gemm.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

// One wave per (32-token block, 32 row elements, k chunk).
__global__ __launch_bounds__(64) void append_gemm_bf16_kernel(const bf16* __restrict__ x,
                                                              const bf16* __restrict__ wdkv,
                                                              float* __restrict__ part, int M,
                                                              int N, int K) {
  append_gemm_block(x, wdkv, part, M, N, K, blockIdx.x, blockIdx.y, blockIdx.z);
}

// fp32 layers: one thread per output element, sequential k order.
__global__ void append_gemm_f32_kernel(const float* __restrict__ x, const float* __restrict__ wt,
                                       float* __restrict__ part, int M, int N, int K) {
  int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= (int64_t)M * N) return;
  int m = (int)(o / N), n = (int)(o % N);
  const float* xr = x + (int64_t)m * K;
  const float* wr = wt + (int64_t)n * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(xr[k], wr[k], acc);
  part[o] = acc;
}

template <typename T>
__global__ __launch_bounds__(64) void append_finish_kernel(
    const float* __restrict__ part, int ksplits, int T_new, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, T* __restrict__ cache, int page_size, int dc, int dr, float base,
    const RopeFreq freq) {
  append_finish_block<T>(part, ksplits, T_new, cu_new, prefix_lens, page_table, max_pages, batch, cache,
                         page_size, dc, dr, base, freq, blockIdx.x, blockIdx.y);
}

// 8-bit float code (OCP E4M3: bias 7, 3 mantissa bits, largest finite 448)
// nearest to x, ties to even; |x| <= 448.  Exponent field 0 holds m * 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a < 0.015625f) {                       // below 2^-6: subnormal codes
    const float m = rintf(a * 512.f);        // exact scaling, round to nearest even
    return sign | (uint32_t)m;               // m == 8 is the smallest normal, code 0x08
  }
  const uint32_t ab = __float_as_uint(a);
  uint32_t E = (ab >> 23) - 120u;            // fp32 exponent (bias 127) -> bias 7
  uint32_t m3 = (ab >> 20) & 7u;
  const uint32_t rem = ab & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  if (m3 == 8u) {
    m3 = 0u;
    ++E;
  }
  return sign | (E << 3) | m3;
}

// FP8 cache rows: one workgroup per new token, thread i owns latent elements
// 2i, 2i+1 (and threads 0..31 also rope pair i).  The row's largest |c| sets
// the scale 2^e, e the smallest integer with max|c| <= 448 * 2^e; the codes
// are c * 2^-e rounded to nearest even; the rope key is rotated and rounded
// to bf16 as in a bf16 cache.
__global__ __launch_bounds__(256) void append_finish_fp8_kernel(
    const float* __restrict__ part, int ksplits, int T_new, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, uint8_t* __restrict__ cache, int page_size, const RopeFreq freq) {
  constexpr int D = 576;
  const int t = blockIdx.x;
  const int i = threadIdx.x;
  const int64_t stride = (int64_t)T_new * D;
  const float* src = part + (int64_t)t * D + 2 * i;
  const float* rsrc = part + (int64_t)t * D + 512 + 2 * (i & 31);
  float u0 = 0.f, u1 = 0.f, r0 = 0.f, r1 = 0.f;
  for (int j = 0; j < ksplits; ++j) {        // split order, as the bf16 path
    const float2 w = *reinterpret_cast<const float2*>(src + j * stride);
    u0 += w.x;
    u1 += w.y;
    if (i < 32) {
      const float2 r = *reinterpret_cast<const float2*>(rsrc + j * stride);
      r0 += r.x;
      r1 += r.y;
    }
  }
  __shared__ CuStage cu_st;
  __shared__ float wmax[4];
  const int32_t* cu = stage_cu(cu_st, cu_new, batch);
  float m = fmaxf(fabsf(u0), fabsf(u1));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((i & 63) == 0) wmax[i >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  int e = 0;
  if (amax > 0.f) {
    int x;
    const float mant = frexpf(amax, &x);     // amax = mant 2^x, mant in [0.5, 1)
    e = mant <= 0.875f ? x - 9 : x - 8;      // 448 = 0.875 2^9
  }
  const int b = seq_of_token(cu, batch, t);
  const int pos = prefix_lens[b] + (t - cu[b]);
  const int page = page_table[(int64_t)b * max_pages + pos / page_size];
  uint8_t* pbase = cache + (int64_t)page * page_size * (kFp8RowBytes + 4);
  uint8_t* row = pbase + (int64_t)(pos % page_size) * kFp8RowBytes;
  const uint32_t c0 = e4m3_code(ldexpf(u0, -e)), c1 = e4m3_code(ldexpf(u1, -e));
  *reinterpret_cast<uint16_t*>(row + 2 * i) = (uint16_t)(c0 | (c1 << 8));
  if (i < 32) {
    float c, s;
    rope_cos_sin_reduced(pos, freq.theta[i], &c, &s);
    bf16* rope = reinterpret_cast<bf16*>(row + 512);
    rope[2 * i] = from_f32<bf16>(r0 * c - r1 * s);
    rope[2 * i + 1] = from_f32<bf16>(r0 * s + r1 * c);
  }
  if (i == 0)
    reinterpret_cast<float*>(pbase + (int64_t)page_size * kFp8RowBytes)[pos % page_size] = ldexpf(1.f, e);
}

}  // namespace

int append_ksplits_bf16(int K) { return K / kAppendKChunk; }

void launch_append_finish_fp8(const float* part, int ksplits, int T, const int32_t* cu_new,
                              const int32_t* prefix_lens, const int32_t* page_table, int max_pages,
                              int batch, void* cache, int page_size, const RopeFreq& freq,
                              hipStream_t st) {
  append_finish_fp8_kernel<<<T, 256, 0, st>>>(part, ksplits, T, cu_new, prefix_lens, page_table,
                                              max_pages, batch, (uint8_t*)cache, page_size, freq);
}

void launch_append_gemm_bf16(const void* x, const void* wdkv, float* part, int M, int N, int K,
                             hipStream_t st) {
  dim3 grid((M + 31) / 32, N / 32, K / kAppendKChunk);
  append_gemm_bf16_kernel<<<grid, 64, 0, st>>>((const bf16*)x, (const bf16*)wdkv, part, M, N, K);
}

void launch_append_gemm_f32(const void* x, const void* wt, float* part, int M, int N, int K,
                            hipStream_t st) {
  int64_t n = (int64_t)M * N;
  append_gemm_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const float*)x,
                                                                      (const float*)wt, part, M,
                                                                      N, K);
}

void launch_append_finish(int elem, const float* part, int ksplits, int T, const int32_t* cu_new,
                          const int32_t* prefix_lens, const int32_t* page_table, int max_pages,
                          int batch, void* cache, int page_size, int dc, int dr, float base,
                          const RopeFreq& freq, hipStream_t st) {
  dim3 grid(T, ((dc + dr) / 2 + 63) / 64);
  if (elem == 2)
    append_finish_kernel<bf16><<<grid, 64, 0, st>>>(part, ksplits, T, cu_new, prefix_lens, page_table,
                                                    max_pages, batch, (bf16*)cache, page_size, dc, dr,
                                                    base, freq);
  else
    append_finish_kernel<float><<<grid, 64, 0, st>>>(part, ksplits, T, cu_new, prefix_lens, page_table,
                                                     max_pages, batch, (float*)cache, page_size, dc,
                                                     dr, base, freq);
}

}  // namespace mla

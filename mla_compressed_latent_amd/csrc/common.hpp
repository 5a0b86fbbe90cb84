// Device-side building blocks shared by the MLA decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ numbers
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// Two floats as a packed bf16 pair (round to nearest even), lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {from_f32<bf16>(lo), from_f32<bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Rotary angle for pair i at position pos, computed in double:
// theta_i = base^(-2i/d_rope), angle = pos * theta_i.  Long positions
// (1e5 and more) need the double product and double sin/cos.
__device__ __forceinline__ void rope_cos_sin(int pos, int pair, int d_rope, float base,
                                             float* c, float* s) {
  double theta = pow(static_cast<double>(base), -2.0 * pair / static_cast<double>(d_rope));
  double ang = static_cast<double>(pos) * theta;
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}

// Rotary frequencies of a bf16 layer (d_rope = 64), computed once on the
// host in double: theta_i = base^(-2i/d_rope).
constexpr int kRopePairs = 32;
struct RopeFreq {
  double theta[kRopePairs];
};

// cos/sin of pos * theta: the angle is formed and reduced modulo 2 pi in
// double (2 pi split into two doubles), and only the reduced angle in
// [-pi, pi] goes through single-precision sincos -- accurate to a few 1e-7
// at positions past 1e5, far below the bf16 rounding of the rotated values.
__device__ __forceinline__ void rope_cos_sin_reduced(int pos, double theta, float* c, float* s) {
  const double a = (double)pos * theta;
  const double k = rint(a * 0.15915494309189535);
  double r = fma(-k, 6.283185307179586, a);
  r = fma(-k, 2.4492935982947064e-16, r);
  sincosf((float)r, s, c);
}

// Index of the sequence that owns flat token t, given cu[0..batch] (cu[0]=0,
// nondecreasing).  Largest b with cu[b] <= t.
__device__ __forceinline__ int seq_of_token(const int32_t* __restrict__ cu, int batch, int t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Token -> sequence lookups for one workgroup: cu[0..batch] is copied to LDS
// once (one coalesced pass) when it fits, so each lookup is a binary search
// in LDS rather than a chain of dependent global loads.
constexpr int kCuStage = 1025;
struct CuStage {
  int32_t v[kCuStage];
};
__device__ __forceinline__ const int32_t* stage_cu(CuStage& st, const int32_t* __restrict__ cu,
                                                   int batch) {
  if (batch + 1 > kCuStage) return cu;
  for (int i = threadIdx.x; i <= batch; i += blockDim.x) st.v[i] = cu[i];
  __syncthreads();
  return st.v;
}

// ---------------------------------------------------------------- matrix core
// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l holds A row (l % 32) and B column (l % 32), eight consecutive k
// values each; both operands use the same k assignment.  Accumulator
// element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row32(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Four consecutive values as fp32 (split partials are fp32 or bf16).
__device__ __forceinline__ f32x4 load4_f32(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4_f32(const bf16* p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
               static_cast<float>(v[3])};
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Fragment-tiled operand layout of a bf16 matrix with R rows (R % 32 == 0)
// and contraction length K (K % 16 == 0), used for the folded weights: the
// fragment of row block rb and k-step s is 64 lanes x 8 elements, lane l
// holding row 32 rb + l % 32 and k = 16 s + 8 (l / 32) + 0..7 -- exactly
// one operand of the 32x32x16 matrix instruction -- so a wave fetches it with
// one contiguous 1 KB read.
__host__ __device__ __forceinline__ int64_t tiled_index(int row, int k, int K) {
  return (((int64_t)(row >> 5) * (K >> 4) + (k >> 4)) * 64 + (row & 31) + 32 * ((k >> 3) & 1)) * 8 +
         (k & 7);
}
__device__ __forceinline__ bf16x8 load_fragment(const bf16* __restrict__ base, int rb, int s, int K,
                                                int lane) {
  return load_bf16x8(base + (((int64_t)rb * (K >> 4) + s) * 64 + lane) * 8);
}

// XCD-aware block order: the hardware deals consecutive workgroup ids to the
// 8 XCDs in turn; this maps them so that consecutive *logical* ids run on
// the same XCD (and share its L2).
__device__ __forceinline__ int xcd_logical_block(int id, int n) {
  constexpr int kXcd = 8;
  int per = (n + kXcd - 1) / kXcd;
  int xcd = id % kXcd, local = id / kXcd;
  // the last XCDs get fewer blocks when n is not a multiple of 8
  int full = n - (per - 1) * kXcd;  // number of XCDs holding `per` blocks
  int base = xcd < full ? xcd * per : full * per + (xcd - full) * (per - 1);
  return base + local;
}

}  // namespace mla

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
#include "append_gemm.hpp"
#include "attn_tile.hpp"
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

constexpr int kAbsorbTokBlocks = 8;   // 32-token blocks one absorb wave handles
constexpr int kRopeTok = 4;       // query tokens per rope workgroup
constexpr int kRopeHeads = 16;    // heads per rope workgroup

__device__ __forceinline__ void store_bf16x4(bf16* dst, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = {from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c), from_f32<bf16>(d)};
  *reinterpret_cast<bf16x4*>(dst) = v;
}

// q_lat^T block = W_uk_h^T (32 latent rows x d_nope) . q_nope^T (d_nope x 32
// tokens): the folded weight is the A operand, streamed as contiguous
// fragments; the 32 query rows are the B operand.  One wave per (head, JB
// blocks of 32 latent columns, up to kAbsorbTokBlocks token blocks): its
// weight fragments stay in registers while the token blocks stream past, so
// W_uk is read about once per step however many query tokens there are.
// The 32 x JB*32 output block goes through LDS so that it leaves as whole
// JB*64-byte row segments (16-byte stores, JB*4 lanes per row) instead of
// 8-byte pieces of 32 rows per store (measured on the DeepSeek-V2 shape,
// 32 tokens: 7.2 -> 5.1 us for the W_uk stream).  The stored score
// operand (q_lat and the rotated rope part) is pre-multiplied by qscale =
// softmax scale * log2(e), so the attention kernel's scores come out in log2
// units.
//
// Workgroups past the GEMM blocks rotate the rope part of the queries: one
// per (sequence, block of kRopeTok of its query tokens, block of kRopeHeads
// heads), so each angle is computed once and applied to every head of the
// block.  Lane l handles pair l % 32 (d_rope = 64) for heads of parity l / 32.
template <int NS, int JB>   // d_nope / 16, 32-column blocks per wave (held in registers)
__device__ __forceinline__ void absorb_block(
    const bf16* __restrict__ q, const bf16* __restrict__ wuk, bf16* __restrict__ abuf,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int Tq, int H, int dr,
    int dc, int gemm_blocks, int TC, const RopeFreq& freq, float qscale, int bid) {
  constexpr int dn = NS * 16;
  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
  if (bid >= gemm_blocks) {
    const int p = l32, hpar = g;
    const int HG = (H + kRopeHeads - 1) / kRopeHeads;
    const int rid = bid - gemm_blocks;
    const int hg = rid % HG, tc = (rid / HG) % TC, b = rid / (HG * TC);
    const int q0 = cu_q[b], Lq = cu_q[b + 1] - q0, L = seq_lens[b];
    const int dq = dn + dr, D = dc + dr;
    const double theta = freq.theta[p];
    for (int i = tc * kRopeTok; i < min(Lq, (tc + 1) * kRopeTok); ++i) {
      const int64_t t = q0 + i;
      uint32_t v[kRopeHeads / 2];
#pragma unroll
      for (int m = 0; m < kRopeHeads / 2; ++m) {
        const int h = hg * kRopeHeads + hpar + 2 * m;
        if (h < H) v[m] = *reinterpret_cast<const uint32_t*>(q + (t * H + h) * dq + dn + 2 * p);
      }
      float c, sn;
      rope_cos_sin_reduced(L - Lq + i, theta, &c, &sn);
#pragma unroll
      for (int m = 0; m < kRopeHeads / 2; ++m) {
        const int h = hg * kRopeHeads + hpar + 2 * m;
        if (h >= H) continue;
        const float x0 = __uint_as_float(v[m] << 16), x1 = __uint_as_float(v[m] & 0xffff0000u);
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 r = {from_f32<bf16>((x0 * c - x1 * sn) * qscale), from_f32<bf16>((x0 * sn + x1 * c) * qscale)};
        *reinterpret_cast<bf16x2*>(abuf + (t * H + h) * D + dc + 2 * p) = r;
      }
    }
    return;
  }
  const int JG = dc / 32 / JB;
  const int ntb = (Tq + 31) / 32;
  const int TBW = min(ntb, kAbsorbTokBlocks);   // token blocks per wave
  const int id = bid;
  const int jg = id % JG, h = (id / JG) % H, tbg = id / (JG * H);
  const int dq = dn + dr, D = dc + dr;
  const bf16* wh = wuk + (int64_t)h * dc * dn;
  __shared__ __attribute__((aligned(16))) bf16 ost[32][JB * 32 + 8];
  bf16x8 wa[JB][NS];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int s = 0; s < NS; ++s) wa[jb][s] = load_fragment(wh, jg * JB + jb, s, dn, lane);
  const int tb_end = min(ntb, (tbg + 1) * TBW);
  auto load_q = [&](int tb, bf16x8 (&dst)[NS]) {
    const bf16* qrow = q + ((int64_t)min(tb * 32 + l32, Tq - 1) * H + h) * dq + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) dst[s] = load_bf16x8(qrow + 16 * s);
  };
  auto compute = [&](int tb, const bf16x8 (&bq)[NS]) {
    // acc[4 r4 + e] is latent column jb*32 + 8 r4 + 4 g + e of token row l32
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      f32x16 acc = zero_f32x16();
#pragma unroll
      for (int s = 0; s < NS; ++s) acc = mfma32(wa[jb][s], bq[s], acc);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store_bf16x4(&ost[l32][jb * 32 + 8 * r4 + 4 * g], acc[4 * r4] * qscale, acc[4 * r4 + 1] * qscale,
                     acc[4 * r4 + 2] * qscale, acc[4 * r4 + 3] * qscale);
    }
    __syncthreads();
    constexpr int kLanesPerRow = JB * 4, kRowsPerStore = 64 / kLanesPerRow;
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += kRowsPerStore) {
      const int r = r0 + lane / kLanesPerRow, c = (lane % kLanesPerRow) * 8;
      const int t = tb * 32 + r;
      if (t < Tq)
        *reinterpret_cast<bf16x8*>(abuf + ((int64_t)t * H + h) * D + jg * JB * 32 + c) =
            *reinterpret_cast<const bf16x8*>(&ost[r][c]);
    }
    __syncthreads();   // the next token block reuses ost
  };
  // ping-pong over two statically indexed query buffers
  bf16x8 qa[NS], qb[NS];
  load_q(tbg * TBW, qa);
  for (int tb = tbg * TBW; tb < tb_end; tb += 2) {
    if (tb + 1 < tb_end) load_q(tb + 1, qb);
    compute(tb, qa);
    if (tb + 1 < tb_end) {
      if (tb + 2 < tb_end) load_q(tb + 2, qa);
      compute(tb + 1, qb);
    }
  }
}

template <int NS, int JB>
__global__ __launch_bounds__(64) void absorb_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ wuk, bf16* __restrict__ abuf,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int Tq, int H, int dr,
    int dc, int gemm_blocks, int TC, const RopeFreq freq, float qscale) {
  absorb_block<NS, JB>(q, wuk, abuf, cu_q, seq_lens, Tq, H, dr, dc, gemm_blocks, TC, freq, qscale,
                       blockIdx.x);
}

// A decode step's two independent weight-streaming GEMMs in one launch: the
// append GEMM of the new tokens' rows (blocks [0, app_blocks), token blocks
// fastest, then row-element blocks, then k chunks) and the query absorb with
// its rope rotation (the rest).  Both are one-wave blocks; the absorb, the
// longer of the two, hides the append behind it.
template <int NS, int JB>
__global__ __launch_bounds__(64) void absorb_append_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ wuk, bf16* __restrict__ abuf,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int Tq, int H, int dr,
    int dc, int gemm_blocks, int TC, const RopeFreq freq, float qscale, const bf16* __restrict__ x,
    const bf16* __restrict__ wdkv, float* __restrict__ part, int M, int N, int K, int app_blocks) {
  const int bid = blockIdx.x;
  if (bid < app_blocks) {
    const int MB = (M + 31) / 32, NB = N / 32;
    append_gemm_block(x, wdkv, part, M, N, K, bid % MB, (bid / MB) % NB, bid / (MB * NB));
    return;
  }
  absorb_block<NS, JB>(q, wuk, abuf, cu_q, seq_lens, Tq, H, dr, dc, gemm_blocks, TC, freq, qscale,
                       bid - app_blocks);
}

// The query absorb with its rope rotation and the append finish in one
// launch (the append GEMM ran in the launch before): finish blocks first
// (new token bid / fin_py, pair block bid % fin_py, for bid < fin_blocks),
// then the absorb blocks.  The finish reads only the GEMM's partials and
// writes only the new rows; the absorb reads only the queries and W_uk: the
// short finish runs under the longer absorb.
template <int NS, int JB>
__global__ __launch_bounds__(64) void absorb_finish_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ wuk, bf16* __restrict__ abuf,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int Tq, int H, int dr,
    int dc, int gemm_blocks, int TC, const RopeFreq freq, float qscale, const float* __restrict__ part,
    int ksplits, int T_new, const int32_t* __restrict__ cu_new, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ page_table, int max_pages, int batch, bf16* __restrict__ cache,
    int page_size, int fin_py, int fin_blocks) {
  const int bid = blockIdx.x;
  if (bid < fin_blocks) {
    append_finish_block<bf16>(part, ksplits, T_new, cu_new, prefix_lens, page_table, max_pages, batch, cache,
                              page_size, dc, dr, 0.f, freq, bid / fin_py, bid % fin_py);
    return;
  }
  absorb_block<NS, JB>(q, wuk, abuf, cu_q, seq_lens, Tq, H, dr, dc, gemm_blocks, TC, freq, qscale,
                       bid - fin_blocks);
}

// out^T block = W_uv_h^T (32 value rows x d_c) . o_lat^T (d_c x 32 tokens).
// One wave per (32-token block, head, 32 value columns); the 32 k-steps of
// both operands stream in groups of 8, two groups in flight.
__global__ __launch_bounds__(64) void out_proj_bf16_kernel(const bf16* __restrict__ olat,
                                                           const bf16* __restrict__ wuv,
                                                           bf16* __restrict__ out, int Tq, int H,
                                                           int dv) {
  constexpr int kDc = 512, NS = kDc / 16, kGrp = 8, NG = NS / kGrp;
  const int lane = threadIdx.x, g = lane >> 5, l32 = lane & 31;
  const int VB = dv / 32;
  const int id = blockIdx.x;
  const int vb = id % VB, h = (id / VB) % H, tb = id / (VB * H);
  const int t = tb * 32 + l32;
  const bf16* orow = olat + ((int64_t)min(t, Tq - 1) * H + h) * kDc + 8 * g;
  const bf16* wh = wuv + (int64_t)h * dv * kDc;
  bf16x8 a[2][kGrp], b[2][kGrp];
  auto load_group = [&](int grp, int slot) {
#pragma unroll
    for (int u = 0; u < kGrp; ++u) {
      a[slot][u] = load_fragment(wh, vb, grp * kGrp + u, kDc, lane);
      b[slot][u] = load_bf16x8(orow + 16 * (grp * kGrp + u));
    }
  };
  load_group(0, 0);
  load_group(1, 1);
  f32x16 acc = zero_f32x16();
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
    for (int u = 0; u < kGrp; ++u) acc = mfma32(a[grp & 1][u], b[grp & 1][u], acc);
    if (grp + 2 < NG) load_group(grp + 2, grp & 1);
  }
  if (t < Tq) {
    bf16* dst = out + ((int64_t)t * H + h) * dv + vb * 32 + 4 * g;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      store_bf16x4(dst + 8 * r4, acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]);
  }
}

// Split combine fused with the output projection (bf16 layers).  One
// workgroup of 8 waves per (TB query tokens, head), TB in {32, 16, 8, 4}
// chosen by the launcher so that the grid covers the chip:
//   1. per row: weights w_s = 2^(lse_s - max lse) over the splits that hold
//      part of the row's sequence, and 1 / sum w_s (all lse loads of the
//      block issued at once);
//   2. o_lat rows = sum_s w_s O_s / sum w_s (normalised partials), rounded to
//      bf16 into LDS; each thread keeps 16 row-split loads of 16 bytes in
//      flight, the first 16 issued before step 1's lse loads;
//   3. out^T = W_uv_h^T . o_lat^T on the matrix core, waves 0..3 taking value
//      column blocks w, w + 4, ...; the B operand comes from LDS (columns past
//      TB hold stale values and are never stored).  The A operand of a wave's
//      first block: k-steps 0..15 loaded into registers at the start, 16..31
//      copied HBM -> LDS at the start by wave w + 4 (otherwise idle then), so
//      the matrix loop waits on no global load.
// Splits past a row's sequence were never written: their weight is zero and
// their (arbitrary) values are never added.
constexpr int kCombThreads = 512;
constexpr int kCombRowPad = 8;   // bf16 pad per LDS row of o_lat

// E consecutive elements of a bf16 split partial row, loaded as one vector
// (16 bytes, or 8 in blocks of 4 tokens) and read as floats.
template <typename P, int E> struct PartVec;
template <> struct PartVec<bf16, 4> {
  typedef __bf16 T __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ T load(const bf16* p) { return *reinterpret_cast<const T*>(p); }
  static __device__ __forceinline__ float get(const T& v, int e) { return static_cast<float>(v[e]); }
};
template <> struct PartVec<bf16, 8> {
  typedef bf16x8 T;
  static __device__ __forceinline__ T load(const bf16* p) { return *reinterpret_cast<const T*>(p); }
  static __device__ __forceinline__ float get(const T& v, int e) { return static_cast<float>(v[e]); }
};

template <int TB, typename P>
__global__ __launch_bounds__(kCombThreads) void combine_out_bf16_kernel(
    const P* __restrict__ opart, const float* __restrict__ lse, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const bf16* __restrict__ wuv, bf16* __restrict__ out,
    int batch, int Tq, int H, int dv, int chunk, int S_max) {
  static_assert(TB == 32 || TB == 16 || TB == 8 || TB == 4, "token block");
  constexpr int kDc = 512;
  __shared__ CuStage cu_st;
  __shared__ float w_s[kCombineMaxSplits][TB];
  __shared__ float inv_s[TB];
  __shared__ int sb_s[TB];
  __shared__ __attribute__((aligned(16))) bf16 ob[32][kDc + kCombRowPad];
  constexpr int kGrp = 8;
  __shared__ __attribute__((aligned(1024))) bf16 wsec[4][2 * kGrp * 512];   // 16 fragments per wave
  const int tid = threadIdx.x;
  const int h = blockIdx.x % H, tb = blockIdx.x / H;
  const int64_t rows_total = (int64_t)Tq * H;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;

  // W_uv fragments of the first value-column block of waves 0..3, loaded
  // first so that their latency hides under the combine
  const bf16* wh = wuv + (int64_t)h * dv * kDc;
  bf16x8 a[2][kGrp];
  if (wave < 4 && wave < dv / 32) {
#pragma unroll
    for (int u = 0; u < kGrp; ++u) {
      a[0][u] = load_fragment(wh, wave, u, kDc, lane);
      a[1][u] = load_fragment(wh, wave, kGrp + u, kDc, lane);
    }
  }
  const int wsel = __builtin_amdgcn_readfirstlane(wave - 4);
  const bool copies_half = wave >= 4 && wsel < dv / 32;
  if (copies_half) {
    const uint32_t dst = lds_address(&wsec[wsel][0]);
#pragma unroll
    for (int u = 0; u < 2 * kGrp; ++u)
      dma16(wh + ((int64_t)wsel * (kDc / 16) + 2 * kGrp + u) * 64 * 8, (uint32_t)lane * 16u, dst + u * 1024);
  }

  // This thread's partial rows and the block's log2-sum-exps.  The lse loads
  // are issued before the number of splits each row's sequence has is known
  // (the workspace holds S_max splits of every row, so they stay in bounds;
  // splits past a sequence's end hold stale values that the weights below
  // mask); the partial rows are loaded only for splits the sequence has.
  // Each thread takes kE consecutive elements (16 bytes of partial) of rows
  // r0, r0 + kGroups, ...
  constexpr int kE = (sizeof(P) == 2 && TB >= 8) ? 8 : 4;
  constexpr int kThrRow = kDc / kE;                    // threads per row
  constexpr int kGroups = kCombThreads / kThrRow;      // rows in flight at once
  constexpr int kRows = TB / kGroups;                  // rows per thread
  constexpr int kSp = 16 / kRows;                      // splits per round of loads
  typedef PartVec<P, kE> PV;
  const int j = kE * (tid % kThrRow), r0 = tid / kThrRow;
  float oacc[kRows][kE];
  const P* src[kRows];
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
#pragma unroll
    for (int e = 0; e < kE; ++e) oacc[u][e] = 0.f;
    const int t = min(tb * TB + r0 + kGroups * u, Tq - 1);   // rows past Tq read a valid row, weight 0
    src[u] = opart + ((int64_t)t * H + h) * kDc + j;
  }
  typename PV::T v[kSp][kRows];

  constexpr int kLseTot = kCombineMaxSplits * TB;   // (split, row) pairs
  constexpr int kLsePerThread = (kLseTot + kCombThreads - 1) / kCombThreads;
  float x[kLsePerThread];
#pragma unroll
  for (int u = 0; u < kLsePerThread; ++u) {
    const int k = tid + kCombThreads * u, sp = k / TB, r = k % TB;
    const int t = min(tb * TB + r, Tq - 1);
    x[u] = (k < kLseTot && sp < S_max) ? lse[sp * rows_total + (int64_t)t * H + h] : -INFINITY;
  }

  const int32_t* cu = stage_cu(cu_st, cu_q, batch);
  if (tid < TB) {
    const int t = tb * TB + tid;
    int sb = 0;
    if (t < Tq) sb = (seq_lens[seq_of_token(cu, batch, t)] + chunk - 1) / chunk;
    sb_s[tid] = sb;
  }
  __syncthreads();
  // splits a row's sequence has (the rows of one thread are the same for
  // the whole wave, so these guards never diverge)
  int sb[kRows], smax = 0;
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    sb[u] = sb_s[r0 + kGroups * u];
    smax = max(smax, sb[u]);
  }
  auto load_round = [&](int sp0) {
#pragma unroll
    for (int d = 0; d < kSp; ++d)
#pragma unroll
      for (int u = 0; u < kRows; ++u)
        if (sp0 + d < sb[u])
          v[d][u] = PV::load(src[u] + (sp0 + d) * rows_total * kDc);
  };
  load_round(0);
#pragma unroll
  for (int u = 0; u < kLsePerThread; ++u) {
    const int k = tid + kCombThreads * u, sp = k / TB, r = k % TB;
    if (k < kLseTot && sp < S_max) w_s[sp][r] = sp < sb_s[r] ? x[u] : -INFINITY;
  }
  __syncthreads();
  if (tid < TB) {
    float m = -INFINITY;
    for (int sp = 0; sp < S_max; ++sp) m = fmaxf(m, w_s[sp][tid]);
    float sum = 0.f;
    for (int sp = 0; sp < S_max; ++sp) {
      const float x = w_s[sp][tid];
      const float w = (x == -INFINITY) ? 0.f : exp2f(x - m);
      w_s[sp][tid] = w;
      sum += w;
    }
    inv_s[tid] = sum > 0.f ? 1.f / sum : 0.f;
  }
  __syncthreads();

  {
    for (int sp0 = 0; sp0 < smax; sp0 += kSp) {
      if (sp0 > 0) load_round(sp0);
#pragma unroll
      for (int d = 0; d < kSp; ++d)
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
          const float w = (sp0 + d < sb[u]) ? w_s[sp0 + d][r0 + kGroups * u] : 0.f;
          if (w != 0.f) {
#pragma unroll
            for (int e = 0; e < kE; ++e) oacc[u][e] += w * PV::get(v[d][u], e);
          }
        }
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int r = r0 + kGroups * u;
      const float inv = inv_s[r];
#pragma unroll
      for (int e = 0; e < kE; e += 4) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 o = {from_f32<bf16>(oacc[u][e] * inv), from_f32<bf16>(oacc[u][e + 1] * inv),
                    from_f32<bf16>(oacc[u][e + 2] * inv), from_f32<bf16>(oacc[u][e + 3] * inv)};
        *reinterpret_cast<bf16x4*>(&ob[r][j + e]) = o;
      }
    }
  }
  if (copies_half) wait_vmcnt<0>();   // the copied half-block is in LDS
  __syncthreads();

  if (wave >= 4) return;
  const int t = tb * TB + l32;
  for (int vb = wave; vb < dv / 32; vb += 4) {
    constexpr int NS = kDc / 16;
    f32x16 acc = zero_f32x16();
    if (vb != wave) {
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        a[0][u] = load_fragment(wh, vb, u, kDc, lane);
        a[1][u] = load_fragment(wh, vb, kGrp + u, kDc, lane);
      }
    }
#pragma unroll
    for (int grp = 0; grp < NS / kGrp; ++grp) {
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        const int sk = grp * kGrp + u;
        const bf16x8 bo = *reinterpret_cast<const bf16x8*>(&ob[l32][16 * sk + 8 * g]);
        acc = mfma32(a[grp & 1][u], bo, acc);
      }
      if (grp + 2 < NS / kGrp) {
        if (vb == wave) {   // k-steps 16..31 of the first block: from LDS
#pragma unroll
          for (int u = 0; u < kGrp; ++u)
            a[grp & 1][u] = *reinterpret_cast<const bf16x8*>(&wsec[wave][((grp * kGrp + u) * 64 + lane) * 8]);
        } else {
#pragma unroll
          for (int u = 0; u < kGrp; ++u)
            a[grp & 1][u] = load_fragment(wh, vb, (grp + 2) * kGrp + u, kDc, lane);
        }
      }
    }
    if (l32 < TB && t < Tq) {
      bf16* dst = out + ((int64_t)t * H + h) * dv + vb * 32 + 4 * g;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store_bf16x4(dst + 8 * r4, acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]);
    }
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

namespace {
// Grid of the bf16 absorb: GEMM waves, then rope workgroups.
struct AbsorbGrid {
  int jb;            // 32-column weight blocks per wave
  int gemm_blocks;   // GEMM waves
  int TC;            // rope workgroups per sequence and head block
  int blocks;        // total
};
AbsorbGrid absorb_grid(int batch, int Tq, int max_q_len, int H, int dn, int dc) {
  AbsorbGrid a;
  const int ntb = (Tq + 31) / 32;
  const int tbw = ntb < kAbsorbTokBlocks ? ntb : kAbsorbTokBlocks;
  // weight blocks per wave: 4 (2 when d_nope > 128) amortise the weight
  // registers over many token blocks
  a.jb = dn / 16 <= 8 ? 4 : 2;
  a.gemm_blocks = ((ntb + tbw - 1) / tbw) * H * (dc / 32 / a.jb);
  a.TC = (max_q_len + kRopeTok - 1) / kRopeTok;
  const int HG = (H + kRopeHeads - 1) / kRopeHeads;
  a.blocks = a.gemm_blocks + batch * a.TC * HG;
  return a;
}
}  // namespace

void launch_absorb_append(const void* q, const void* wuk, void* abuf, const int32_t* cu_q,
                          const int32_t* seq_lens, int batch, int Tq, int max_q_len, int H, int dn,
                          int dr, int dc, const RopeFreq& freq, float qscale, const void* x,
                          const void* wdkv, float* part, int M, int N, int K, hipStream_t st) {
  const AbsorbGrid a = absorb_grid(batch, Tq, max_q_len, H, dn, dc);
  const int gemm_blocks = a.gemm_blocks, TC = a.TC;
  const int app_blocks = ((M + 31) / 32) * (N / 32) * (K / kAppendKChunk);
  const unsigned blocks = (unsigned)(app_blocks + a.blocks);
  switch (dn / 16 * 8 + a.jb) {
#define MLA_FUSED_CASE(NS, JB)                                                                     \
  case NS * 8 + JB:                                                                                \
    absorb_append_bf16_kernel<NS, JB><<<blocks, 64, 0, st>>>(                                      \
        (const bf16*)q, (const bf16*)wuk, (bf16*)abuf, cu_q, seq_lens, Tq, H, dr, dc, gemm_blocks, \
        TC, freq, qscale, (const bf16*)x, (const bf16*)wdkv, part, M, N, K, app_blocks);           \
    break;
    MLA_FUSED_CASE(2, 4) MLA_FUSED_CASE(4, 4) MLA_FUSED_CASE(6, 4) MLA_FUSED_CASE(8, 4)
    MLA_FUSED_CASE(10, 2) MLA_FUSED_CASE(12, 2) MLA_FUSED_CASE(14, 2) MLA_FUSED_CASE(16, 2)
#undef MLA_FUSED_CASE
    default: break;   // excluded by the config check
  }
}

void launch_absorb_finish(const void* q, const void* wuk, void* abuf, const int32_t* cu_q,
                          const int32_t* seq_lens, int batch, int Tq, int max_q_len, int H, int dn,
                          int dr, int dc, const RopeFreq& freq, float qscale, const float* part,
                          int ksplits, int T_new, const int32_t* cu_new, const int32_t* prefix_lens,
                          const int32_t* page_table, int max_pages, void* cache, int page_size,
                          hipStream_t st) {
  const AbsorbGrid a = absorb_grid(batch, Tq, max_q_len, H, dn, dc);
  const int gemm_blocks = a.gemm_blocks, TC = a.TC;
  const int fin_py = ((dc + dr) / 2 + 63) / 64;
  const int fin_blocks = T_new * fin_py;
  const unsigned blocks = (unsigned)(fin_blocks + a.blocks);
  switch (dn / 16 * 8 + a.jb) {
#define MLA_FIN_CASE(NS, JB)                                                                        \
  case NS * 8 + JB:                                                                                 \
    absorb_finish_bf16_kernel<NS, JB><<<blocks, 64, 0, st>>>(                                       \
        (const bf16*)q, (const bf16*)wuk, (bf16*)abuf, cu_q, seq_lens, Tq, H, dr, dc, gemm_blocks,  \
        TC, freq, qscale, part, ksplits, T_new, cu_new, prefix_lens, page_table, max_pages, batch,  \
        (bf16*)cache, page_size, fin_py, fin_blocks);                                               \
    break;
    MLA_FIN_CASE(2, 4) MLA_FIN_CASE(4, 4) MLA_FIN_CASE(6, 4) MLA_FIN_CASE(8, 4)
    MLA_FIN_CASE(10, 2) MLA_FIN_CASE(12, 2) MLA_FIN_CASE(14, 2) MLA_FIN_CASE(16, 2)
#undef MLA_FIN_CASE
    default: break;   // excluded by the config check
  }
}

void launch_absorb(int elem, const void* q, const void* wuk, void* abuf, const int32_t* cu_q,
                   const int32_t* seq_lens, int batch, int Tq, int max_q_len, int H, int dn, int dr,
                   int dc, float base, const RopeFreq& freq, float qscale, hipStream_t st) {
  if (elem == 2) {
    const AbsorbGrid a = absorb_grid(batch, Tq, max_q_len, H, dn, dc);
    const int gemm_blocks = a.gemm_blocks, TC = a.TC;
    const unsigned blocks = (unsigned)a.blocks;
    switch (dn / 16 * 8 + a.jb) {
#define MLA_ABSORB_CASE(NS, JB)                                                                    \
  case NS * 8 + JB:                                                                                \
    absorb_bf16_kernel<NS, JB><<<blocks, 64, 0, st>>>((const bf16*)q, (const bf16*)wuk,           \
                                                      (bf16*)abuf, cu_q, seq_lens, Tq, H, dr, dc, \
                                                      gemm_blocks, TC, freq, qscale);             \
    break;
      MLA_ABSORB_CASE(2, 4) MLA_ABSORB_CASE(4, 4) MLA_ABSORB_CASE(6, 4) MLA_ABSORB_CASE(8, 4)
      MLA_ABSORB_CASE(10, 2) MLA_ABSORB_CASE(12, 2) MLA_ABSORB_CASE(14, 2) MLA_ABSORB_CASE(16, 2)
#undef MLA_ABSORB_CASE
      default: break;   // excluded by the config check
    }
  } else {
    int64_t n = (int64_t)Tq * H * (dc + dr / 2);
    absorb_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        (const float*)q, (const float*)wuk, (float*)abuf, cu_q, seq_lens, batch, Tq, H, dn, dr,
        dc, base);
  }
}

void launch_out_proj(int elem, const void* olat, const void* wuv, void* out, int Tq, int H, int dc,
                     int dv, hipStream_t st) {
  if (elem == 2) {
    const unsigned blocks = (unsigned)(((Tq + 31) / 32) * H * (dv / 32));
    out_proj_bf16_kernel<<<blocks, 64, 0, st>>>((const bf16*)olat, (const bf16*)wuv, (bf16*)out, Tq,
                                                H, dv);
  } else {
    int64_t n = (int64_t)Tq * H * dv;
    out_proj_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        (const float*)olat, (const float*)wuv, (float*)out, Tq, H, dc, dv);
  }
}

void launch_combine_out(const SplitPlan& plan, const void* opart, const float* lse,
                        const int32_t* cu_q, const int32_t* seq_lens, const void* wuv, void* out,
                        int batch, int Tq, int H, int dv, int num_cus, hipStream_t st) {
  // the largest token block that still gives every compute unit a workgroup
  int TB = 32;
  while (TB > 4 && (int64_t)((Tq + TB - 1) / TB) * H < num_cus) TB /= 2;
  const unsigned blocks = (unsigned)(((Tq + TB - 1) / TB) * H);
  switch (TB) {
#define MLA_COMBINE_CASE(N)                                                                    \
  case N:                                                                                      \
    combine_out_bf16_kernel<N, bf16><<<blocks, kCombThreads, 0, st>>>(                         \
        (const bf16*)opart, lse, cu_q, seq_lens, (const bf16*)wuv, (bf16*)out, batch, Tq, H, dv, \
        plan.chunk, plan.S_max);                                                               \
    break;
    MLA_COMBINE_CASE(32) MLA_COMBINE_CASE(16) MLA_COMBINE_CASE(8) MLA_COMBINE_CASE(4)
#undef MLA_COMBINE_CASE
    default: break;
  }
}

}  // namespace mla

// Split-KV attention over the paged latent cache, and the split combine.
//
// Every head scores the SAME cached row [c | k_rope] ("Multi-head Latent
// Attention: the KV cache, compressed", section "The one formula": the latent
// is shared across every head), so for one sequence the step is a dense
// contraction with the (query, head) rows as one dimension:
//     S[row][t]   = scale * A[row] . cache[t]          (K = d_c + d_rope)
//     O[row][:]  += softmax_t(S) cache[t][:d_c]        (K = tokens)
// which is "still softmax(Q K^T / sqrt d) V with K factored" (section
// "Absorption: the part that makes it free").  Each workgroup takes one
// chunk of one sequence's tokens ("split"), keeps a running max and sum per
// row (online softmax), and leaves a normalised partial O and its log-sum-exp;
// the combine kernel merges the splits.
//
// bf16 path (d_c = 512, d_rope = 64), per workgroup of 4 waves:
//   * a 32-token tile of cached rows is copied HBM -> LDS by the LDS-DMA path
//     (global_load_lds, 16 B per lane), NBUF tiles in flight; rows are XOR
//     swizzled in 16-byte chunks so both operand reads below are free of bank
//     conflicts;
//   * scores: wave w < NB holds the A rows of row block w (32 rows x 576,
//     in registers for the whole kernel) and runs S^T = tile . A^T on the
//     32x32x16 bf16 matrix core (36 MFMAs per tile), then the online softmax
//     in the accumulator layout (one row per lane pair, shuffles across the
//     pair);
//   * the probabilities (bf16) go through LDS to all four waves, each of which
//     accumulates O^T for all rows over its own quarter of d_c (128 columns;
//     8*NB MFMAs per tile) reading the tile transposed from LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kDC = 512, kDR = 64, kD = kDC + kDR;
constexpr int kChunks = kD / 8;              // 16-byte chunks per cached row (72)
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kD * 2;
constexpr int kDmaPerWave = kTileBytes / 16 / 64 / 4;   // 9 wave-wide DMAs per wave per tile
constexpr float kRescaleThreshold = 8.0f;    // log2 units: P may grow to 2^8 before rescale

// LDS chunk slot of (token t, 16-byte chunk c) inside a tile.
__device__ __forceinline__ int tile_slot(int t, int c) { return t * kChunks + (c ^ (t & 7)); }

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  if (ahead <= 0) wait_vmcnt<0>();
  else if (ahead == 1) wait_vmcnt<kDmaPerWave>();
  else if (ahead == 2) wait_vmcnt<2 * kDmaPerWave>();
  else wait_vmcnt<3 * kDmaPerWave>();
}

// One wave-wide 16-byte-per-lane copy HBM -> LDS: lane i's 16 bytes from
// gbase + voff land at LDS byte address lds_addr + 16 i.  Issued as inline
// assembly so that the only waits on it are the explicit vmcnt waits.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %0"
      :
      : "s"(gbase), "v"(voff), "s"(lds_addr)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Score MFMAs with the accumulator in VGPRs.  The compiler keeps every other
// matrix-core accumulator of this kernel (the 256 registers of O) in AGPRs;
// issuing the score chain as assembly keeps its 16 accumulators out of that
// file.  Back-to-back accumulation into the same registers needs no wait
// states; the last block ends with 32 wait states so that ordinary vector
// instructions may read the result (more than the pass count plus margin
// the hardware requires); each block starts with two wait states in case the
// compiler has just moved an operand into place with a vector ALU op.
__device__ __forceinline__ void qk_mfma4(f32x16& acc, const bf16x8& a0, const bf16x8& b0,
                                         const bf16x8& a1, const bf16x8& b1, const bf16x8& a2,
                                         const bf16x8& b2, const bf16x8& a3, const bf16x8& b3) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %4, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %7, %8, %0"
      : "+v"(acc)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1), "v"(a2), "v"(b2), "v"(a3), "v"(b3));
}

__device__ __forceinline__ void qk_mfma4_first(f32x16& acc, const bf16x8& a0, const bf16x8& b0,
                                               const bf16x8& a1, const bf16x8& b1,
                                               const bf16x8& a2, const bf16x8& b2,
                                               const bf16x8& a3, const bf16x8& b3) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %4, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %7, %8, %0"
      : "=&v"(acc)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1), "v"(a2), "v"(b2), "v"(a3), "v"(b3));
}

__device__ __forceinline__ void qk_mfma4_last(f32x16& acc, const bf16x8& a0, const bf16x8& b0,
                                              const bf16x8& a1, const bf16x8& b1,
                                              const bf16x8& a2, const bf16x8& b2,
                                              const bf16x8& a3, const bf16x8& b3) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %4, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %7, %8, %0\n\t"
      "s_nop 15\n\t"
      "s_nop 15"
      : "+v"(acc)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1), "v"(a2), "v"(b2), "v"(a3), "v"(b3));
}

template <int NB, int NBUF>
__global__ __launch_bounds__(256, 1) void splitkv_bf16_kernel(
    const bf16* __restrict__ abuf, const bf16* __restrict__ cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, int H, int page_size, int chunk, int S_max, int RQ, float scale_log2e, int Tq,
    float* __restrict__ opart, float* __restrict__ lse) {
  static_assert(NBUF >= 2 && NBUF <= 5, "tile buffers");
  __shared__ __attribute__((aligned(1024))) bf16 tiles[NBUF][kTileTok * kD];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[NB][2][64];
  __shared__ __attribute__((aligned(16))) bf16x8 qrope_s[NB][kDR / 16][64];
  __shared__ float alpha_s[NB][32];
  __shared__ float lrow_s[NB][32];

  const int nblocks = batch * S_max * RQ;
  const int logical = xcd_logical_block(blockIdx.x, nblocks);
  const int rq = logical % RQ;
  const int s = (logical / RQ) % S_max;
  const int b = logical / (RQ * S_max);

  const int q0 = cu_q[b];
  const int Lq = cu_q[b + 1] - q0;
  const int L = seq_lens[b];
  const int R = Lq * H;
  const int row_base = rq * NB * 32;
  const int tok_begin = s * chunk;
  if (row_base >= R || tok_begin >= L) return;
  const int tok_end = min(tok_begin + chunk, L);
  const int ntiles = (tok_end - tok_begin + kTileTok - 1) / kTileTok;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t rows_total = (int64_t)Tq * H;

  // Per-lane source offsets of this wave's DMA slots (loop invariant).  Slot
  // (t, c') of the LDS tile receives global chunk (t, c' ^ (t & 7)).
  uint32_t dma_off[kDmaPerWave];
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u) {
    const int slot = (wave * kDmaPerWave + u) * 64 + lane;
    const int t = slot / kChunks;
    const int c = (slot % kChunks) ^ (t & 7);
    dma_off[u] = (uint32_t)(t * kChunks + c) * 16u;
  }
  const uint32_t lds_tiles = lds_address(&tiles[0][0]);
  auto issue_tile = [&](int it, int buf) {
    const int tok0 = tok_begin + it * kTileTok;
    const int page =
        __builtin_amdgcn_readfirstlane(page_table[(int64_t)b * max_pages + tok0 / page_size]);
    const bf16* base = cache + ((int64_t)page * page_size + (tok0 % page_size)) * kD;
    const uint32_t lds0 = lds_tiles + (uint32_t)(buf * kTileBytes + wave * kDmaPerWave * 1024);
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) dma16(base, dma_off[u], lds0 + u * 1024);
  };

  // ---- this wave's score rows (waves < NB): A operand kept in registers
  const int my_row = row_base + wave * 32 + l32;         // row within the sequence
  const bool row_ok = (wave < NB) && (my_row < R);
  const int my_i = row_ok ? my_row / H : 0;
  const int my_h = row_ok ? my_row % H : 0;
  const int my_limit = row_ok ? (L - Lq + my_i) : -1;    // last visible position
  // Content part (d_c) of the score operand in registers, rope part in LDS.
  constexpr int kQReg = kDC / 16;          // 32 k-steps in registers
  bf16x8 qf[kQReg];
  {
    // rows outside the sequence read row 0 and are zeroed (no branches)
    const bf16* qrow = abuf + ((int64_t)(q0 + my_i) * H + my_h) * kD + 8 * g;
    const uint32_t keep = row_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      u32x4 v = __builtin_bit_cast(u32x4, load_bf16x8(qrow + 16 * ks));
      v &= keep;
      if (ks < kQReg) qf[ks] = __builtin_bit_cast(bf16x8, v);
      else if (wave < NB) qrope_s[wave][ks - kQReg][lane] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // LDS byte offsets inside a tile.  The swizzle only touches the low three
  // bits of the chunk index, so every read below is one of a few per-lane
  // base offsets plus a compile-time constant.
  //   score operand, k-step ks: chunk 2ks+g of token l32
  //     = qk_base[ks & 3] + 128 * (ks >> 2)
  //   value operand (token tk, dim): tk = 16ks + 8h + (4g + e),  e < 4, h < 2
  //     = pv_base[db & 1][e] + 9216 * (2ks + h) + 128 * (db >> 1)
  uint32_t qk_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    qk_base[j] = (uint32_t)(l32 * kChunks + ((2 * j + g) ^ (l32 & 7))) * 16u;
  uint32_t pv_base[2][4];
#pragma unroll
  for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dim = wave * 128 + d2 * 32 + l32;
      const int tk = 4 * g + e;
      pv_base[d2][e] = (uint32_t)(tk * kChunks + ((dim >> 3) ^ tk)) * 16u + (uint32_t)(dim & 7) * 2u;
    }

  f32x16 O[4][NB];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) O[db][rb] = zero_f32x16();
  float m_run = -INFINITY, l_run = 0.f;

  for (int p = 0; p < NBUF - 1; ++p)
    if (p < ntiles) issue_tile(p, p);

  for (int it = 0; it < ntiles; ++it) {
    wait_tiles_ahead(min(NBUF - 2, ntiles - 1 - it));   // this tile's copies have landed
    __syncthreads();                                     // ... for every wave; prior tile retired
    if (it + NBUF - 1 < ntiles) issue_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);

    const int buf = it % NBUF;
    const char* tileb = reinterpret_cast<const char*>(&tiles[buf][0]);
    const int tok0 = tok_begin + it * kTileTok;
    const int nvalid = min(kTileTok, tok_end - tok0);

    if (wave < NB) {
      // S^T[token][row] = sum_k tile[token][k] * A[row][k]   (36 MFMAs)
      f32x16 acc;
#pragma unroll
      for (int grp = 0; grp < kD / 64; ++grp) {
        bf16x8 a[4], qv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[j] = *reinterpret_cast<const bf16x8*>(tileb + qk_base[j] + 128 * grp);
          qv[j] = (4 * grp + j < kQReg) ? qf[(4 * grp + j) % kQReg] : qrope_s[wave][j][lane];
        }
        if (grp == 0)
          qk_mfma4_first(acc, a[0], qv[0], a[1], qv[1], a[2], qv[2], a[3], qv[3]);
        else if (grp == kD / 64 - 1)
          qk_mfma4_last(acc, a[0], qv[0], a[1], qv[1], a[2], qv[2], a[3], qv[3]);
        else
          qk_mfma4(acc, a[0], qv[0], a[1], qv[1], a[2], qv[2], a[3], qv[3]);
      }
      // online softmax, one row per lane pair (lanes l and l ^ 32)
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = tok0 + acc_row32(r, lane);
        acc[r] = (tok <= my_limit) ? acc[r] * scale_log2e : -INFINITY;
        tmax = fmaxf(tmax, acc[r]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = (tmax > m_run + kRescaleThreshold) ? tmax : m_run;
      const float alpha = (m_new == m_run) ? 1.f : exp2f(m_run - m_new);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      float rs = 0.f;
      bf16x8 pf0, pf1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2f(acc[r] - m_ref);
        rs += pv;
        if (r < 8) pf0[r] = from_f32<bf16>(pv);
        else pf1[r - 8] = from_f32<bf16>(pv);
      }
      rs += __shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      pbuf[wave][0][lane] = pf0;
      pbuf[wave][1][lane] = pf1;
      if (g == 0) alpha_s[wave][l32] = alpha;
    }
    __syncthreads();

    // O^T[dim][row] += sum_tok tile[tok][dim] * P[row][tok], this wave's 128 dims
    // rare: a row's running max grew past the threshold -> rescale its O
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const float al = alpha_s[rb][l32];
      if (__any(al != 1.f)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          O[db][rb] *= al;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // tokens at or past nvalid are outside the sequence: zero their values
    const uint32_t lim_lo = (uint32_t)nvalid;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb[NB];
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) pb[rb] = pbuf[rb][ks][lane];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        u32x4 packed;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // element pair (e, e+1) of the fragment: tokens tk and tk + 1
          const int h = e2 >> 1, e = 2 * (e2 & 1);
          const uint32_t off = 9216u * (2 * ks + h) + 128u * (db >> 1);
          uint32_t lo = *reinterpret_cast<const unsigned short*>(tileb + pv_base[db & 1][e] + off);
          uint32_t hi = *reinterpret_cast<const unsigned short*>(tileb + pv_base[db & 1][e + 1] + off);
          if (nvalid < kTileTok) {
            const uint32_t tk = 16 * ks + 8 * h + 4 * g + e;
            lo = tk < lim_lo ? lo : 0u;
            hi = tk + 1 < lim_lo ? hi : 0u;
          }
          packed[e2] = lo | (hi << 16);
        }
        const bf16x8 a = __builtin_bit_cast(bf16x8, packed);
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) O[db][rb] = mfma32(a, pb[rb], O[db][rb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: row statistics, then normalised partials
  if (wave < NB) {
    if (g == 0) lrow_s[wave][l32] = l_run;
    if (g == 0 && my_row < R) {
      const int64_t rowg = (int64_t)(q0 + my_i) * H + my_h;
      lse[(int64_t)s * rows_total + rowg] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
    }
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = row_base + rb * 32 + l32;
    if (row >= R) continue;
    const float lr = lrow_s[rb][l32];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    const int64_t rowg = (int64_t)(q0 + row / H) * H + row % H;
    float* dst = opart + ((int64_t)s * rows_total + rowg) * kDC + wave * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = O[db][rb][4 * q4 + e] * inv;
        *reinterpret_cast<f32x4*>(dst + db * 32 + 8 * q4 + 4 * g) = v;
      }
  }
}

// ---------------------------------------------------------------- fp32 path
// One workgroup per (query row, split); 64-token tiles; VALU dot products.
constexpr int kF32Tile = 64;

__global__ __launch_bounds__(256) void splitkv_f32_kernel(
    const float* __restrict__ abuf, const float* __restrict__ cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, int H, int dc, int dr, int page_size, int chunk, int S_max, float scale_log2e, int Tq,
    float* __restrict__ opart, float* __restrict__ lse) {
  extern __shared__ float smem[];
  const int D = dc + dr;
  float* qs = smem;                    // [D]
  float* ps = smem + D;                // [kF32Tile]
  const int64_t rowg = blockIdx.x / S_max;
  const int s = blockIdx.x % S_max;
  const int t = (int)(rowg / H);
  const int b = seq_of_token(cu_q, batch, t);
  const int Lq = cu_q[b + 1] - cu_q[b];
  const int L = seq_lens[b];
  if (s * chunk >= L) return;                        // split beyond this sequence
  const int limit = L - Lq + (t - cu_q[b]);          // last visible position
  const int tok_begin = s * chunk;
  const int tok_end = min(tok_begin + chunk, limit + 1);
  const int64_t rows_total = (int64_t)Tq * H;
  const int tid = threadIdx.x;
  for (int k = tid; k < D; k += blockDim.x) qs[k] = abuf[rowg * D + k];
  constexpr int kMaxPer = 4;                          // d_c <= 1024
  float o[kMaxPer];
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) o[u] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();
  for (int tb = tok_begin; tb < tok_end; tb += kF32Tile) {
    const int n = min(kF32Tile, tok_end - tb);
    {  // 4 threads per token
      const int tk = tid >> 2, part = tid & 3;
      float acc = 0.f;
      if (tk < n) {
        const int pos = tb + tk;
        const int page = page_table[(int64_t)b * max_pages + pos / page_size];
        const float* row = cache + ((int64_t)page * page_size + pos % page_size) * D;
        for (int k = part; k < D; k += 4) acc = fmaf(row[k], qs[k], acc);
      }
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      if (tk < n && part == 0) ps[tk] = acc * scale_log2e;
    }
    __syncthreads();
    float tmax = -INFINITY;
    for (int k = 0; k < n; ++k) tmax = fmaxf(tmax, ps[k]);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);        // m_run = -inf on the first tile -> 0
    float psum = 0.f;
    for (int k = 0; k < n; ++k) psum += exp2f(ps[k] - m_new);
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      const int j = tid + u * blockDim.x;
      if (j >= dc) break;
      float acc = o[u] * alpha;
      for (int k = 0; k < n; ++k) {
        const int pos = tb + k;
        const int page = page_table[(int64_t)b * max_pages + pos / page_size];
        acc = fmaf(exp2f(ps[k] - m_new), cache[((int64_t)page * page_size + pos % page_size) * D + j], acc);
      }
      o[u] = acc;
    }
    m_run = m_new;
    __syncthreads();
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    const int j = tid + u * blockDim.x;
    if (j < dc) opart[((int64_t)s * rows_total + rowg) * dc + j] = o[u] * inv;
  }
  if (tid == 0) lse[(int64_t)s * rows_total + rowg] = l_run > 0.f ? m_run + log2f(l_run) : -INFINITY;
}

// ---------------------------------------------------------------- combine
template <typename T>
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ opart,
                                                      const float* __restrict__ lse,
                                                      const int32_t* __restrict__ cu_q,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int batch, int Tq, int H, int dc, int chunk,
                                                      T* __restrict__ olat) {
  const int64_t rowg = blockIdx.x;
  const int t = (int)(rowg / H);
  const int b = seq_of_token(cu_q, batch, t);
  const int L = seq_lens[b];
  const int S_b = (L + chunk - 1) / chunk;
  const int64_t rows_total = (int64_t)Tq * H;
  float M = -INFINITY;
  for (int s = 0; s < S_b; ++s) M = fmaxf(M, lse[s * rows_total + rowg]);
  float wsum = 0.f;
  for (int s = 0; s < S_b; ++s) {
    const float x = lse[s * rows_total + rowg];
    wsum += (x == -INFINITY) ? 0.f : exp2f(x - M);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  for (int j = threadIdx.x; j < dc; j += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < S_b; ++s) {
      const float x = lse[s * rows_total + rowg];
      if (x == -INFINITY) continue;
      acc = fmaf(exp2f(x - M), opart[(s * rows_total + rowg) * dc + j], acc);
    }
    olat[rowg * dc + j] = from_f32<T>(acc * inv);
  }
}

}  // namespace

void launch_splitkv(int elem, const SplitPlan& plan, const void* abuf, const void* cache,
                    const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                    int max_pages, int batch, int Tq, int H, int dc, int dr, int page_size,
                    float scale, float* opart, float* lse, hipStream_t st) {
  const float scale_log2e = scale * 1.4426950408889634f;
  if (elem == 2) {
    const int nblocks = batch * plan.S_max * plan.RQ;
    switch (plan.NB) {
      case 4:
        splitkv_bf16_kernel<4, 3><<<nblocks, 256, 0, st>>>(
            (const bf16*)abuf, (const bf16*)cache, cu_q, seq_lens, page_table, max_pages, batch, H,
            page_size, plan.chunk, plan.S_max, plan.RQ, scale_log2e, Tq, opart, lse);
        break;
      case 2:
        splitkv_bf16_kernel<2, 3><<<nblocks, 256, 0, st>>>(
            (const bf16*)abuf, (const bf16*)cache, cu_q, seq_lens, page_table, max_pages, batch, H,
            page_size, plan.chunk, plan.S_max, plan.RQ, scale_log2e, Tq, opart, lse);
        break;
      default:
        splitkv_bf16_kernel<1, 4><<<nblocks, 256, 0, st>>>(
            (const bf16*)abuf, (const bf16*)cache, cu_q, seq_lens, page_table, max_pages, batch, H,
            page_size, plan.chunk, plan.S_max, plan.RQ, scale_log2e, Tq, opart, lse);
        break;
    }
  } else {
    const int64_t nblocks = (int64_t)Tq * H * plan.S_max;
    const size_t shm = (size_t)(dc + dr + kF32Tile) * sizeof(float);
    splitkv_f32_kernel<<<(unsigned)nblocks, 256, shm, st>>>(
        (const float*)abuf, (const float*)cache, cu_q, seq_lens, page_table, max_pages, batch, H, dc,
        dr, page_size, plan.chunk, plan.S_max, scale_log2e, Tq, opart, lse);
  }
}

void launch_combine(int elem, const SplitPlan& plan, const float* opart, const float* lse,
                    const int32_t* cu_q, const int32_t* seq_lens, int batch, int Tq, int H, int dc,
                    void* olat, hipStream_t st) {
  const unsigned rows = (unsigned)((int64_t)Tq * H);
  if (elem == 2)
    combine_kernel<bf16><<<rows, 128, 0, st>>>(opart, lse, cu_q, seq_lens, batch, Tq, H, dc,
                                               plan.chunk, (bf16*)olat);
  else
    combine_kernel<float><<<rows, 128, 0, st>>>(opart, lse, cu_q, seq_lens, batch, Tq, H, dc,
                                                plan.chunk, (float*)olat);
}

}  // namespace mla

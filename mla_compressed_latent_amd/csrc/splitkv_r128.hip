// Split-KV attention over the paged latent cache, 128 query rows per
// workgroup, four waves (one per SIMD, up to 512 registers each).
//
// The step is the dense contraction of the other split-KV kernels
// ("Multi-head Latent Attention: the KV cache, compressed", sections "The one
// formula" and "Absorption: the part that makes it free": every head scores
// the same cached row [c | k_rope]):
//     S[row][t]  = scale * A[row] . cache[t]          (K = 576)
//     O[row][:] += softmax_t(S) cache[t][:512]        (K = tokens)
// with an online softmax per row and normalised partials + log2-sum-exp per
// (row, split).  Partials are bf16 ([split][row][512], as those of the
// 64- and 32-row kernels; the fp32 kernel writes fp32), rounded once from
// the fp32 accumulators.
//
// All matrix work is on the 32x32x16 bf16 instruction.  Wave w (pair
// p = w / 2, half d = w % 2):
//   * scores S^T = tile . A^T for the 64 rows of row blocks 2p and 2p+1 over
//     the 288 dims [288 d, 288 d + 288) of each cached row -- two
//     accumulators, one per row block, each tile fragment read from LDS once
//     for both; its share of the score operand (64 rows x 288 dims) stays in
//     144 VGPRs.  Splitting the dims between the pair instead of the rows
//     halves the tile reads: with every wave reading the whole tile, the LDS
//     reads held back the tile copies' writes into LDS and the loop waited on
//     memory (measured: 2.3k of 6.7k cycles per tile spent issuing copies);
//   * the pair swaps partial scores through LDS: wave w finishes row block w
//     (its own half plus its partner's), runs the online softmax of those 32
//     rows (per lane plus one lane-half swap) and publishes bf16
//     probabilities and rescale factors in the value product's layout;
//   * O^T for latent columns [128 w, 128 w + 128) of all 128 rows (16 blocks
//     of 32 x 32, the 256 AGPRs), value operand read with the transposing LDS
//     load, the probabilities of all four row blocks as the B operand.
// Each iteration interleaves the two score chains of tile `it` with the
// value product of tile it-1.  Four tile buffers (two in use, two in flight)
// and a 16 KB swap buffer fill the 160 KB of LDS: a wave's slot holds its
// partial scores for its partner, then, once the partner has read them, the
// partner's probabilities for everyone.
#include "attn_tile.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kRRows = 128;
constexpr int kRBuf = 4;
constexpr int kRDma = kTileBytes / 1024 / 4;   // 9 wave-wide copies per wave per tile
constexpr int kRSteps = 18;                    // k-steps of one 288-dim half
constexpr int kRRing = 2;                      // score-operand reads in flight (four MFMAs each in the loop)

// Chunk swizzle of this kernel's tiles: 16-byte chunk c of token t sits at
// position c ^ swz_r(t) of the token's LDS row (inside c's aligned group of
// 8).  Chosen by an exhaustive search over XOR maps of the token bits so
// that both operand reads are free of bank conflicts on the 64-bank LDS
// (zero conflicts measured): the score operand (16 lanes = 16 consecutive
// tokens, one chunk each) and the transposing value-operand read (32 lanes =
// 4 tokens x 64 bytes).
__device__ __forceinline__ int swz_r(int t) {
  return ((t >> 1) & 1) | (((t >> 2) & 1) << 1) | ((((t >> 1) ^ (t >> 3)) & 1) << 2);
}

// Both score chains on one tile fragment, each followed by an independent
// value MFMA, so the matrix core never waits on a chain's dependency.  Two
// wait states first (an operand may have just been assembled by a vector
// instruction).
__device__ __forceinline__ void svsv(f32x16& s0, f32x16& s1, const bf16x8& a, const bf16x8& q0,
                                     const bf16x8& q1, f32x16& o0, f32x16& o1, const bf16x8& v,
                                     const bf16x8& p0, const bf16x8& p1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %7, %8, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %6, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %7, %9, %3"
      : "+v"(s0), "+v"(s1), "+a"(o0), "+a"(o1)
      : "v"(a), "v"(q0), "v"(q1), "v"(v), "v"(p0), "v"(p1));
}
__device__ __forceinline__ void ss(f32x16& s0, f32x16& s1, const bf16x8& a, const bf16x8& q0,
                                   const bf16x8& q1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1"
      : "+v"(s0), "+v"(s1)
      : "v"(a), "v"(q0), "v"(q1));
}
__device__ __forceinline__ void ss_first(f32x16& s0, f32x16& s1, const bf16x8& a, const bf16x8& q0,
                                         const bf16x8& q1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %2, %4, 0"
      : "=&v"(s0), "=&v"(s1)
      : "v"(a), "v"(q0), "v"(q1));
}
__device__ __forceinline__ void svsv_first(f32x16& s0, f32x16& s1, const bf16x8& a, const bf16x8& q0,
                                           const bf16x8& q1, f32x16& o0, f32x16& o1, const bf16x8& v,
                                           const bf16x8& p0, const bf16x8& p1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %5, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %7, %8, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %6, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %7, %9, %3"
      : "=&v"(s0), "=&v"(s1), "+a"(o0), "+a"(o1)
      : "v"(a), "v"(q0), "v"(q1), "v"(v), "v"(p0), "v"(p1));
}
__device__ __forceinline__ void vv(f32x16& o0, f32x16& o1, const bf16x8& v, const bf16x8& p0,
                                   const bf16x8& p1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1"
      : "+a"(o0), "+a"(o1)
      : "v"(v), "v"(p0), "v"(p1));
}
__device__ __forceinline__ void v_one(f32x16& o, const bf16x8& v, const bf16x8& p) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
      : "+a"(o)
      : "v"(v), "v"(p));
}
// wait states after the last score MFMAs before vector instructions read them
__device__ __forceinline__ void s_drain(f32x16& s0, f32x16& s1) {
  asm volatile("s_nop 15\n\ts_nop 15" : "+v"(s0), "+v"(s1));
}
__device__ __forceinline__ void o_drain(f32x16 (&o)[4][4]) {
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    asm volatile("s_nop 7" : "+a"(o[cb][0]), "+a"(o[cb][1]), "+a"(o[cb][2]), "+a"(o[cb][3]));
}

__global__ __launch_bounds__(256, 1) void splitkv_bf16_r128_kernel(
    const bf16* __restrict__ abuf, const bf16* __restrict__ cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, int H, int page_size, int chunk, int S_max, int RQ, int Tq,
    bf16* __restrict__ opart, float* __restrict__ lse, const int2* __restrict__ items,
    const int* __restrict__ list_hdr) {
  __shared__ __attribute__((aligned(1024))) bf16 tiles[kRBuf][kTileTok * kD];
  // swap slot of wave w: first w's partial scores of row block w ^ 1 (16
  // registers x 64 lanes, fp32), then row block w ^ 1's probabilities
  // ([k-step][lane] bf16x8, 2 KB) and rescale factors (32 floats)
  __shared__ __attribute__((aligned(1024))) float xs[4][16 * 64];

  int b, s, rq;
  if (!split_work_item(items, list_hdr, batch, S_max, RQ, &b, &s, &rq)) return;

  const int q0 = cu_q[b];
  const int Lq = cu_q[b + 1] - q0;
  const int L = seq_lens[b];
  const int R = Lq * H;
  const int row_base = rq * kRRows;
  const int tok_begin = s * chunk;
  if (row_base >= R || tok_begin >= L) return;
  // stop at the last key any row of the block can see, keeping at least one
  // token so that the split still writes its (empty) partial
  const int last_vis = L - Lq + (min(row_base + kRRows, R) - 1) / H;
  // (block-uniform values pinned to scalar registers: the loop is short of
  // VGPRs)
  const int tok_end =
      __builtin_amdgcn_readfirstlane(min(min(tok_begin + chunk, L), max(tok_begin + 1, last_vis + 1)));
  const int ntiles = __builtin_amdgcn_readfirstlane((tok_end - tok_begin + kTileTok - 1) / kTileTok);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int pr = wave >> 1, hd = wave & 1;   // pair (row blocks 2 pr, 2 pr + 1), dims half
  const int64_t rows_total = (int64_t)Tq * H;

  // ---- tile copies: LDS position (t, c') of a tile receives global chunk
  // (t, c' ^ swz_r(t)); each wave copies 9 of the tile's 36 wave-wide chunks.
  // Copy u of wave w fills positions p = 576 w + 64 u + lane; since 72 and 64
  // are multiples of 8, c' mod 8 = lane mod 8, so the source chunk is
  // p - lane % 8 + ((lane % 8) ^ swz_r(p / 72)): the byte offset
  // 16 (576 w + 64 u) goes on the scalar base, and p / 72 = 8 w + k_u +
  // (lane >= th_u) with k_u = 64 u / 72, th_u = 72 (k_u + 1) - 64 u, so the
  // swizzle is one of two block-uniform values per copy.  The per-lane part
  // is formed at each issue from the lane id (opaque to the compiler, so it
  // is not hoisted into registers the loop cannot spare).
  // Page ids are read with scalar loads as each tile is issued.
  const uint32_t lds_tiles = lds_address(&tiles[0][0]);
  const int32_t* __restrict__ ptab = page_table + (int64_t)b * max_pages;
  auto issue_tile = [&](int it) {
    const int tok0 = tok_begin + it * kTileTok;
    const int page = __builtin_amdgcn_readfirstlane(ptab[tok0 / page_size]);
    const char* src = reinterpret_cast<const char*>(cache + ((int64_t)page * page_size + (tok0 % page_size)) * kD) +
                      16 * 576 * wave;
    const uint32_t dst = lds_tiles + (uint32_t)((it % kRBuf) * kTileBytes + wave * kRDma * 1024);
    int ln = (int)threadIdx.x & 63;
    asm volatile("" : "+v"(ln));
    const uint32_t lane8 = (uint32_t)(ln & ~7) * 16u, l7 = (uint32_t)(ln & 7);
#pragma unroll
    for (int u = 0; u < kRDma; ++u) {
      const int ku = 64 * u / kChunks, th = kChunks * (ku + 1) - 64 * u;
      const uint32_t s_lo = (uint32_t)swz_r(8 * wave + ku), s_hi = (uint32_t)swz_r(8 * wave + ku + 1);
      const uint32_t sw = ln >= th ? s_hi : s_lo;
      dma16(src + 1024 * u, lane8 + ((l7 ^ sw) << 4), dst + u * 1024);
    }
  };
  // this wave's softmax rows: row block `wave`
  const int my_row = row_base + 32 * wave + l32;
  const bool row_ok = my_row < R;
  const int my_i = row_ok ? my_row / H : 0, my_h = row_ok ? my_row % H : 0;
  const int my_lim = row_ok ? L - Lq + my_i : -1;

  // score operand (A) of k-step st of this wave's half: token l32, chunk
  // c = 36 hd + 2 st + g = a_base[st & 3] + 128 (st >> 2) (st + 4 moves c by
  // 8: the next group of 8 chunks; the swizzle stays in the low 3 bits)
  // (the four byte offsets, each < 36 KB, two per register)
  uint32_t a_base2[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 36 * hd + 2 * j + g;
    const uint32_t off = (uint32_t)(l32 * kChunks + (c & ~7) + ((c & 7) ^ swz_r(l32))) * 16u;
    if (j & 1) a_base2[j >> 1] |= off << 16;
    else a_base2[j >> 1] = off;
  }
  // value operand (A) of column block cb, k-step ks through the transposing
  // read: in 16-lane group G, source lane 4 j + q points at dims 4q .. 4q+3 of
  // the group's 16 (cols 128 w + 32 cb + 16 (G & 1) ..) of token 16 ks +
  // 4 (G >> 1) + 8 r + j (r: which half of the fragment), so that result lane
  // i holds col 16 (G & 1) + i of those four tokens: the token order of the
  // score accumulator rows (8 (e / 4) + 4 g + e % 4), i.e. of the
  // probabilities.  swz_r ignores token bit 4 and flips chunk bit 2 with token
  // bit 3, so every (cb, ks, r) address is one of two per-lane bases plus a
  // constant: v_base[(cb & 1) ^ r] + 18432 ks + 9216 r + 128 (cb >> 1).
  // (both < 36 KB, packed in one register)
  uint32_t v_base2 = 0;
  {
    const int G = lane >> 4, j = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1) {
      const int t = 4 * (G >> 1) + j;
      const int c = 16 * wave + 4 * c1 + 2 * (G & 1) + (q >> 1);   // chunk of the 8 dims
      v_base2 |= ((uint32_t)(t * kChunks + (c ^ swz_r(t))) * 16u + 8u * (q & 1)) << (16 * c1);
    }
  }
  auto v_addr = [&](int cb, int ks, int r) {
    const int c1 = (cb & 1) ^ r;
    return (c1 ? (v_base2 >> 16) : (v_base2 & 0xffffu)) + (uint32_t)(18432 * ks + 9216 * r + 128 * (cb >> 1));
  };

  f32x16 O[4][4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      O[cb][hb] = zero_f32x16();
      asm volatile("" : "+a"(O[cb][hb]));
    }
  float m_run = -INFINITY, l_run = 0.f;

  auto tile_ptr = [&](int it) { return reinterpret_cast<const char*>(&tiles[it % kRBuf][0]); };
  auto a_frag = [&](const char* ts, int st) {
    const uint32_t w2 = a_base2[(st & 3) >> 1];
    const uint32_t ab = (st & 1) ? (w2 >> 16) : (w2 & 0xffffu);
    return *reinterpret_cast<const bf16x8*>(ts + ab + 128 * (st >> 2));
  };
  // ---- the score operand.  This workgroup's 128 query rows (abuf rows
  // q0 H + row_base .. + 127, contiguous) are copied HBM -> LDS as four
  // 32-row tiles (row block hb into tile buffer hb, the cached rows'
  // swizzle), then each wave reads its B fragments (row block 2 pr + j,
  // k-step st: rows 32 (2 pr + j) + l32, dims 288 hd + 16 st + 8 g .. + 7)
  // with the score operand's conflict-free reads.  (Loading them straight
  // into registers took 36 loads per lane that each touched 32 rows.)  Rows
  // past R copy row R - 1 (finite; their results are never stored).
  bf16x8 qf[2][kRSteps];
  {
    const bf16* qsrc = abuf + ((int64_t)q0 * H + row_base) * kD;
    const int nrows = min(kRRows, R - row_base);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const uint32_t dst = lds_tiles + (uint32_t)(hb * kTileBytes + wave * kRDma * 1024);
#pragma unroll
      for (int u = 0; u < kRDma; ++u) {
        const int slot = (wave * kRDma + u) * 64 + lane;
        const int t = slot / kChunks, c = slot % kChunks;
        const int row = min(32 * hb + t, nrows - 1);
        dma16(qsrc, (uint32_t)(row * kChunks + (c ^ swz_r(t))) * 16u, dst + u * 1024);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int st = 0; st < kRSteps; ++st) qf[j][st] = a_frag(tile_ptr(2 * pr + j), st);
    __syncthreads();   // every wave holds its fragments: the buffers take cached rows
  }
  for (int p = 0; p < 2; ++p)
    if (p < ntiles) issue_tile(p);

  char* const xsb = reinterpret_cast<char*>(&xs[0][0]);
  // probabilities of row block hb (k-step ks) and their rescale factors sit
  // in the swap slot of wave hb ^ 1
  auto p_frag = [&](int hb, int ks) {
    return *reinterpret_cast<const bf16x8*>(xsb + (hb ^ 1) * 4096 + ks * 1024 + lane * 16);
  };
  auto p_alpha = [&](int hb) {
    return *reinterpret_cast<const float*>(xsb + (hb ^ 1) * 4096 + 2048 + l32 * 4);
  };

  // Top of iteration `it`: own copies of tile `it` landed (tile it+1's may
  // still be in flight), barrier (tile `it` everywhere, P(it-1) published,
  // tile it-2's buffer free), the copies of tile it+2 into that buffer, and
  // the value columns of rows past the sequence's end zeroed (the page holds
  // whatever it held there; the value product reads them next iteration).
  auto top = [&](int it) {
    if (it < ntiles) {
      if (it + 1 < ntiles) wait_vmcnt<kRDma>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    if (it + 2 < ntiles) issue_tile(it + 2);
    if (it < ntiles) {
      const int nvalid = tok_end - (tok_begin + it * kTileTok);
      if (nvalid < kTileTok) {
        char* tz = reinterpret_cast<char*>(&tiles[it % kRBuf][0]);
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int i = threadIdx.x; i < (kTileTok - nvalid) * (kDC / 8); i += 256)
          *reinterpret_cast<u32x4*>(tz + (nvalid + i / (kDC / 8)) * kD * 2 + (i % (kDC / 8)) * 16) = z;
      }
    }
  };
  // O is rescaled when a row's running max moved at the previous tile (rare)
  auto rescale = [&](const float (&al)[4]) {
    bool any = false;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) any |= al[hb] != 1.f;
    if (__any(any)) {
      o_drain(O);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          O[cb][hb] *= al[hb];
          asm volatile("" : "+a"(O[cb][hb]));
        }
    }
  };
  // The pair's partial scores meet: this wave hands its accumulator of the
  // partner's row block to the partner through its own slot, then adds the
  // partner's half of its own row block (the sum is the same either way
  // round), runs the online softmax of its 32 rows over tile `it` (token
  // tok0 + acc_row32(r, lane) of S[r]; scores are already in log2 units) and
  // leaves the probabilities and rescale factors in the partner's slot,
  // which it has just read.  vstep(i), i = 0..7, is called between the steps
  // (the steady state issues pairs of value MFMAs there, so that the matrix
  // core works under the swap, the barrier and the vector work).
  auto finish_tile = [&](int it, f32x16& S0, f32x16& S1, auto&& vstep) {
    f32x16& mine = hd ? S1 : S0;
    f32x16& other = hd ? S0 : S1;
    {
      f32x4* dst = reinterpret_cast<f32x4*>(xsb + wave * 4096) + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[64 * q] = f32x4{other[4 * q], other[4 * q + 1], other[4 * q + 2], other[4 * q + 3]};
    }
    vstep(0);
    __syncthreads();
    f32x4 part[4];
    {
      const f32x4* src = reinterpret_cast<const f32x4*>(xsb + (wave ^ 1) * 4096) + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) part[q] = src[64 * q];
    }
    vstep(1);
    f32x16 S;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[4 * q + e] = mine[4 * q + e] + part[q][e];
    const int tok0 = tok_begin + it * kTileTok;
    if (tok0 + kTileTok - 1 > L - Lq) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (tok0 + acc_row32(r, lane) > my_lim) S[r] = -INFINITY;
    }
    float tmax = max_raw(max_raw(max_raw(S[0], S[1]), max_raw(S[2], S[3])),
                         max_raw(max_raw(S[4], S[5]), max_raw(S[6], S[7])));
    tmax = max_raw(tmax, max_raw(max_raw(max_raw(S[8], S[9]), max_raw(S[10], S[11])),
                                 max_raw(max_raw(S[12], S[13]), max_raw(S[14], S[15]))));
    vstep(2);
    {
      const float2 h = lane_halves(tmax);
      tmax = max_raw(h.x, h.y);
    }
    const float m_new = (tmax > m_run + kRescaleThreshold) ? tmax : m_run;
    const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    vstep(3);
    float p[16];
#pragma unroll
    for (int r = 0; r < 8; ++r) p[r] = __builtin_amdgcn_exp2f(S[r] - m_ref);
    vstep(4);
#pragma unroll
    for (int r = 8; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(S[r] - m_ref);
    vstep(5);
    bf16x8 pf0, pf1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      pf0[r] = from_f32<bf16>(p[r]);
      pf1[r] = from_f32<bf16>(p[8 + r]);
    }
    char* slot = xsb + (wave ^ 1) * 4096;
    *reinterpret_cast<bf16x8*>(slot + lane * 16) = pf0;
    *reinterpret_cast<bf16x8*>(slot + 1024 + lane * 16) = pf1;
    if (g == 0) *reinterpret_cast<float*>(slot + 2048 + l32 * 4) = alpha;
    float rs = (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) +
               (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
    vstep(6);
    {
      const float2 h = lane_halves(rs);
      rs = h.x + h.y;
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    vstep(7);
  };

  // ---- tile 0: scores only
  {
    top(0);
    const char* ts = tile_ptr(0);
    f32x16 S0, S1;
    bf16x8 ring[kRRing];
#pragma unroll
    for (int k = 0; k < kRRing; ++k) ring[k] = a_frag(ts, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < kRSteps; ++st) {
      bf16x8& a = ring[st % kRRing];
      if (st == 0) ss_first(S0, S1, a, qf[0][0], qf[1][0]);
      else ss(S0, S1, a, qf[0][st], qf[1][st]);
      if (st + kRRing < kRSteps) a = a_frag(ts, st + kRRing);
      __builtin_amdgcn_sched_barrier(0);
    }
    s_drain(S0, S1);
    finish_tile(0, S0, S1, [](int) {});
  }

  // ---- steady state: score k-steps 0, 1 of tile `it` (both chains) alone,
  // under the reads of the rescale factors, the first k-step of P(it-1) and
  // the first value fragments; then k-step st = 2..17 with value pair
  // jp = st - 2 of tile it-1 (value fragment f = jp / 2 = (k-step f / 4,
  // column block f % 4), row blocks 2 (jp % 2) and 2 (jp % 2) + 1).  The
  // second k-step of P(it-1) (pairs 8..15) is read into the same registers as
  // the first one's pairs finish; a barrier after that read (every wave then
  // holds what it needs of P(it-1)) frees the swap slots for tile `it`.
  // (Running half of the value pairs inside the swap and softmax instead was
  // tried: holding their operands there needs more than the 256 VGPRs left
  // beside the score operand, and the spill reloads waited on the tile
  // copies.)
  for (int it = 1; it < ntiles; ++it) {
    top(it);
    float al[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) al[hb] = p_alpha(hb);
    const char* ts = tile_ptr(it);
    const char* tv = tile_ptr(it + kRBuf - 1);
    bf16x8 ring[kRRing];
#pragma unroll
    for (int k = 0; k < kRRing; ++k) ring[k] = a_frag(ts, k);
    bf16x8 pb[4];   // P(it-1) of the four row blocks, k-step 0, then k-step 1
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) pb[hb] = p_frag(hb, 0);
    v4bf16 vf[2][2];   // two value fragments in flight
    auto load_vf = [&](int f, v4bf16 (&d)[2]) {
      const int ks = f >> 2, cb = f & 3;
#pragma unroll
      for (int r = 0; r < 2; ++r) d[r] = ds_read_tr16(tv + v_addr(cb, ks, r));
    };
    load_vf(0, vf[0]);
    load_vf(1, vf[1]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 S0, S1;
    ss_first(S0, S1, ring[0], qf[0][0], qf[1][0]);
    ring[0] = a_frag(ts, kRRing);
    __builtin_amdgcn_sched_barrier(0);
    ss(S0, S1, ring[1], qf[0][1], qf[1][1]);
    ring[1] = a_frag(ts, kRRing + 1);
    rescale(al);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 2; st < kRSteps; ++st) {
      bf16x8& a = ring[st % kRRing];
      const int jp = st - 2, f = jp >> 1, h0 = 2 * (jp & 1), cb = f & 3;
      const bf16x8 v = __builtin_shufflevector(vf[f & 1][0], vf[f & 1][1], 0, 1, 2, 3, 4, 5, 6, 7);
      svsv(S0, S1, a, qf[0][st], qf[1][st], O[cb][h0], O[cb][h0 + 1], v, pb[h0], pb[h0 + 1]);
      if ((jp & 1) && f + 2 < 8) load_vf(f + 2, vf[f & 1]);
      if (st + kRRing < kRSteps) a = a_frag(ts, st + kRRing);
      if (jp == 6 || jp == 7) {   // last k-step-0 use of row blocks h0, h0 + 1
        pb[h0] = p_frag(h0, 1);
        pb[h0 + 1] = p_frag(h0 + 1, 1);
      }
      if (jp == 8) __syncthreads();   // P(it-1) read everywhere: the swap slots are free
      __builtin_amdgcn_sched_barrier(0);
    }
    s_drain(S0, S1);
    finish_tile(it, S0, S1, [](int) {});
  }

  // ---- the last tile's value product
  {
    top(ntiles);
    float al[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) al[hb] = p_alpha(hb);
    rescale(al);
    const char* tv = tile_ptr(ntiles + kRBuf - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pb[hb] = p_frag(hb, ks);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        v4bf16 d[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) d[r] = ds_read_tr16(tv + v_addr(cb, ks, r));
        const bf16x8 v = __builtin_shufflevector(d[0], d[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) v_one(O[cb][hb], v, pb[hb]);
      }
    }
  }
  o_drain(O);

  // ---- epilogue: row sums and log2-sum-exps, then the normalised partials
  // in bf16: staged through LDS as rows of 512 (+ 8 bytes against bank
  // conflicts) and written out as whole 1 KB rows (written straight from the
  // accumulator layout, every store touched 32 rows)
  float* lrow_s = reinterpret_cast<float*>(&tiles[(ntiles + 2) % kRBuf][0]);
  if (g == 0) lrow_s[32 * wave + l32] = l_run;
  if (g == 0 && row_ok) {
    const int64_t rowg = (int64_t)(q0 + my_i) * H + my_h;
    lse[(int64_t)s * rows_total + rowg] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
  }
  __syncthreads();
  float inv[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const float lr = lrow_s[32 * hb + l32];
    inv[hb] = lr > 0.f ? 1.f / lr : 0.f;
  }
  __syncthreads();   // row sums read and every value read done: the tile buffers take the rows
  constexpr int kStRow = kDC * 2 + 8;
  char* const stg = reinterpret_cast<char*>(&tiles[0][0]);
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& o = O[cb][hb];
        const bf16x4 v = {from_f32<bf16>(o[4 * q4] * inv[hb]), from_f32<bf16>(o[4 * q4 + 1] * inv[hb]),
                          from_f32<bf16>(o[4 * q4 + 2] * inv[hb]), from_f32<bf16>(o[4 * q4 + 3] * inv[hb])};
        *reinterpret_cast<bf16x4*>(stg + (32 * hb + l32) * kStRow +
                                   (128 * wave + 32 * cb + 8 * q4 + 4 * g) * 2) = v;
      }
  __syncthreads();
  bf16* const part = opart;
  for (int r = wave; r < kRRows; r += 4) {
    const int row = row_base + r;
    if (row >= R) break;
    const int64_t rowg = (int64_t)q0 * H + row;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * kStRow + lane * 16);
    *reinterpret_cast<u32x4*>(part + ((int64_t)s * rows_total + rowg) * kDC + lane * 8) = v;
  }
}

}  // namespace

void launch_splitkv_r128(const SplitPlan& plan, const void* abuf, const void* cache,
                         const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                         int max_pages, int batch, int Tq, int H, int page_size, void* opart,
                         float* lse, const int2* items, const int* list_hdr, hipStream_t st) {
  const int nblocks = items ? work_list_grid(batch, plan) : batch * plan.S_max * plan.RQ;
  splitkv_bf16_r128_kernel<<<nblocks, 256, 0, st>>>(
      (const bf16*)abuf, (const bf16*)cache, cu_q, seq_lens, page_table, max_pages, batch, H,
      page_size, plan.chunk, plan.S_max, plan.RQ, Tq, (bf16*)opart, lse, items, list_hdr);
}

}  // namespace mla

// Split-KV attention over the paged latent cache, and the split combine.
//
// Every head scores the SAME cached row [c | k_rope] ("Multi-head Latent
// Attention: the KV cache, compressed", section "The one formula": one latent
// row per token serves all heads), so for one sequence the step is a dense
// contraction with the (query, head) rows as one dimension:
//     S[row][t]   = scale * A[row] . cache[t]          (K = d_c + d_rope)
//     O[row][:]  += softmax_t(S) cache[t][:d_c]        (K = tokens)
// which is "still softmax(Q K^T / sqrt d) V with K factored" (section
// "Absorption: the part that makes it free").  Each workgroup takes one
// chunk of one sequence's tokens ("split"), keeps a running max and sum per
// row (online softmax), and leaves a normalised partial O (bf16 for bf16
// layers, rounded once from the fp32 accumulators) and its log-sum-exp;
// the combine kernel merges the splits.
//
// bf16 path, at most 32 rows per sequence (d_c = 512, d_rope = 64; more rows
// go to the eight-wave kernel of splitkv_x8.hip), one workgroup of 4 waves per
// (sequence, split):
//   * 32-token tiles of cached rows are copied HBM -> LDS by the LDS-DMA path
//     (global_load_lds, 16 bytes per lane, every wave copies 8 rows) into a
//     ring of four: two in use (the value waves' and the score wave's), two
//     in flight; 16-byte chunks are swizzled per row (swz) so that both
//     operand reads below are free of bank conflicts;
//   * the score wave (0) keeps the 32 rows of the score operand (32 x 576
//     bf16) in registers and computes S^T = tile . A^T on the 32x32x16 bf16
//     matrix core (36 MFMAs per tile), then the online softmax in the
//     accumulator layout (one row per lane pair), and hands the bf16
//     probabilities to LDS;
//   * value waves (2, 3) each accumulate O^T for the 32 rows over half of d_c
//     (256 columns), reading the value operand straight out of the
//     token-major tile with the transposing LDS load (ds_read_b64_tr_b16);
//   * the score waves work one tile ahead of the value waves, so the two kinds
//     of matrix work overlap; one barrier per tile.
#include "attn_tile.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kNBuf = 4;                      // tiles resident in LDS (2 in use, 2 in flight)
constexpr int kQkRing = 3;                    // score-operand read groups in flight
constexpr int kPvRing = 6;                    // value-operand reads in flight

// F8: MLA_CACHE_FP8 pages.  Waves 1-3 copy each FP8 tile to one of two
// staging buffers (seven 1 KB copies each) and convert it into the bf16 tile
// ring (three tiles) -- wave 1, which has no matrix work, half the latent
// codes and all rope keys, the value waves a quarter each -- while the score
// wave scores the tile before it and the value waves use the one before that.
template <int NB, bool F8>
__global__ __launch_bounds__(256, 1) void splitkv_bf16_kernel(
    const bf16* __restrict__ abuf, const void* __restrict__ cache_v, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, int H, int page_size, int chunk, int S_max, int RQ, float scale_log2e, int Tq,
    bf16* __restrict__ opart, float* __restrict__ lse) {
  static_assert(NB == 1, "one 32-row block per workgroup");
  constexpr int kDbPerPv = kDC / 32 / 2;       // 32-wide value blocks per value wave (8)
  constexpr int kBuf = F8 ? 3 : kNBuf;
  __shared__ __attribute__((aligned(1024))) bf16 tiles[kBuf][kTileTok * kD];
  __shared__ __attribute__((aligned(1024))) char stage[F8 ? 2 : 1][F8 ? kF8StageBytes : 16];
  const bf16* __restrict__ cache = reinterpret_cast<const bf16*>(cache_v);
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][NB][2][64];
  __shared__ float alpha_s[2][NB][32];
  __shared__ float lrow_s[NB][32];
  __shared__ int pages_s[kMaxChunkPages];

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
  const bool score_wave = wave < NB;
  const bool value_wave = wave >= 2;
  const int pw = wave - 2;                       // value wave index: dims [256 pw, 256 pw + 256)
  const int64_t rows_total = (int64_t)Tq * H;

  // ---- page ids of this chunk, staged once
  const int page0 = tok_begin / page_size;
  const int npages = (tok_end - 1) / page_size - page0 + 1;
  for (int i = threadIdx.x; i < npages; i += blockDim.x)
    pages_s[i] = page_table[(int64_t)b * max_pages + page0 + i];

  // ---- per-lane DMA source offsets (loop invariant): LDS slot (t, c') of a
  // tile receives global chunk (t, c' ^ swz(t)).  Each wave copies 8 token rows.
  uint32_t dma_off[kDmaPerWave];
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u) {
    const int slot = (wave * kDmaPerWave + u) * 64 + lane;
    const int t = slot / kChunks;
    dma_off[u] = (uint32_t)(t * kChunks + ((slot % kChunks) ^ swz(t))) * 16u;
  }
  const uint32_t lds_tiles = lds_address(&tiles[0][0]);
  __syncthreads();
  auto issue_tile = [&](int it) {
    const int tok0 = tok_begin + it * kTileTok;
    const int page = __builtin_amdgcn_readfirstlane(pages_s[tok0 / page_size - page0]);
    const bf16* base = cache + ((int64_t)page * page_size + (tok0 % page_size)) * kD;
    const uint32_t lds0 =
        lds_tiles + (uint32_t)((it % kBuf) * kTileBytes + wave * kDmaPerWave * 1024);
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) dma16(base, dma_off[u], lds0 + u * 1024);
  };
  // FP8 (waves 1-3): this wave's seven of tile `it`'s 21 copies into staging
  // buffer it & 1 (wave 1 also the scales), and its third of the conversion
  // of a staged tile into tiles[it % 3]
  const int cw = wave - 1;
  auto f8_issue_part = [&](int it) {
    const int tok0 = tok_begin + it * kTileTok;
    const int page = __builtin_amdgcn_readfirstlane(pages_s[tok0 / page_size - page0]);
    const uint8_t* pg = reinterpret_cast<const uint8_t*>(cache_v) + (int64_t)page * page_size * (kF8Row + 4);
    const uint8_t* rows = pg + (int64_t)(tok0 % page_size) * kF8Row;
    const uint32_t dst = lds_address(&stage[it & 1][0]);
    const int n = cw == 0 ? 6 : 7;            // 6 + 7 + 7 row blocks, and the scales
    const int blk0 = cw == 0 ? 0 : 6 + 7 * (cw - 1);
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      if (u < n) {
        const int blk = blk0 + u;
        dma16(rows, (uint32_t)((blk * 64 + lane) * 16),
              __builtin_amdgcn_readfirstlane(dst + (uint32_t)blk * 1024u));
      }
    }
    if (cw == 0)
      dma16(pg + (int64_t)page_size * kF8Row + (tok0 % page_size) * 4, (uint32_t)((lane & 7) * 16),
            dst + kF8RowsBytes);
  };
  // wave 1 has no other work: it converts latent items 0..511 and every rope
  // item; the value waves 512..767 and 768..1023
  auto f8_convert_part = [&](int it) {
    char* dst = reinterpret_cast<char*>(&tiles[it % kBuf][0]);
    const int nvalid = tok_end - (tok_begin + it * kTileTok);
    if (cw == 0)
      f8_convert<8>(&stage[it & 1][0], dst, nvalid, lane, 64, 512, 0);
    else
      f8_convert<4>(&stage[it & 1][0], dst, nvalid, 256 + 256 * cw + lane, 64, 512 + 256 * cw, 256);
  };

  // ---- score waves: their 32 rows of the score operand, in registers
  const int my_row = row_base + wave * 32 + l32;
  const bool row_ok = score_wave && (my_row < R);
  const int my_i = row_ok ? my_row / H : 0;
  const int my_h = row_ok ? my_row % H : 0;
  const int my_limit = row_ok ? (L - Lq + my_i) : -1;   // last visible position
  bf16x8 qf[kD / 16];
  if (score_wave) {
    const bf16* qrow = abuf + ((int64_t)(q0 + my_i) * H + my_h) * kD + 8 * g;
    const uint32_t keep = row_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      u32x4 v = __builtin_bit_cast(u32x4, load_bf16x8(qrow + 16 * ks));
      v &= keep;
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // score operand: chunk 2ks+g of token l32 sits at qk_base[ks & 3] + 128 (ks >> 2)
  uint32_t qk_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qk_base[j] = (uint32_t)(l32 * kChunks + ((2 * j + g) ^ swz(l32))) * 16u;

  // value operand through the transposing LDS read: in each 16-lane group,
  // source lane 4j + q points at 4 dims (4q..4q+3 of the group's 16) of token
  // 4g + j + 8 L + 16 ks; lane 4q' + r receives dim 4q'+r of those 4 tokens.
  // The swizzle depends on the token: +16 tokens flips chunk bit 0 (a base of
  // its own), +8 tokens flips chunk bit 2, i.e. swaps the two e1 bases.
  // Address = pv_base[(db & 1) ^ L][ks] + 9216 L + 128 (db >> 1).
  uint32_t pv_base[2][2];
  {
    const int k = lane >> 4, sl = lane & 15, j = sl >> 2, q = sl & 3;
#pragma unroll
    for (int e1 = 0; e1 < 2; ++e1)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int t = 4 * g + j + 16 * ks;
        const int c = 32 * (pw & 1) + 4 * e1 + 2 * (k & 1) + (q >> 1);
        pv_base[e1][ks] = (uint32_t)(t * kChunks + (c ^ swz(t))) * 16u + 8u * (q & 1);
      }
  }

  f32x16 O[kDbPerPv][NB];
#pragma unroll
  for (int db = 0; db < kDbPerPv; ++db)
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) O[db][rb] = zero_f32x16();
  float m_run = -INFINITY, l_run = 0.f;

  // scores, online softmax and probability fragments of tile `it`.  The tile
  // fragments stream through a ring of kQkRing groups of 4 (LDS latency is
  // several MFMA groups long under load), so the matrix core never waits on a
  // read issued just before it.
  auto score_tile = [&](int it) {
    const char* tileb = reinterpret_cast<const char*>(&tiles[it % kBuf][0]);
    const int tok0 = tok_begin + it * kTileTok;
    constexpr int kGroups = kD / 64;          // 9 groups of 4 k-steps
    bf16x8 ring[kQkRing][4];
#pragma unroll
    for (int grp = 0; grp < kQkRing; ++grp)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ring[grp][j] = *reinterpret_cast<const bf16x8*>(tileb + qk_base[j] + 128 * grp);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc;
#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) {
      bf16x8 (&a)[4] = ring[grp % kQkRing];
      if (grp == 0)
        qk_mfma4_first(acc, a[0], qf[0], a[1], qf[1], a[2], qf[2], a[3], qf[3]);
      else if (grp == kGroups - 1)
        qk_mfma4_last(acc, a[0], qf[4 * grp], a[1], qf[4 * grp + 1], a[2], qf[4 * grp + 2], a[3],
                      qf[4 * grp + 3]);
      else
        qk_mfma4(acc, a[0], qf[4 * grp], a[1], qf[4 * grp + 1], a[2], qf[4 * grp + 2], a[3],
                 qf[4 * grp + 3]);
      if (grp + kQkRing < kGroups) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a[j] = *reinterpret_cast<const bf16x8*>(tileb + qk_base[j] + 128 * (grp + kQkRing));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pf0, pf1;
    const bool masked = tok0 + kTileTok - 1 > L - Lq;
    const float alpha = softmax_tile(acc, masked, tok0, my_limit, scale_log2e, m_run, l_run, pf0, pf1);
    pbuf[it & 1][wave][0][lane] = pf0;
    pbuf[it & 1][wave][1][lane] = pf1;
    if (g == 0) alpha_s[it & 1][wave][l32] = alpha;
  };

  // O^T[dim][row] += sum_tok tile[tok][dim] P[row][tok] over this value wave's
  // 256 dims: 16 (k-step, dim block) steps, transposed reads kPvRing steps ahead.
  auto value_tile = [&](int it) {
    const char* tileb = reinterpret_cast<const char*>(&tiles[it % kBuf][0]);
    constexpr int kSteps = 2 * kDbPerPv;
    auto frag_addr = [&](int step, int hl) {
      const int ks = step / kDbPerPv, db = step % kDbPerPv;
      return tileb + pv_base[(db & 1) ^ hl][ks] + kChunks * 16 * 8 * hl + 128 * (db >> 1);
    };
    v4bf16 ring[kPvRing][2];
#pragma unroll
    for (int st = 0; st < kPvRing; ++st) {
      ring[st][0] = ds_read_tr16(frag_addr(st, 0));
      ring[st][1] = ds_read_tr16(frag_addr(st, 1));
    }
    bf16x8 pb[2][NB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) pb[ks][rb] = pbuf[it & 1][rb][ks][lane];
    {  // rare: a row's running max grew past the threshold -> rescale its O
      float al[NB];
      bool any = false;
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        al[rb] = alpha_s[it & 1][rb][l32];
        any |= __any(al[rb] != 1.f);
      }
      if (any) {
        pv_drain<NB, kDbPerPv>(O);
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
#pragma unroll
          for (int db = 0; db < kDbPerPv; ++db) {
            O[db][rb] *= al[rb];
            asm volatile("" : "+a"(O[db][rb]));   // back to the accumulator file, block by block
          }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int ks = st / kDbPerPv, db = st % kDbPerPv;
      v4bf16 (&f)[2] = ring[st % kPvRing];
      const bf16x8 a = __builtin_shufflevector(f[0], f[1], 0, 1, 2, 3, 4, 5, 6, 7);
      pv_mfma<NB>(O[db], a, pb[ks]);
      if (st + kPvRing < kSteps) {
        f[0] = ds_read_tr16(frag_addr(st + kPvRing, 0));
        f[1] = ds_read_tr16(frag_addr(st + kPvRing, 1));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The sequence's last tile may end before its 32 rows do; the rows past the
  // end hold whatever the page held.  Zero them before the value waves read
  // them, so that zero probabilities never meet a NaN.
  auto zero_tail = [&](int it) {
    const int nvalid = tok_end - (tok_begin + it * kTileTok);
    if (nvalid < kTileTok) {
      u32x4* rows = reinterpret_cast<u32x4*>(&tiles[it % kBuf][0]) + nvalid * kChunks;
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int i = threadIdx.x; i < (kTileTok - nvalid) * kChunks; i += blockDim.x) rows[i] = z;
      __syncthreads();
    }
  };

  // ---- pipeline: score waves run one tile ahead of value waves
  if constexpr (F8) {
    // every copy is issued by waves 1-3; before each barrier a wave waits for
    // its own copies (all seven per tile land in order) and its own LDS writes
    const bool copier = wave >= 1;
    if (copier) {
      f8_issue_part(0);
      if (ntiles > 1) {
        f8_issue_part(1);
        wait_vmcnt<7>();                        // tile 0's copies (tile 1's may fly)
      } else {
        wait_vmcnt<0>();
      }
    }
    __syncthreads();                            // staged tile 0 complete
    if (copier) {
      f8_convert_part(0);
      wait_vmcnt<0>();
      __builtin_amdgcn_s_waitcnt(0xc07f);
    }
    __syncthreads();                            // tile 0 converted, staged tile 1 complete
    if (copier) {
      if (ntiles > 2) f8_issue_part(2);         // into staging 0 (tile 0 is converted)
      if (ntiles > 1) f8_convert_part(1);
    }
    if (score_wave) score_tile(0);
    for (int it = 0; it < ntiles; ++it) {
      if (copier) {
        wait_vmcnt<0>();                        // staged tile it+2 landed
        __builtin_amdgcn_s_waitcnt(0xc07f);     // own conversion of tile it+1 written
      }
      __syncthreads();   // P(it) and tile it+1 visible; tile it-1 fully consumed
      if (copier) {
        if (it + 3 < ntiles) f8_issue_part(it + 3);   // staging of tile it+1, converted already
        if (it + 2 < ntiles) f8_convert_part(it + 2);  // into tiles[(it - 1) % 3]
      }
      if (score_wave && it + 1 < ntiles) score_tile(it + 1);
      if (value_wave) value_tile(it);
    }
  } else {
    for (int p = 0; p < kNBuf - 1; ++p)
      if (p < ntiles) issue_tile(p);
    wait_tiles_ahead(min(kNBuf - 2, ntiles - 1));
    __syncthreads();
    zero_tail(0);
    if (score_wave) score_tile(0);
    for (int it = 0; it < ntiles; ++it) {
      // tile it+1 must have landed: tiles issued after it are min(ntiles-1, it+2) - (it+1)
      wait_tiles_ahead(min(ntiles - 1, it + kNBuf - 2) - (it + 1));
      __syncthreads();   // P(it) and tile it+1 visible; tile it-1 fully consumed
      if (it + kNBuf - 1 < ntiles) issue_tile(it + kNBuf - 1);
      if (it + 1 < ntiles) zero_tail(it + 1);
      if (score_wave && it + 1 < ntiles) score_tile(it + 1);
      if (value_wave) value_tile(it);
    }
  }
  if (value_wave) pv_drain<NB, kDbPerPv>(O);

  // ---- epilogue: row statistics, then normalised partials
  if (score_wave) {
    if (g == 0) lrow_s[wave][l32] = l_run;
    if (g == 0 && my_row < R) {
      const int64_t rowg = (int64_t)(q0 + my_i) * H + my_h;
      lse[(int64_t)s * rows_total + rowg] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
    }
  }
  __syncthreads();
  if (!value_wave) return;
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = row_base + rb * 32 + l32;
    if (row >= R) continue;
    const float lr = lrow_s[rb][l32];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    const int64_t rowg = (int64_t)(q0 + row / H) * H + row % H;
    bf16* dst = opart + ((int64_t)s * rows_total + rowg) * kDC + pw * 256;
    // lane half g holds columns 8 q4 + 4 g .. + 3; one swap of the lane
    // halves per dword gives the lower half all of group q4 = 2p and the
    // upper half all of group 2p + 1, written as 16 bytes per lane
#pragma unroll
    for (int db = 0; db < kDbPerPv; ++db)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t a[2], bq[2];   // groups 2p (a) and 2p + 1 (bq), this lane's 4 columns as 2 dwords
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          a[k] = pack_bf16x2(O[db][rb][8 * p + 2 * k] * inv, O[db][rb][8 * p + 2 * k + 1] * inv);
          bq[k] = pack_bf16x2(O[db][rb][8 * p + 4 + 2 * k] * inv, O[db][rb][8 * p + 4 + 2 * k + 1] * inv);
        }
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t send = g ? a[k] : bq[k];
          const auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
          const uint32_t got = g ? r[0] : r[1];   // the other half's dword
          w[k] = g ? got : a[k];
          w[2 + k] = g ? bq[k] : got;
        }
        *reinterpret_cast<u32x4*>(dst + 32 * db + 16 * p + 8 * g) = w;
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
// One workgroup per (query, head) row: split weights once, then each thread
// merges four consecutive latent elements across the splits.
constexpr int kMaxSplits = 1024;

template <typename T, typename P>
__global__ __launch_bounds__(128) void combine_kernel(const P* __restrict__ opart,
                                                      const float* __restrict__ lse,
                                                      const int32_t* __restrict__ cu_q,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int batch, int Tq, int H, int dc, int chunk,
                                                      T* __restrict__ olat) {
  __shared__ float w_s[kMaxSplits];
  __shared__ float red[2];
  __shared__ CuStage cu_st;
  const int32_t* cu = stage_cu(cu_st, cu_q, batch);
  const int64_t rowg = blockIdx.x;
  const int t = (int)(rowg / H);
  const int b = seq_of_token(cu, batch, t);
  const int L = seq_lens[b];
  const int S_b = min((L + chunk - 1) / chunk, kMaxSplits);
  const int64_t rows_total = (int64_t)Tq * H;
  if (threadIdx.x < 64) {
    float m = -INFINITY;
    for (int s = threadIdx.x; s < S_b; s += 64) m = fmaxf(m, lse[s * rows_total + rowg]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.f;
    for (int s = threadIdx.x; s < S_b; s += 64) {
      const float x = lse[s * rows_total + rowg];
      const float w = (x == -INFINITY) ? 0.f : exp2f(x - m);
      w_s[s] = w;
      sum += w;
    }
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (threadIdx.x == 0) red[0] = sum > 0.f ? 1.f / sum : 0.f;
  }
  __syncthreads();
  const float inv = red[0];
  for (int j = 4 * threadIdx.x; j < dc; j += 4 * blockDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S_b; ++s) {
      const f32x4 v = load4_f32(opart + (s * rows_total + rowg) * dc + j);
      acc += w_s[s] * v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) olat[rowg * dc + j + e] = from_f32<T>(acc[e] * inv);
  }
}

}  // namespace

namespace {

constexpr int kListThreads = 1024;
constexpr int kListBins = kMaxChunkTokens / 32 + 1;   // tile counts of a split: 1 .. chunk / 32
static_assert(kListBins <= kListThreads, "one thread per tile count in the rank scan");

// Busy work items of a split-KV launch, balanced over the 8 XCDs.  A split
// (b, s) of sequence b brings min(RQ, ceil(rows_b / rows)) row groups, which
// stay together on one XCD (they read the same tiles through its L2).  The
// splits are ranked by tile count, largest first (counting sort), and dealt
// to the XCDs in a snake (ranks 16 k + x and 16 k + 15 - x go to XCD x), so
// every XCD gets a similar mix of long and short splits and starts its long
// ones first.  Header: [0] busy items, [1 + x] items of XCD x, [9 + x] where
// they start; grp (batch x S_max entries) holds the ranked splits.  One
// workgroup: ranks come from atomic counters in LDS, so equal-size splits
// take an arbitrary order among themselves (each item's results do not
// depend on where it runs).
__global__ __launch_bounds__(kListThreads) void work_list_kernel(const int32_t* __restrict__ cu_q,
                                                                 const int32_t* __restrict__ seq_lens, int batch,
                                                                 int H, int rows, int chunk, int S_max, int RQ,
                                                                 int* __restrict__ hdr, int2* __restrict__ items,
                                                                 int2* __restrict__ grp) {
  __shared__ int bins[kListBins];
  __shared__ int tot[kListThreads];
  __shared__ int n_groups, xcount[8], xstart[8];
  const int tid = threadIdx.x;
  for (int i = tid; i < kListBins; i += kListThreads) bins[i] = 0;
  __syncthreads();
  const int per = (batch + kListThreads - 1) / kListThreads;
  const int b0 = min(batch, tid * per), b1 = min(batch, b0 + per);
  auto groups = [&](int b) { return min(RQ, ((cu_q[b + 1] - cu_q[b]) * H + rows - 1) / rows); };
  auto splits = [&](int b) { return min(S_max, (seq_lens[b] + chunk - 1) / chunk); };
  auto tiles = [&](int b, int sp) { return (min(chunk, seq_lens[b] - sp * chunk) + 31) / 32; };
  // histogram of the splits' tile counts
  for (int b = b0; b < b1; ++b) {
    if (groups(b) <= 0) continue;
    const int ns = splits(b);
    for (int sp = 0; sp < ns; ++sp) atomicAdd(&bins[tiles(b, sp)], 1);
  }
  __syncthreads();
  // first rank of each tile count, largest count first: a block-wide scan
  // with thread t on count kListBins - 1 - t
  const int cnt = tid < kListBins ? bins[kListBins - 1 - tid] : 0;
  tot[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kListBins; off <<= 1) {
    const int v = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  if (tid < kListBins) bins[kListBins - 1 - tid] = tot[tid] - cnt;
  if (tid == kListBins - 1) n_groups = tot[tid];
  __syncthreads();
  for (int b = b0; b < b1; ++b) {
    const int ng = groups(b);
    if (ng <= 0) continue;
    const int ns = splits(b);
    for (int sp = 0; sp < ns; ++sp) {
      const int r = atomicAdd(&bins[tiles(b, sp)], 1);
      grp[r] = make_int2(b, (sp << 12) | (ng - 1));
    }
  }
  __threadfence_block();
  __syncthreads();
  // XCD x = tid / 128 takes its splits j = 0, 1, ... (rank 16 (j / 2) + x for
  // even j, + 15 - x for odd j); 128 threads per XCD each take a contiguous
  // range of j, and a scan of their row-group counts places their items
  const int G = n_groups;
  const int x = tid >> 7, lt = tid & 127;
  const int rem = G % 16;
  const int gx = 2 * (G / 16) + (x < rem ? 1 : 0) + (15 - x < rem ? 1 : 0);
  auto rank = [&](int j) { return 16 * (j >> 1) + ((j & 1) ? 15 - x : x); };
  const int jper = (gx + 127) / 128;
  const int j0 = min(gx, lt * jper), j1 = min(gx, j0 + jper);
  int mine = 0;
  for (int j = j0; j < j1; ++j) mine += (grp[rank(j)].y & 4095) + 1;
  tot[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 128; off <<= 1) {
    const int v = lt >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  if (lt == 127) xcount[x] = tot[tid];
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int y = 0; y < 8; ++y) {
      xstart[y] = acc;
      hdr[1 + y] = xcount[y];
      hdr[9 + y] = acc;
      acc += xcount[y];
    }
    hdr[0] = acc;
  }
  __syncthreads();
  int pos = xstart[x] + tot[tid] - mine;
  for (int j = j0; j < j1; ++j) {
    const int2 g = grp[rank(j)];
    const int sp = g.y >> 12, ng = (g.y & 4095) + 1;
    for (int rq = 0; rq < ng; ++rq) items[pos++] = make_int2(g.x, (sp << 12) | rq);
  }
}

}  // namespace

void launch_splitkv(int elem, const SplitPlan& plan, const void* abuf, const void* cache,
                    const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                    int max_pages, int batch, int Tq, int H, int dc, int dr, int page_size,
                    float scale, float* opart, float* lse, bool fp8, void* work, hipStream_t st) {
  // bf16 layers: the absorbed queries already carry scale * log2(e)
  const float scale_log2e = elem == 2 ? 1.f : scale * 1.4426950408889634f;
  if (elem == 2) {
    const int nblocks = batch * plan.S_max * plan.RQ;
    const int2* items = nullptr;
    const int* list_hdr = nullptr;
    if (plan.list && (plan.NB == 8 || plan.NB == 128)) {
      int* hdr = reinterpret_cast<int*>(work);
      int2* list = reinterpret_cast<int2*>(hdr + kListHeaderInts);
      int2* grp = list + (size_t)batch * plan.S_max * plan.RQ;
      work_list_kernel<<<1, kListThreads, 0, st>>>(cu_q, seq_lens, batch, H, plan.NB == 128 ? 128 : 64,
                                                   plan.chunk, plan.S_max, plan.RQ, hdr, list, grp);
      items = list;
      list_hdr = hdr;
    }
    switch (plan.NB) {
      case 8:
        launch_splitkv_x8(plan, abuf, cache, cu_q, seq_lens, page_table, max_pages, batch, Tq, H,
                          page_size, opart, lse, fp8, items, list_hdr, st);
        break;
      case 128:
        launch_splitkv_r128(plan, abuf, cache, cu_q, seq_lens, page_table, max_pages, batch, Tq, H,
                            page_size, opart, lse, items, list_hdr, st);
        break;
      default:
        if (fp8)
          splitkv_bf16_kernel<1, true><<<nblocks, 256, 0, st>>>(
              (const bf16*)abuf, cache, cu_q, seq_lens, page_table, max_pages, batch, H, page_size,
              plan.chunk, plan.S_max, plan.RQ, scale_log2e, Tq, (bf16*)opart, lse);
        else
          splitkv_bf16_kernel<1, false><<<nblocks, 256, 0, st>>>(
              (const bf16*)abuf, cache, cu_q, seq_lens, page_table, max_pages, batch, H, page_size,
              plan.chunk, plan.S_max, plan.RQ, scale_log2e, Tq, (bf16*)opart, lse);
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

void launch_combine(int elem, const SplitPlan& plan, const void* opart, bool part_bf16, const float* lse,
                    const int32_t* cu_q, const int32_t* seq_lens, int batch, int Tq, int H, int dc,
                    void* olat, hipStream_t st) {
  const unsigned rows = (unsigned)((int64_t)Tq * H);
  if (elem == 2)
    if (part_bf16)
      combine_kernel<bf16, bf16><<<rows, 128, 0, st>>>((const bf16*)opart, lse, cu_q, seq_lens, batch, Tq,
                                                       H, dc, plan.chunk, (bf16*)olat);
    else
      combine_kernel<bf16, float><<<rows, 128, 0, st>>>((const float*)opart, lse, cu_q, seq_lens, batch, Tq, H, dc,
                                               plan.chunk, (bf16*)olat);
  else
    combine_kernel<float, float><<<rows, 128, 0, st>>>((const float*)opart, lse, cu_q, seq_lens, batch, Tq, H, dc,
                                                plan.chunk, (float*)olat);
}

}  // namespace mla

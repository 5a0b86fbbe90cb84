// Split-KV attention over the paged latent cache, 64 query rows per workgroup,
// eight waves: two per SIMD, so that one wave's LDS reads and softmax overlap
// the other's matrix-core work.
//
// The step is the same dense contraction as in the other split-KV kernels
// ("Multi-head Latent Attention: the KV cache, compressed", sections "The one
// formula" and "Absorption: the part that makes it free": every head scores
// the same cached row [c | k_rope]):
//     S[row][t]  = scale * A[row] . cache[t]          (K = 576)
//     O[row][:] += softmax_t(S) cache[t][:512]        (K = tokens)
// with an online softmax per row and normalised partials + log2-sum-exp per
// (row, split).
//
// Roles (waves w and w + 4 share a SIMD):
//   * score wave w < 4: 16 whole rows (16 w .. 16 w + 15).  Its score operand
//     (16 rows x 576, 72 registers) lives in AGPRs and is the B operand of the
//     16x16x32 bf16 matrix instruction; the tile rows are the A operand, read
//     from LDS (two 16-token halves per k-step).  It runs the online softmax
//     of its rows over whole tiles and writes bf16 probabilities, already in
//     the value product's operand layout, to a double-buffered LDS block.
//   * value wave v = w - 4: O^T for latent columns [128 v, 128 v + 128) of all
//     64 rows (8 blocks of 32x32, 128 AGPRs), value operand read with the
//     transposing LDS load, probabilities as the B operand.  Value waves also
//     issue the tile copies (global_load_lds, 9 per wave per tile) and work
//     one tile behind the score waves.
// One barrier per tile publishes the tile that landed and the probabilities
// of the previous one.
//
// F8 (MLA_CACHE_FP8 pages): three bf16 tiles and two FP8 staging buffers; the
// value waves copy each FP8 tile to staging one tile ahead (and convert tile
// 0 before the loop); the score waves convert all of tile it+1 -- four
// latent items and one rope item per lane, its staging reads issued before
// their score MFMAs of tile it, the conversions and writes after their
// softmax, where they would otherwise wait at the barrier for the value
// waves (on the value waves' chain the conversion measured 1.5-1.7k of a
// 3.5k-clock tile; spread between the score MFMAs its LDS writes held up
// the operand reads).  Score and value waves run separate loops with the same
// barrier sequence, so their operands (query, O) can share the AGPR file.
#include "attn_tile.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kX8Rows = 64;
constexpr int kX8Buf = 4;                               // tiles resident: 2 in use, 2 in flight
constexpr int kX8Dma = kTileBytes / 16 / 64 / 4;        // 9 copies per value wave per tile
constexpr int kQSteps = kD / 32;                        // 18 k-steps of the 16x16x32 score product
constexpr int kX8Ring = 6;                              // k-steps of tile reads in flight (2 reads each)

template <bool F8>
__global__ __launch_bounds__(512, 1) void splitkv_bf16_x8_kernel(
    const bf16* __restrict__ abuf, const void* __restrict__ cache_v, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, int H, int page_size, int chunk, int S_max, int RQ, int Tq,
    bf16* __restrict__ opart, float* __restrict__ lse, const int2* __restrict__ items,
    const int* __restrict__ list_hdr) {
  constexpr int kBuf = F8 ? 3 : kX8Buf;
  __shared__ __attribute__((aligned(1024))) bf16 tiles[kBuf][kTileTok * kD];
  __shared__ __attribute__((aligned(1024))) char stage[F8 ? 2 : 1][F8 ? kF8StageBytes : 16];
  const bf16* __restrict__ cache = reinterpret_cast<const bf16*>(cache_v);
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][4][64];   // [tile parity][2 rb + ks][lane]
  __shared__ float alpha_s[2][kX8Rows];   // rescale factor of O per row, per tile parity
  __shared__ float lrow_s[kX8Rows];       // row sums at the end
  __shared__ int pages_s[kMaxChunkPages];

  int b, s, rq;
  if (!split_work_item(items, list_hdr, batch, S_max, RQ, &b, &s, &rq)) return;

  const int q0 = cu_q[b];
  const int Lq = cu_q[b + 1] - q0;
  const int L = seq_lens[b];
  const int R = Lq * H;
  const int row_base = rq * kX8Rows;
  const int tok_begin = s * chunk;
  if (row_base >= R || tok_begin >= L) return;
  // keys past the last visible position of the block's last row are masked
  // for every row of the block: stop there, keeping at least one token so the
  // split still writes its (empty) partial
  const int last_vis = L - Lq + (min(row_base + kX8Rows, R) - 1) / H;
  const int tok_end = min(min(tok_begin + chunk, L), max(tok_begin + 1, last_vis + 1));
  const int ntiles = (tok_end - tok_begin + kTileTok - 1) / kTileTok;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows_total = (int64_t)Tq * H;
  const uint32_t lds_tiles = lds_address(&tiles[0][0]);

  const int page0 = tok_begin / page_size;
  const int npages = (tok_end - 1) / page_size - page0 + 1;
  for (int i = threadIdx.x; i < npages; i += blockDim.x)
    pages_s[i] = page_table[(int64_t)b * max_pages + page0 + i];
  __syncthreads();

  if (wave < 4) {
    // =========================== score waves ===========================
    const int G = lane >> 4, c16 = lane & 15;
    const int row = row_base + 16 * wave + c16;   // this lane's row (column of S^T)
    const bool valid = row < R;
    const int qi = valid ? row / H : 0, h = valid ? row % H : 0;
    const int lim = valid ? L - Lq + qi : -1;
    // score operand: B fragment of k-step st holds dims 32 st + 8 G .. + 7 of
    // the row.  Rows past R read row 0 of the block (finite values; their
    // results are never stored).  Loaded straight into AGPRs.
    bf16x8 qf[kQSteps];
    {
      const bf16* src = abuf + ((int64_t)(q0 + qi) * H + h) * kD + 8 * G;
#pragma unroll
      for (int st = 0; st < kQSteps; ++st) {
        qf[st] = load_bf16x8(src + 32 * st);
        asm volatile("" : "+a"(qf[st]));
      }
    }
    // A operand of (token half m, k-step st): token 16 m + c16, chunk 4 st + G
    // = base[m][st & 1] + 128 bytes per pair of steps (the swizzle stays in the
    // low three chunk bits).
    uint32_t a_base[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int t = 16 * m + c16;
        a_base[m][p] = (uint32_t)(t * kChunks + ((4 * p + G) ^ swz(t))) * 16u;
      }
    // this lane's probabilities: value-product B fragment f = 2 rb + m (rb =
    // wave >> 1), lane 16 (wave & 1) + c16 + 32 (G >> 1), bytes 8 (G & 1) ..
    const int lp = 16 * (wave & 1) + c16 + 32 * (G >> 1);
    const int fb = 2 * (wave >> 1);
    float m_run = -INFINITY, l_run = 0.f;

    if constexpr (F8) __syncthreads();   // the value waves' staging prologue
    for (int it = 0; it <= ntiles; ++it) {
      if constexpr (F8) __builtin_amdgcn_s_waitcnt(0xc07f);   // own conversion writes done
      __syncthreads();   // tile `it` landed; probabilities of tile it-1 published
      if (it == ntiles) break;
      const char* tileb = reinterpret_cast<const char*>(&tiles[it % kBuf][0]);
      // FP8: this lane's items of tile it+1 (its staging landed before the
      // barrier): latent items 64 wave + lane + 256 u, u < 4 (row i / 32,
      // codes 16 (i % 32) .. + 15 -> bf16 chunks 2 (i % 32), + 1) and rope
      // item 64 wave + lane (row i / 8, chunk 64 + i % 8); rows past the
      // tile's valid rows are written as zeros.  Their staging reads go out
      // now, the conversions and writes after this tile's softmax.
      const u32x4 zero4 = {0u, 0u, 0u, 0u};
      u32x4 cw[4], rw = zero4;
      float cs[4];
      int nv1 = 0;
      char* ctile = reinterpret_cast<char*>(&tiles[(it + 1) % kBuf][0]);
      const bool conv = F8 && it + 1 < ntiles;
      if constexpr (F8) {
        if (conv) {
          const char* stg = &stage[(it + 1) & 1][0];
          const float* scales = reinterpret_cast<const float*>(stg + kF8RowsBytes);
          nv1 = tok_end - (tok_begin + (it + 1) * kTileTok);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 64 * wave + lane + 256 * u, t = i >> 5;
            cw[u] = t < nv1 ? *reinterpret_cast<const u32x4*>(stg + t * kF8Row + (i & 31) * 16) : zero4;
            cs[u] = t < nv1 ? scales[t] : 0.f;
          }
          const int i = 64 * wave + lane, t = i >> 3;
          if (t < nv1) rw = *reinterpret_cast<const u32x4*>(stg + t * kF8Row + 512 + (i & 7) * 16);
        }
      }
      auto put_latent = [&](int u) {
        const int i = 64 * wave + lane + 256 * u, t = i >> 5, k = i & 31;
        u32x4 lo = zero4, hi = zero4;
        if (t < nv1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[u][q], cs[u], false));
            const uint32_t y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[u][q], cs[u], true));
            if (q < 2) {
              lo[2 * q] = x;
              lo[2 * q + 1] = y;
            } else {
              hi[2 * q - 4] = x;
              hi[2 * q - 3] = y;
            }
          }
        }
        const int sw = swz(t);
        *reinterpret_cast<u32x4*>(ctile + (t * kChunks + ((2 * k) ^ sw)) * 16) = lo;
        *reinterpret_cast<u32x4*>(ctile + (t * kChunks + ((2 * k + 1) ^ sw)) * 16) = hi;
      };
      f32x4 acc[2];
      {
        bf16x8 ring[kX8Ring][2];
#pragma unroll
        for (int st = 0; st < kX8Ring; ++st)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            ring[st][m] = *reinterpret_cast<const bf16x8*>(tileb + a_base[m][st & 1] + 128 * (st >> 1));
#pragma unroll
        for (int st = 0; st < kQSteps; ++st) {
          bf16x8 (&a)[2] = ring[st % kX8Ring];
          if (st == 0) qk16x2_first(acc[0], acc[1], a[0], a[1], qf[0]);
          else qk16x2(acc[0], acc[1], a[0], a[1], qf[st]);
          if (st + kX8Ring < kQSteps) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
              a[m] = *reinterpret_cast<const bf16x8*>(tileb + a_base[m][(st + kX8Ring) & 1] +
                                                      128 * ((st + kX8Ring) >> 1));
          }
        }
        qk16_drain(acc[0], acc[1]);
      }
      // online softmax of this lane's row over the tile's 32 tokens
      // (token 16 m + 4 G + i of acc[m][i])
      const int tok0 = tok_begin + it * kTileTok;
      const bool masked = tok0 + kTileTok - 1 > L - Lq;
      // scores are already in log2 units (the absorbed queries carry the scale)
      if (masked) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tok0 + 16 * m + 4 * G + i > lim) acc[m][i] = -INFINITY;
      }
      float tmax = max_raw(max_raw(max_raw(acc[0][0], acc[0][1]), max_raw(acc[0][2], acc[0][3])),
                           max_raw(max_raw(acc[1][0], acc[1][1]), max_raw(acc[1][2], acc[1][3])));
      tmax = quad_max(tmax);
      const float m_new = (tmax > m_run + kRescaleThreshold) ? tmax : m_run;
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      float p[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[m][i] = __builtin_amdgcn_exp2f(acc[m][i] - m_ref);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x4 pv = {from_f32<bf16>(p[m][0]), from_f32<bf16>(p[m][1]), from_f32<bf16>(p[m][2]),
                     from_f32<bf16>(p[m][3])};
        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(&pbuf[it & 1][fb + m][lp]) + 8 * (G & 1)) = pv;
      }
      float rs = ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
      rs = quad_sum(rs);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (G == 0) alpha_s[it & 1][16 * wave + c16] = alpha;
      if constexpr (F8) {   // tile it+1's conversion, in the time the barrier would otherwise take
        if (conv) {
#pragma unroll
          for (int u = 0; u < 4; ++u) put_latent(u);
          const int i = 64 * wave + lane, t = i >> 3;
          *reinterpret_cast<u32x4*>(ctile + (t * kChunks + 64 + ((i & 7) ^ swz(t))) * 16) = rw;
        }
      }
    }
    if (G == 0) lrow_s[16 * wave + c16] = l_run;
    __syncthreads();   // row sums published
    if (G == 0 && valid) {
      const int64_t rowg = (int64_t)(q0 + qi) * H + h;
      lse[(int64_t)s * rows_total + rowg] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
    }
  } else {
    // =========================== value waves ===========================
    const int v = wave - 4;
    const int g = lane >> 5, l32 = lane & 31;
    uint32_t dma_off[kX8Dma];
#pragma unroll
    for (int u = 0; u < kX8Dma; ++u) {
      const int slot = (v * kX8Dma + u) * 64 + lane;
      const int t = slot / kChunks;
      dma_off[u] = (uint32_t)(t * kChunks + ((slot % kChunks) ^ swz(t))) * 16u;
    }
    auto issue_tile = [&](int it) {
      const int tok0 = tok_begin + it * kTileTok;
      const int page = __builtin_amdgcn_readfirstlane(pages_s[tok0 / page_size - page0]);
      const bf16* base = cache + ((int64_t)page * page_size + (tok0 % page_size)) * kD;
      const uint32_t lds0 =
          lds_tiles + (uint32_t)((it % kBuf) * kTileBytes + v * kX8Dma * 1024);
#pragma unroll
      for (int u = 0; u < kX8Dma; ++u) dma16(base, dma_off[u], lds0 + u * 1024);
    };
    // FP8: this wave's share of tile it's copies into staging buffer it & 1
    // (five of the twenty 1 KB row blocks; wave 0 also the scales)
    auto f8_issue_part = [&](int it) {
      const int tok0 = tok_begin + it * kTileTok;
      const int page = __builtin_amdgcn_readfirstlane(pages_s[tok0 / page_size - page0]);
      const uint8_t* pg = reinterpret_cast<const uint8_t*>(cache_v) + (int64_t)page * page_size * (kF8Row + 4);
      const uint8_t* rows = pg + (int64_t)(tok0 % page_size) * kF8Row;
      const uint32_t dst = lds_address(&stage[it & 1][0]);
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        const int blk = 5 * v + u;
        dma16(rows, (uint32_t)((blk * 64 + lane) * 16), dst + blk * 1024);
      }
      if (v == 0)
        dma16(pg + (int64_t)page_size * kF8Row + (tok0 % page_size) * 4, (uint32_t)((lane & 7) * 16),
              dst + kF8RowsBytes);
    };
    // tile 0, before the loop: all of its latent and rope items (the score
    // waves convert every later tile)
    auto f8_convert_tile = [&](int it) {
      f8_convert<4>(&stage[it & 1][0], reinterpret_cast<char*>(&tiles[it % kBuf][0]),
                    tok_end - (tok_begin + it * kTileTok), 64 * v + lane, 256, kTileTok * 32, 0);
    };
    // value operand (transposing read, natural token order): in 16-lane group
    // G, source lane 4 j + q points at dims 4q..4q+3 of the group's 16 dims,
    // token 16 ks + 8 (G >> 1) + 4 r + j; result lane i gets dim i of those 4
    // tokens.  Base per (ks, r, db & 1); db >> 1 adds 8 chunks (128 bytes).
    uint32_t pv_base[2][2][2];
    {
      const int G = lane >> 4, j = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int e1 = 0; e1 < 2; ++e1) {
            const int t = 16 * ks + 8 * (G >> 1) + 4 * r + j;
            const int c = 16 * v + 4 * e1 + 2 * (G & 1) + (q >> 1);
            pv_base[ks][r][e1] = (uint32_t)(t * kChunks + (c ^ swz(t))) * 16u + 8u * (q & 1);
          }
    }
    f32x16 O[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        O[db][rb] = zero_f32x16();
        asm volatile("" : "+a"(O[db][rb]));   // accumulators live in AGPRs from the start
      }

    // value operands of dim blocks 2h, 2h + 1, both k-steps
    auto load_pv_operands = [&](const char* tb, int h, v4bf16 (&f)[2][2][2]) {
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int db = 2 * h + d;
            f[d][ks][r] = ds_read_tr16(tb + pv_base[ks][r][db & 1] + 128 * (db >> 1));
          }
    };
    auto pv_mfmas = [&](int h, const v4bf16 (&f)[2][2][2], const bf16x8 (&pb)[2][2]) {
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = __builtin_shufflevector(f[d][ks][0], f[d][ks][1], 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 pr[2] = {pb[0][ks], pb[1][ks]};
          pv_mfma<2>(O[2 * h + d], a, pr);
        }
    };

    if constexpr (F8) {
      f8_issue_part(0);
      if (ntiles > 1) f8_issue_part(1);
      if (ntiles > 1) {
        if (v == 0) wait_vmcnt<6>();
        else wait_vmcnt<5>();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();   // staged tile 0 complete
      f8_convert_tile(0);
    } else {
      issue_tile(0);
      if (ntiles > 1) issue_tile(1);
    }
    for (int it = 0; it <= ntiles; ++it) {
      if constexpr (F8) {
        // own copies of tile it+1 landed; own conversion writes of tile it done
        wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xc07f);
      } else if (it < ntiles) {
        if (it + 1 < ntiles) wait_vmcnt<kX8Dma>();
        else wait_vmcnt<0>();
      }
      __syncthreads();   // tile `it` landed; probabilities of tile it-1 published
      if constexpr (F8) {
        if (it + 2 < ntiles) f8_issue_part(it + 2);   // staging of tile it, converted already
      } else {
        if (it + 2 < ntiles) issue_tile(it + 2);
      }
      // then the LDS reads (probabilities, rescale factors, value operands of
      // the first half), whose latency runs under the tail-zeroing below
      const int pt = (it - 1) & 1;
      const char* tb = reinterpret_cast<const char*>(&tiles[(it + kBuf - 1) % kBuf][0]);
      bf16x8 pb[2][2];
      float al[2];
      v4bf16 f0[2][2][2];
      if (it > 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) pb[rb][ks] = pbuf[pt][2 * rb + ks][lane];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) al[rb] = alpha_s[pt][32 * rb + l32];
        load_pv_operands(tb, 0, f0);
      }
      if (!F8 && it < ntiles) {
        // rows past the sequence's end hold whatever the page held; zero their
        // value columns so that zero probabilities never meet a NaN (the FP8
        // conversion writes those rows as zeros itself)
        const int nvalid = tok_end - (tok_begin + it * kTileTok);
        if (nvalid < kTileTok) {
          char* tz = reinterpret_cast<char*>(&tiles[it % kBuf][0]);
          const u32x4 z = {0u, 0u, 0u, 0u};
          for (int i = threadIdx.x - 256; i < (kTileTok - nvalid) * (kDC / 8); i += 256)
            *reinterpret_cast<u32x4*>(tz + (nvalid + i / (kDC / 8)) * kD * 2 + (i % (kDC / 8)) * 16) = z;
        }
      }
      if (it == 0) continue;
      bool any = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) any |= __any(al[rb] != 1.f);
      if (any) {   // rare: a running max moved past the threshold
        pv_drain<2, 4>(O);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            O[db][rb] *= al[rb];
            asm volatile("" : "+a"(O[db][rb]));
          }
      }
      v4bf16 f1[2][2][2];
      load_pv_operands(tb, 1, f1);
      pv_mfmas(0, f0, pb);
      pv_mfmas(1, f1, pb);
    }
    pv_drain<2, 4>(O);
    __syncthreads();   // row sums published
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = row_base + 32 * rb + l32;
      if (row >= R) continue;
      const float l = lrow_s[32 * rb + l32];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int64_t rowg = (int64_t)(q0 + row / H) * H + row % H;
      bf16* dst = opart + ((int64_t)s * rows_total + rowg) * kDC + 128 * v;
      // lane half g holds columns 8 q4 + 4 g .. + 3; one swap of the lane
      // halves per dword gives the lower half all of group q4 = 2p and the
      // upper half all of group 2p + 1, written as 16 bytes per lane
#pragma unroll
      for (int db = 0; db < 4; ++db)
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
}

}  // namespace

void launch_splitkv_x8(const SplitPlan& plan, const void* abuf, const void* cache,
                       const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                       int max_pages, int batch, int Tq, int H, int page_size, void* opart,
                       float* lse, bool fp8, const int2* items, const int* list_hdr, hipStream_t st) {
  const int nblocks = items ? work_list_grid(batch, plan) : batch * plan.S_max * plan.RQ;
  if (fp8)
    splitkv_bf16_x8_kernel<true><<<nblocks, 512, 0, st>>>(
        (const bf16*)abuf, cache, cu_q, seq_lens, page_table, max_pages, batch, H, page_size,
        plan.chunk, plan.S_max, plan.RQ, Tq, (bf16*)opart, lse, items, list_hdr);
  else
    splitkv_bf16_x8_kernel<false><<<nblocks, 512, 0, st>>>(
        (const bf16*)abuf, cache, cu_q, seq_lens, page_table, max_pages, batch, H, page_size,
        plan.chunk, plan.S_max, plan.RQ, Tq, (bf16*)opart, lse, items, list_hdr);
}

}  // namespace mla

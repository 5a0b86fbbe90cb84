// Split-KV attention over the paged latent cache, 64 query rows per workgroup,
// eight waves, software-pipelined across tiles.
//
// The step is the dense contraction of the other split-KV kernels
// ("Multi-head Latent Attention: the KV cache, compressed", sections "The one
// formula" and "Absorption: the part that makes it free": every head scores
// the same cached row [c | k_rope]):
//     S[row][t]  = A[row] . cache[t]                  (K = 576, log2 units)
//     O[row][:] += softmax_t(S) cache[t][:512]        (K = tokens)
// with an online softmax per row and normalised partials + log2-sum-exp per
// (row, split).
//
// Roles (waves w and w + 4 share a SIMD):
//   * score wave w < 4: 16 whole rows.  In loop step i it issues the score
//     matrix instructions of tile i and, between them, runs the softmax of
//     tile i - 1 (whose scores it kept in registers), so the vector work of
//     the softmax hides under the matrix-core work instead of following it.
//     Probabilities of tile i - 1 go to LDS in the value product's operand
//     layout.
//   * value wave v = w - 4: O^T for latent columns [128 v, 128 v + 128) of all
//     64 rows (128 AGPRs).  In step i it accumulates tile i - 2 from the value
//     operand it read into registers one step earlier (transposing LDS load)
//     and refills those registers with the operand of tile i - 1, so no LDS
//     latency sits in front of its matrix instructions.  Value waves also issue
//     the tile copies (global_load_lds, 9 per wave per tile, two tiles ahead),
//     spread between their matrix instructions.
// One barrier per step.  Tiles resident: the one being scored, the one whose
// value operand is being read, and two in flight.
#include "attn_tile.hpp"
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace mla {
namespace {

constexpr int kPRows = 64;
constexpr int kPBuf = 4;
constexpr int kPDma = kTileBytes / 16 / 64 / 4;   // 9 copies per value wave per tile
constexpr int kPSteps = kD / 32;                  // 18 k-steps of the 16x16x32 score product
constexpr int kPRing = 6;                         // k-steps of tile reads in flight

template <int N>
using ic = std::integral_constant<int, N>;

__global__ __launch_bounds__(512, 1) void splitkv_bf16_x8p_kernel(
    const bf16* __restrict__ abuf, const bf16* __restrict__ cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, int H, int page_size, int chunk, int S_max, int RQ, int Tq,
    float* __restrict__ opart, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) bf16 tiles[kPBuf][kTileTok * kD];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][4][64];   // [tile parity][2 rb + ks][lane]
  __shared__ float alpha_s[2][kPRows];   // rescale factor of O per row, per tile parity
  __shared__ float lrow_s[kPRows];       // row sums at the end
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
  const int row_base = rq * kPRows;
  const int tok_begin = s * chunk;
  if (row_base >= R || tok_begin >= L) return;
  const int tok_end = min(tok_begin + chunk, L);
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
    // the row (rows past R read row 0 of the block: finite, never stored)
    bf16x8 qf[kPSteps];
    {
      const bf16* src = abuf + ((int64_t)(q0 + qi) * H + h) * kD + 8 * G;
#pragma unroll
      for (int st = 0; st < kPSteps; ++st) {
        qf[st] = load_bf16x8(src + 32 * st);
        asm volatile("" : "+a"(qf[st]));
      }
    }
    // A operand of (token half m, k-step st): token 16 m + c16, chunk 4 st + G
    uint32_t a_base[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int t = 16 * m + c16;
        a_base[m][p] = (uint32_t)(t * kChunks + ((4 * p + G) ^ swz(t))) * 16u;
      }
    // this lane's probabilities: value-product B fragment 2 (wave >> 1) + m,
    // lane 16 (wave & 1) + c16 + 32 (G >> 1), bytes 8 (G & 1) ..
    const int lp = 16 * (wave & 1) + c16 + 32 * (G >> 1);
    const int fb = 2 * (wave >> 1);
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[2][2];   // [tile parity][token half]: scores, token 16 m + 4 G + i

    // One loop step: scores of tile `it` into acc[P] (QK) interleaved with
    // the softmax of tile it - 1 from acc[1 - P] (SM).
    auto step = [&](auto PC, auto QKC, auto SMC, int it) {
      constexpr int P = decltype(PC)::value;
      constexpr bool QK = decltype(QKC)::value != 0, SM = decltype(SMC)::value != 0;
      const char* tileb = reinterpret_cast<const char*>(&tiles[it % kPBuf][0]);
      f32x4 (&cur)[2] = acc[P];
      f32x4 (&prev)[2] = acc[1 - P];
      float tmax = 0.f, m_new = 0.f, alpha = 1.f, rs = 0.f;
      float p[2][4];
      auto sm_stage = [&](int k) {
        if (k == 0) {
          // mask tokens past the row's last visible position (branch-free)
          const int d = lim - (tok_begin + (it - 1) * kTileTok) - 4 * G;
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * m + i > d) prev[m][i] = -INFINITY;
          tmax = max_raw(max_raw(max_raw(prev[0][0], prev[0][1]), max_raw(prev[0][2], prev[0][3])),
                         max_raw(max_raw(prev[1][0], prev[1][1]), max_raw(prev[1][2], prev[1][3])));
          tmax = quad_max(tmax);
        } else if (k == 1) {
          m_new = (tmax > m_run + kRescaleThreshold) ? tmax : m_run;
          alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[m][i] = __builtin_amdgcn_exp2f(prev[m][i] - m_ref);
        } else if (k == 2) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            bf16x4 pv = {from_f32<bf16>(p[m][0]), from_f32<bf16>(p[m][1]), from_f32<bf16>(p[m][2]),
                         from_f32<bf16>(p[m][3])};
            *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(&pbuf[1 - P][fb + m][lp]) + 8 * (G & 1)) = pv;
          }
          rs = ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
        } else {
          rs = quad_sum(rs);
          l_run = l_run * alpha + rs;
          m_run = m_new;
          alpha_s[1 - P][16 * wave + c16] = alpha;   // the four lanes of a row agree
        }
      };
      bf16x8 ring[kPRing][2];
      if constexpr (QK) {
#pragma unroll
        for (int st = 0; st < kPRing; ++st)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            ring[st][m] = *reinterpret_cast<const bf16x8*>(tileb + a_base[m][st & 1] + 128 * (st >> 1));
      }
#pragma unroll
      for (int st = 0; st < kPSteps; ++st) {
        if constexpr (QK) {
          bf16x8 (&a)[2] = ring[st % kPRing];
          if (st == 0) qk16x2_first(cur[0], cur[1], a[0], a[1], qf[0]);
          else qk16x2(cur[0], cur[1], a[0], a[1], qf[st]);
          if (st + kPRing < kPSteps) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
              a[m] = *reinterpret_cast<const bf16x8*>(tileb + a_base[m][(st + kPRing) & 1] +
                                                      128 * ((st + kPRing) >> 1));
          }
        }
        if constexpr (SM) {
          if (st == 0) sm_stage(0);
          if (st == 3) sm_stage(1);
          if (st == 6) sm_stage(2);
          if (st == 9) sm_stage(3);
        }
      }
      if constexpr (QK) qk16_drain(cur[0], cur[1]);
    };
    auto body = [&](auto PC, int it) {
      __syncthreads();   // tile `it` landed; probabilities of tile it - 2 consumed
      const bool qk = it < ntiles, sm = it >= 1 && it <= ntiles;
      if (qk && sm) step(PC, ic<1>(), ic<1>(), it);
      else if (qk) step(PC, ic<1>(), ic<0>(), it);
      else if (sm) step(PC, ic<0>(), ic<1>(), it);
    };
    for (int it = 0; it < ntiles + 2; it += 2) {
      body(ic<0>(), it);
      if (it + 1 < ntiles + 2) body(ic<1>(), it + 1);
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
    auto tile_base = [&](int t) {
      const int tok0 = tok_begin + t * kTileTok;
      const int page = __builtin_amdgcn_readfirstlane(pages_s[tok0 / page_size - page0]);
      return cache + ((int64_t)page * page_size + (tok0 % page_size)) * kD;
    };
    // copy u (0..8) of this wave for a tile: LDS position slot * 16 holds
    // chunk (slot % 72) ^ swz(t) of token t = slot / 72
    uint32_t dma_off[kPDma];
#pragma unroll
    for (int u = 0; u < kPDma; ++u) {
      const int slot = (v * kPDma + u) * 64 + lane;
      const int tt = slot / kChunks;
      dma_off[u] = (uint32_t)(tt * kChunks + ((slot - tt * kChunks) ^ swz(tt))) * 16u;
    }
    auto copy = [&](const bf16* base, int t, int u) {
      dma16(base, dma_off[u], lds_tiles + (uint32_t)((t % kPBuf) * kTileBytes + (v * kPDma + u) * 1024));
    };
    auto issue_tile = [&](int t) {
      const bf16* base = tile_base(t);
#pragma unroll
      for (int u = 0; u < kPDma; ++u) copy(base, t, u);
    };
    // copies still allowed in flight when tile t must have landed: the next
    // tile's
    auto wait_tile = [&](int t) {
      if (t + 1 < ntiles) wait_vmcnt<kPDma>(); else wait_vmcnt<0>();
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
    // first token of this lane's value-operand elements: 8 (G >> 1) + 16 ks + 4 r
    const int vt0 = 8 * (lane >> 5);
    f32x16 O[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        O[db][rb] = zero_f32x16();
        asm volatile("" : "+a"(O[db][rb]));   // accumulators live in AGPRs from the start
      }
    v4bf16 vf[4][2][2];   // value operand of one tile: [db][ks][r]

    // One loop step: accumulate tile it - 2 (PV) from the value operand read
    // one step earlier, and read the value operand of tile it - 1 (RD) into
    // the same registers, each 32-column block right after its last use.
    auto step = [&](bool PV, bool RD, int it, const bf16x8 (&pb)[2][2], const float (&al)[2],
                    const bf16* cbase, bool CP) {
      if (PV) {
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
      }
      const char* tb = reinterpret_cast<const char*>(&tiles[(it + kPBuf - 1) % kPBuf][0]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        if (PV) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 a = __builtin_shufflevector(vf[db][ks][0], vf[db][ks][1], 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 pr[2] = {pb[0][ks], pb[1][ks]};
            pv_mfma<2>(O[db], a, pr);
          }
        }
        if (CP) {
          // copies of tile it + 2 between the blocks: a copy that waits for a
          // free slot in the memory queue stalls this wave while the matrix
          // core still works on the instructions just issued
#pragma unroll
          for (int u = (db == 0 ? 0 : 1 + 2 * db); u < 3 + 2 * db; ++u) copy(cbase, it + 2, u);
        }
        if (RD) {
          // the refill must not move above the matrix instructions that read
          // these registers (that would need a second register set)
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int r = 0; r < 2; ++r)
              vf[db][ks][r] = ds_read_tr16(tb + pv_base[ks][r][db & 1] + 128 * (db >> 1));
        }
      }
      if (RD) {
        // tokens past the sequence's end hold whatever the page held: zero
        // their value elements so that zero probabilities never meet a NaN
        const int nvalid = tok_end - (tok_begin + (it - 1) * kTileTok);
        if (nvalid < kTileTok) {
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  if (vt0 + 16 * ks + 4 * r + j >= nvalid) vf[db][ks][r][j] = (__bf16)0.f;
        }
      }
    };
    auto body = [&](int it) {
      if (it < ntiles) wait_tile(it);
      // the value-operand reads of the previous step target a buffer that the
      // copies issued after this barrier may overwrite: they must be done
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
      __syncthreads();   // tile `it` landed; probabilities of tile it - 2 published
      const bool pv = it >= 2, rd = it >= 1 && it <= ntiles;
      // probabilities and rescale factors of tile it - 2 first: their LDS
      // latency runs under the copy issue
      bf16x8 pb[2][2];
      float al[2];
      if (pv) {
        const int P = it & 1;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) pb[rb][ks] = pbuf[P][2 * rb + ks][lane];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) al[rb] = alpha_s[P][32 * rb + l32];
      }
      const bool cp = it + 2 < ntiles;
      const bf16* cbase = cp ? tile_base(it + 2) : cache;
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): pb and al landed
      step(pv, rd, it, pb, al, cbase, cp);
    };

    issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    for (int it = 0; it < ntiles + 2; it += 2) {
      body(it);
      if (it + 1 < ntiles + 2) body(it + 1);
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
      float* dst = opart + ((int64_t)s * rows_total + rowg) * kDC + 128 * v;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = O[db][rb][4 * q4 + e] * inv;
          *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * q4 + 4 * g) = o;
        }
    }
  }
}

}  // namespace

void launch_splitkv_x8p(const SplitPlan& plan, const void* abuf, const void* cache,
                        const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                        int max_pages, int batch, int Tq, int H, int page_size, float* opart,
                        float* lse, hipStream_t st) {
  const int nblocks = batch * plan.S_max * plan.RQ;
  splitkv_bf16_x8p_kernel<<<nblocks, 512, 0, st>>>(
      (const bf16*)abuf, (const bf16*)cache, cu_q, seq_lens, page_table, max_pages, batch, H,
      page_size, plan.chunk, plan.S_max, plan.RQ, Tq, opart, lse);
}

}  // namespace mla

// LDS tile machinery shared by the split-KV attention kernels (gfx950):
// cached rows of d_c + d_rope = 576 bf16 stream HBM -> LDS in 32-token tiles
// through the LDS-DMA path, 16-byte chunks XOR-swizzled per token; matrix-core
// helpers with explicit accumulator register classes; the per-tile online
// softmax of the 32x32 score layout.
#pragma once

#include "common.hpp"

namespace mla {
namespace {

constexpr int kDC = 512, kDR = 64, kD = kDC + kDR;
constexpr int kChunks = kD / 8;              // 16-byte chunks per cached row (72)
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kD * 2;
constexpr int kDmaPerWave = kTileBytes / 16 / 64 / 4;   // 9 wave-wide DMAs per wave per tile
constexpr float kRescaleThreshold = 8.0f;    // log2 units: P may grow to 2^8 before rescale
constexpr int kMaxChunkTokens = 8192;         // largest split the attention kernel accepts
constexpr int kMaxChunkPages = kMaxChunkTokens / 64;

// Chunk swizzle: 16-byte chunk c of token t is stored at position
// c ^ swz(t) of the token's LDS row (the XOR stays inside c's aligned group of
// 8, so the 72 chunks of a row stay in the row).  LDS on gfx950 has 64 banks;
// swz mixes token bits 1..3 with bit 4 so that the score-operand reads (one
// chunk of 32 consecutive tokens per half wave) spread over all banks; the
// transposing value-operand reads stay conflict-light too (measured).
__device__ __forceinline__ int swz(int t) { return ((t >> 1) ^ (t >> 4)) & 7; }

typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));

// The (sequence b, split s, row group rq) a split-KV workgroup takes.  Without
// a work list: the block's logical id in the full grid of batch x S_max x RQ
// blocks (row group fastest), some of which find no rows or no tokens and
// exit; consecutive logical ids run on one XCD, so the row groups of a split
// share its L2.  With one (built by the work-list kernel: only busy items,
// item.y = s << 12 | rq, each XCD's items contiguous with a split's row
// groups together): blocks are handed to the 8 XCDs in turn, so block id % 8
// names the XCD and id / 8 the item among its list_hdr[1 + x] items, which
// start at list_hdr[9 + x]; blocks past that count exit at once.
__device__ __forceinline__ bool split_work_item(const int2* __restrict__ items, const int* __restrict__ list_hdr,
                                                int batch, int S_max, int RQ, int* b, int* s, int* rq) {
  if (items) {
    const int x = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int n = __builtin_amdgcn_readfirstlane(list_hdr[1 + x]);
    if (local >= n) return false;
    const int2 it = items[__builtin_amdgcn_readfirstlane(list_hdr[9 + x]) + local];
    *b = __builtin_amdgcn_readfirstlane(it.x);
    const int y = __builtin_amdgcn_readfirstlane(it.y);
    *s = y >> 12;
    *rq = y & 4095;
    return true;
  }
  const int logical = xcd_logical_block(blockIdx.x, batch * S_max * RQ);
  *rq = logical % RQ;
  *s = (logical / RQ) % S_max;
  *b = logical / (RQ * S_max);
  return true;
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i mod 4) of the 8-byte words addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ v4bf16 ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) v4bf16*)(const __attribute__((address_space(3))) char*)p);
}

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

// ---- FP8 cache tiles (MLA_CACHE_FP8 pages: rows of 512 E4M3 codes and 64
// bf16 of rope key, the page's fp32 row scales after its rows).  A tile's 32
// rows and 32 scales are copied to a staging buffer, then converted once into
// the bf16 tile layout above; with power-of-two scales the dequantized values
// code * 2^e are exact in bf16, so the attention arithmetic that follows is
// the bf16 path's.
constexpr int kF8Row = 640;
constexpr int kF8RowsBytes = kTileTok * kF8Row;       // 20480
constexpr int kF8StageBytes = kF8RowsBytes + 1024;     // + one wave-wide copy holding the scales
constexpr int kF8Dma = kF8RowsBytes / 1024 + 1;        // 21 wave-wide copies per tile

typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

// All copies of one FP8 tile, issued by one wave: `page` is the page's first
// byte, `tok_in_page` the tile's first row in it (tiles never cross pages).
__device__ __forceinline__ void f8_issue(const uint8_t* page, int page_size, int tok_in_page,
                                         uint32_t lds_stage, int lane) {
  const uint8_t* rows = page + (size_t)tok_in_page * kF8Row;
#pragma unroll
  for (int u = 0; u < kF8RowsBytes / 1024; ++u)
    dma16(rows, (uint32_t)((u * 64 + lane) * 16), lds_stage + u * 1024);
  // 128 bytes of scales; lanes past the eighth repeat them (never read)
  const uint8_t* sc = page + (size_t)page_size * kF8Row + (size_t)tok_in_page * 4;
  dma16(sc, (uint32_t)((lane & 7) * 16), lds_stage + kF8RowsBytes);
}

// Items item0, item0 + istep, ... of one staged tile into the bf16 tile:
// latent items below latent_end of 0..1023 (row i / 32, codes 16 (i % 32) ..
// + 15 -> bf16 chunks 2 (i % 32) and + 1) and rope items from rope_begin of
// 0..255 (row i / 8, chunk 64 + i % 8).
// Rows at or past nvalid are written as zeros, so that zero probabilities
// never meet whatever the page held there.  U items per lane go at a time:
// all their staging reads first, so that the LDS latency is paid once per
// batch rather than once per item.
template <int U>
__device__ __forceinline__ void f8_convert(const char* stage, char* tile, int nvalid, int item0,
                                           int istep, int latent_end = kTileTok * 32,
                                           int rope_begin = 0) {
  const float* scales = reinterpret_cast<const float*>(stage + kF8RowsBytes);
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll 1
  for (int base = item0; base < latent_end; base += U * istep) {
    u32x4 w[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * istep, t = i >> 5;
      w[u] = zero;
      sc[u] = 0.f;
      if (i < latent_end && t < nvalid) {
        w[u] = *reinterpret_cast<const u32x4*>(stage + t * kF8Row + (i & 31) * 16);
        sc[u] = scales[t];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * istep, t = i >> 5, k = i & 31;
      if (i >= latent_end) break;
      u32x4 lo = zero, hi = zero;
      if (t < nvalid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v2bf16 x = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[u][q], sc[u], false);
          const v2bf16 y = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[u][q], sc[u], true);
          const uint32_t ux = __builtin_bit_cast(uint32_t, x), uy = __builtin_bit_cast(uint32_t, y);
          if (q < 2) {
            lo[2 * q] = ux;
            lo[2 * q + 1] = uy;
          } else {
            hi[2 * q - 4] = ux;
            hi[2 * q - 3] = uy;
          }
        }
      }
      const int sw = swz(t);
      *reinterpret_cast<u32x4*>(tile + (t * kChunks + ((2 * k) ^ sw)) * 16) = lo;
      *reinterpret_cast<u32x4*>(tile + (t * kChunks + ((2 * k + 1) ^ sw)) * 16) = hi;
    }
  }
#pragma unroll 1
  for (int base = rope_begin + item0; base < kTileTok * 8; base += U * istep) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * istep, t = i >> 3;
      w[u] = zero;
      if (i < kTileTok * 8 && t < nvalid)
        w[u] = *reinterpret_cast<const u32x4*>(stage + t * kF8Row + 512 + (i & 7) * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * istep, t = i >> 3;
      if (i >= kTileTok * 8) break;
      *reinterpret_cast<u32x4*>(tile + (t * kChunks + 64 + ((i & 7) ^ swz(t))) * 16) = w[u];
    }
  }
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

// Value MFMAs, accumulators pinned to AGPRs: one A operand (a transposed
// tile fragment) against the probability fragments of NB row blocks.  Starts
// with two wait states (the A operand was just assembled by vector ALU ops).
template <int NB>
__device__ __forceinline__ void pv_mfma(f32x16 (&o)[NB], const bf16x8& a, const bf16x8 (&p)[NB]) {
  if constexpr (NB == 1) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
        : "+a"(o[0])
        : "v"(a), "v"(p[0]));
  } else if constexpr (NB == 2) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1"
        : "+a"(o[0]), "+a"(o[1])
        : "v"(a), "v"(p[0]), "v"(p[1]));
  } else {
    static_assert(NB == 4, "row blocks");
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %4, %6, %1\n\t"
        "v_mfma_f32_32x32x16_bf16 %2, %4, %7, %2\n\t"
        "v_mfma_f32_32x32x16_bf16 %3, %4, %8, %3"
        : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3])
        : "v"(a), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]));
  }
}

// 32 wait states after the last value MFMA before the accumulators are read
// by ordinary instructions; taking them as operands orders the reads after.
template <int NB, int NDB>
__device__ __forceinline__ void pv_drain(f32x16 (&o)[NDB][NB]) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    if constexpr (NB == 1) {
      asm volatile("s_nop 7" : "+a"(o[db][0]));
    } else if constexpr (NB == 2) {
      asm volatile("s_nop 7" : "+a"(o[db][0]), "+a"(o[db][1]));
    } else {
      asm volatile("s_nop 7" : "+a"(o[db][0]), "+a"(o[db][1]), "+a"(o[db][2]), "+a"(o[db][3]));
    }
  }
}

// Both halves of a wave hold the same 32 rows (acc_row32: lane l and l ^ 32
// hold different tokens of row l % 32).  permlane32_swap hands each lane its
// partner's value without going through LDS; r[0] is the lower half's value
// and r[1] the upper half's in every lane, so both halves combine them in the
// same order and agree bit for bit.
__device__ __forceinline__ float2 lane_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Online softmax over one 32-token tile held in the score accumulator
// (row l % 32, token tok0 + acc_row32(r, l)).  Scores are scaled into log2
// units; tokens past the row's last visible position `limit` are masked
// (only needed when the tile reaches past the smallest limit of the block).
// The running max moves lazily: only when a score exceeds it by more than
// kRescaleThreshold, so rescaling O is rare and P stays below 2^threshold.
// Returns the rescale factor alpha for O; writes the bf16 probabilities as the
// two k-step fragments of the value MFMA.
__device__ __forceinline__ float softmax_tile(f32x16& acc, bool masked, int tok0, int limit,
                                              float scale_log2e, float& m_run, float& l_run,
                                              bf16x8& pf0, bf16x8& pf1) {
  const int lane = threadIdx.x & 63;
  float tmax = -INFINITY;
  if (masked) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tok = tok0 + acc_row32(r, lane);
      acc[r] = (tok <= limit) ? acc[r] * scale_log2e : -INFINITY;
      tmax = fmaxf(tmax, acc[r]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[r] *= scale_log2e;
      tmax = fmaxf(tmax, acc[r]);
    }
  }
  {
    const float2 h = lane_halves(tmax);
    tmax = fmaxf(h.x, h.y);
  }
  const float m_new = (tmax > m_run + kRescaleThreshold) ? tmax : m_run;
  const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
  const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    // probabilities below 2^-126 of the running max flush to zero
    const float pv = __builtin_amdgcn_exp2f(acc[r] - m_ref);
    rs += pv;
    if (r < 8) pf0[r] = from_f32<bf16>(pv);
    else pf1[r - 8] = from_f32<bf16>(pv);
  }
  {
    const float2 h = lane_halves(rs);
    rs = h.x + h.y;
  }
  l_run = l_run * alpha + rs;
  m_run = m_new;
  return alpha;
}

// max of two scores (finite or -inf, never NaN here): the bare instruction,
// without the canonicalising moves fmaxf adds for values it cannot prove
// canonical
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// in the same order in every lane.
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two score MFMAs (both 16-token halves of the tile) against one query
// fragment held in AGPRs.  Starts with two wait states (an A operand may have
// been moved into place by a vector instruction).
__device__ __forceinline__ void qk16x2(f32x4& c0, f32x4& c1, const bf16x8& a0, const bf16x8& a1,
                                       const bf16x8& b) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, %1"
      : "+v"(c0), "+v"(c1)
      : "v"(a0), "v"(a1), "a"(b));
}
__device__ __forceinline__ void qk16x2_first(f32x4& c0, f32x4& c1, const bf16x8& a0,
                                             const bf16x8& a1, const bf16x8& b) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, 0"
      : "=&v"(c0), "=&v"(c1)
      : "v"(a0), "v"(a1), "a"(b));
}
// 16 wait states after the last score MFMA before vector instructions read
// the accumulators (more than the pass count plus margin the hardware needs);
// taking them as operands orders the reads after.
__device__ __forceinline__ void qk16_drain(f32x4& c0, f32x4& c1) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
}

}  // namespace
}  // namespace mla

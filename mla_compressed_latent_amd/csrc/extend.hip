// Prefill and chunked extend over the paged latent cache, expanded form.
//
// "Multi-head Latent Attention and KV Cache Compression" (jongkwan.dev),
// sections "The absorption trick and decoupled RoPE" and "What separates
// expressiveness at an equal cache budget": the absorbed query is wider, so
// absorption can raise prefill compute.  "Multi-head Latent Attention: the KV
// cache, compressed" (paperfordummies.in), section "Absorption: the part that
// makes it free": at real d_c / head-width ratios the absorbed form is not
// always fewer multiply-accumulates.
//
// With many query tokens per sequence it is cheaper to build each head's keys
// and values once per cached token (2 d_c (d_nope + d_v) flop per token and
// head) and to score at width d_nope + d_rope instead of d_c + d_rope.  Two
// kernels, both on the matrix cores, every operand streamed HBM -> LDS as
// whole 1 KB MFMA fragments by the LDS-DMA path:
//
//  expand_kv_kernel   one workgroup per (sequence, group of heads, 256
//                     tokens): K_h = C W_uk_h and V_h = C W_uv_h for each
//                     head of the group in turn, stored per 64-token tile as
//                     the attention kernel's operand fragments, so its
//                     copies are contiguous 1 KB reads.
//  extend_attn_kernel one workgroup per (sequence, head, 256 queries), one
//                     wave per 32 queries: causal flash attention.  Scores
//                     are formed transposed (S^T = K Q^T, tokens down the
//                     rows) so each lane owns one query column, the softmax
//                     runs in registers, and the probabilities are already
//                     the B operand of O^T = V^T P^T.  The value fragments
//                     hold their tokens in that register order.
//
// The rotated position key is read from the cache itself (one copy for all
// heads, "The code", decoupled_score); only the content key and the value
// are materialised.
#include "attn_tile.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

// LDS reads of one wave must have returned before a barrier that lets other
// waves overwrite the buffer they came from.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

__device__ __forceinline__ void wait_dma_ahead(int ahead, int per_stage) {
  // s_waitcnt takes an immediate: the counts used here are 0 .. 2 stages of
  // at most 5 copies each.
  switch (ahead * per_stage) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 10: wait_vmcnt<10>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ================================================================ expansion
constexpr int kExpTok = 256;                 // tokens per workgroup, 64 per wave pair
constexpr int kExpStep = 32;                 // latent columns per pipeline stage (two k-steps)
constexpr int kExpStages = kDC / kExpStep;   // 16
constexpr int kExpBuf = 4;                   // stage buffers: one being read, three in flight
constexpr int kExpWaves = 8;

template <int DN, int DV>
struct ExpandDims {
  static constexpr int kFragC = kExpTok * kExpStep * 2 / 1024;   // 1 KB slots of cache rows per stage
  static constexpr int kFragK = (DN / 32) * 2;        // W_uk_h^T fragments per stage
  static constexpr int kFragV = (DV / 32) * 2;        // W_uv_h fragments per stage
  static constexpr int kFrag = kFragC + kFragK + kFragV;
  // copies per wave and stage; slots past kFrag repeat fragment 0 (unused)
  static constexpr int kDma = (kFrag + kExpWaves - 1) / kExpWaves;
  static constexpr int kSlots = kDma * kExpWaves;
};

// Waves 0-3: keys of tokens t0 + 64 w .. + 63, accumulators K^T[i][t]
// (A = W_uk_h^T fragment, B = cache-row fragment).  Waves 4-7: values of the
// same token quarters, accumulators V[t][v] (A = cache rows, B = W_uv_h).
// Both operands are d_c-contiguous, so the two products use the same
// fragments with the roles of A and B swapped.  Two waves share each SIMD,
// so one wave's waits and stores overlap the other's matrix work.
// The nh heads of a workgroup run back to back through one copy pipeline of
// nh * 16 stages: the next head's first stages are in flight while the
// current one finishes, its stores overlap the next head's products, and
// the head's cache-row stages come from L2 (the previous head read them).
template <int DN, int DV>
__global__ __launch_bounds__(512, 1) void expand_kv_kernel(
    const bf16* __restrict__ cache, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int max_pages, int batch, int H, int nh, int page_size,
    int lmax, const bf16* __restrict__ wukt, const bf16* __restrict__ wuv,
    bf16* __restrict__ kexp, bf16* __restrict__ vexp) {
  using Dm = ExpandDims<DN, DV>;
  __shared__ __attribute__((aligned(1024))) bf16 sbuf[kExpBuf][Dm::kSlots * 512];

  const int ntt = lmax / kExpTok;
  const int HG = H / nh;
  const int nblocks = batch * HG * ntt;
  const int logical = xcd_logical_block(blockIdx.x, nblocks);
  const int tt = logical % ntt;
  const int h = ((logical / ntt) % HG) * nh;   // first head of the group
  const int b = logical / (ntt * HG);
  const int L = seq_lens[b];
  const int t0 = tt * kExpTok;
  if (t0 >= L) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const uint32_t lds0 = lds_address(&sbuf[0][0]);

  // Sources of this wave's fragment copies; stage st of head h + k adds
  // st * stride + k * head_step bytes.
  const char* src[Dm::kDma];
  uint32_t voff[Dm::kDma];
  uint32_t stride[Dm::kDma];
  uint32_t head_step[Dm::kDma];
#pragma unroll
  for (int u = 0; u < Dm::kDma; ++u) {
    int f = wave * Dm::kDma + u;
    if (f >= Dm::kFrag) f = 0;
    head_step[u] = 0;   // cache rows: the same for every head
    if (f < Dm::kFragC) {
      // slot f: tokens t0 + 16 f .. + 15 (one page: pages hold a multiple of
      // 64 tokens), the stage's 64 bytes of each row as four 16-byte chunks,
      // lane l at row l / 4, position l % 4 holding chunk (l % 4) ^ swizzle.
      // Rows past the sequence repeat its last row.
      const int tf = min(t0 + 16 * f, L - 1);
      const int page = __builtin_amdgcn_readfirstlane(
          page_table[(int64_t)b * max_pages + tf / page_size]);
      const int tl = min(t0 + 16 * f + (lane >> 2), L - 1);
      const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
      src[u] = reinterpret_cast<const char*>(cache + (int64_t)page * page_size * kD);
      voff[u] = (uint32_t)(((tl % page_size) * kD + 8 * chunk) * 2);
      stride[u] = kExpStep * 2;
    } else if (f < Dm::kFragC + Dm::kFragK) {
      const int g = f - Dm::kFragC, ib = g >> 1, s = g & 1;
      src[u] = reinterpret_cast<const char*>(wukt + (int64_t)h * DN * kDC +
                                             ((int64_t)ib * (kDC / 16) + s) * 512);
      voff[u] = (uint32_t)(lane * 16);
      stride[u] = 2 * 512 * 2;
      head_step[u] = DN * kDC * 2;
    } else {
      const int g = f - Dm::kFragC - Dm::kFragK, vb = g >> 1, s = g & 1;
      src[u] = reinterpret_cast<const char*>(wuv + (int64_t)h * DV * kDC +
                                             ((int64_t)vb * (kDC / 16) + s) * 512);
      voff[u] = (uint32_t)(lane * 16);
      stride[u] = 2 * 512 * 2;
      head_step[u] = DV * kDC * 2;
    }
  }
  // global stage g = 16 k + st: stage st of head h + k
  const int nstages = nh * kExpStages;
  auto issue = [&](int g) {
    const int k = g / kExpStages, st = g % kExpStages;
    const uint32_t dst = lds0 + (uint32_t)(((g % kExpBuf) * Dm::kSlots + wave * Dm::kDma) * 1024);
#pragma unroll
    for (int u = 0; u < Dm::kDma; ++u)
      dma16(src[u] + (int64_t)k * head_step[u] + st * stride[u], voff[u], dst + u * 1024);
  };
  // stage g is in LDS for every wave, and every wave has finished reading
  // stage g - 1 (whose buffer the copies issued next overwrite)
  auto stage_ready = [&](int g) -> const bf16x8* {
    wait_dma_ahead(min(kExpBuf - 2, nstages - 1 - g), Dm::kDma);
    wait_lds();
    __syncthreads();
    if (g + kExpBuf - 1 < nstages) issue(g + kExpBuf - 1);
    return reinterpret_cast<const bf16x8*>(&sbuf[g % kExpBuf][0]);
  };

#pragma unroll
  for (int g = 0; g < kExpBuf - 1; ++g)
    if (g < nstages) issue(g);
  const int th = wave & 3;
  // cache-row operand of row block j: row r = 64 th + 32 j + l32 of the tile,
  // chunk c at 16-byte position 4 r + (c ^ ((r >> 2) & 3)) -- sixteen
  // consecutive rows read one chunk each from sixteen different bank groups
  const int crow[2] = {(64 * th + l32) * 4, (64 * th + 32 + l32) * 4};
  const int cswz = (l32 >> 2) & 3;
  const int tile0 = (t0 >> 6) + th;   // this wave's 64-token tile

  if (wave < 4) {
   for (int k = 0; k < nh; ++k) {
    const int64_t bh = (int64_t)b * H + h + k;
    f32x16 acc[DN / 32][2];
#pragma unroll
    for (int i = 0; i < DN / 32; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = zero_f32x16();
    for (int st = 0; st < kExpStages; ++st) {
      const bf16x8* fr = stage_ready(k * kExpStages + st);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 c[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) c[j] = fr[crow[j] + ((2 * s + hh) ^ cswz)];
#pragma unroll
        for (int i = 0; i < DN / 32; ++i) {
          const bf16x8 a = fr[(Dm::kFragC + i * 2 + s) * 64 + lane];
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a, c[j], acc[i][j]);
        }
      }
    }
    // K^T accumulator: element r is key column d = 32 i + acc_row32(r) of
    // token 32 j + l32 of the wave's tile.  Stored as the attention kernel's
    // score-operand fragments: fragment (j, d / 16) of the tile, lane
    // l32 + 32 ((d / 8) & 1), element d % 8 -- four consecutive r are four
    // consecutive elements, and the wave's stores cover whole 512-byte runs.
#pragma unroll
    for (int i = 0; i < DN / 32; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16* tb = kexp + (((bh * (lmax / 64) + tile0) * 2 + j) * (DN / 16)) * 512;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[i][j];
          bf16x4 v = {from_f32<bf16>(a[4 * q]), from_f32<bf16>(a[4 * q + 1]),
                      from_f32<bf16>(a[4 * q + 2]), from_f32<bf16>(a[4 * q + 3])};
          *reinterpret_cast<bf16x4*>(tb + ((2 * i + (q >> 1)) * 64 + l32 + 32 * (q & 1)) * 8 + 4 * hh) = v;
        }
      }
   }
  } else {
   for (int k = 0; k < nh; ++k) {
    const int64_t bh = (int64_t)b * H + h + k;
    f32x16 acc[2][DV / 32];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < DV / 32; ++i) acc[j][i] = zero_f32x16();
    for (int st = 0; st < kExpStages; ++st) {
      const bf16x8* fr = stage_ready(k * kExpStages + st);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 c[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) c[j] = fr[crow[j] + ((2 * s + hh) ^ cswz)];
#pragma unroll
        for (int i = 0; i < DV / 32; ++i) {
          const bf16x8 w = fr[(Dm::kFragC + Dm::kFragK + i * 2 + s) * 64 + lane];
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[j][i] = mfma32(c[j], w, acc[j][i]);
        }
      }
    }
    // V accumulator: element r is token 32 j + acc_row32(r) of the wave's
    // tile, value column 32 i + l32.  Stored as the attention kernel's
    // value-operand fragments (A operand of O^T = V^T P^T): fragment (i, k)
    // of the tile, lane l, eight tokens whose order matches the probability
    // registers -- elements 0..7 of the accumulator are fragment k = 2 j,
    // elements 8..15 fragment 2 j + 1, each one 16-byte store per lane.
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < DV / 32; ++i) {
        const f32x16& a = acc[j][i];
        bf16* dst = vexp + ((((bh * (lmax / 64) + tile0) * (DV / 32) + i) * 4 + 2 * j) * 64 + lane) * 8;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = from_f32<bf16>(a[8 * g + e]);
          *reinterpret_cast<bf16x8*>(dst + g * 512) = v;
        }
      }
   }
  }
}

// ================================================================ attention
constexpr int kAttWaves = 8;
constexpr int kQBlk = 32 * kAttWaves;   // queries per workgroup, 32 per wave
constexpr int kKTok = 64;               // keys per tile
constexpr int kAttBuf = 3;              // tile buffers: one being read, two in flight

template <int DN, int DV>
struct AttnDims {
  static constexpr int kQS = (DN + kDR) / 16;      // k-steps of the score product
  static constexpr int kFragK = 2 * kQS;           // key fragments per tile (two 32-token halves)
  static constexpr int kVB = DV / 32;
  static constexpr int kFragV = kVB * 4;           // value fragments per tile (four 16-token k-steps)
  static constexpr int kFrag = kFragK + kFragV;
  static_assert(kFrag % kAttWaves == 0, "fragments must split evenly over the waves");
  static constexpr int kDma = kFrag / kAttWaves;
};

// Two waves share each SIMD: while one runs its softmax (vector ALU, as much
// work as the matrix products at these head widths) the other's products run.
template <int DN, int DV>
__global__ __launch_bounds__(512, 1) void extend_attn_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kexp, const bf16* __restrict__ vexp,
    const bf16* __restrict__ cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int max_pages,
    int batch, int H, int page_size, int lmax, int nqb, RopeFreq freq, float scale_log2e,
    bf16* __restrict__ out) {
  using Dm = AttnDims<DN, DV>;
  constexpr int DQ = DN + kDR;
  __shared__ __attribute__((aligned(1024))) bf16 tiles[kAttBuf][Dm::kFrag * 512];

  const int nblocks = batch * H * nqb;
  const int logical = xcd_logical_block(blockIdx.x, nblocks);
  const int qb = nqb - 1 - logical % nqb;   // longer (later) query blocks start first
  const int h = (logical / nqb) % H;
  const int b = logical / (nqb * H);
  const int q0 = cu_q[b];
  const int ql = cu_q[b + 1] - q0;
  if (qb * kQBlk >= ql) return;
  const int L = seq_lens[b];
  const int pos0 = L - ql;                  // position of the sequence's first query
  const int nkt = (pos0 + min(qb * kQBlk + kQBlk - 1, ql - 1)) / kKTok + 1;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int i0 = qb * kQBlk + 32 * wave;    // this wave's first query
  const bool wave_on = i0 < ql;
  const int wave_last = pos0 + min(i0 + 31, ql - 1);
  const bool q_valid = i0 + l32 < ql;
  const int qi = min(i0 + l32, ql - 1);     // past the end: repeat the last query
  const int pos = pos0 + qi;
  const int64_t bh = (int64_t)b * H + h;

  // ---- copies of this wave's fragments of a tile
  // kind 0: content key rows from kexp; 1: rotated key rows from the cache
  // page; 2: value fragments from vexp
  int kind[Dm::kDma];
  uint32_t voff[Dm::kDma];
#pragma unroll
  for (int u = 0; u < Dm::kDma; ++u) {
    const int f = wave * Dm::kDma + u;
    if (f < Dm::kFragK) {
      const int tb = f / Dm::kQS, s = f % Dm::kQS;
      if (16 * s < DN) {
        kind[u] = 0;
        voff[u] = (uint32_t)((((tb * (DN / 16) + s) * 64) + lane) * 16);
      } else {
        kind[u] = 1;
        voff[u] = (uint32_t)(((32 * tb + l32) * kD + kDC + 16 * s - DN + 8 * hh) * 2);
      }
    } else {
      const int g = f - Dm::kFragK, vb = g / 4, s2 = g % 4;
      kind[u] = 2;
      voff[u] = (uint32_t)((((vb * 4 + s2) * 64) + lane) * 16);
    }
  }
  const uint32_t lds0 = lds_address(&tiles[0][0]);
  const bf16* kbase = kexp + bh * lmax * DN;
  const bf16* vbase = vexp + bh * (lmax / kKTok) * DV * kKTok;
  auto issue = [&](int kt) {
    const int tok = kt * kKTok;
    const int page = __builtin_amdgcn_readfirstlane(page_table[(int64_t)b * max_pages + tok / page_size]);
    const bf16* rbase = cache + ((int64_t)page * page_size + tok % page_size) * kD;
    const bf16* kt_k = kbase + (int64_t)tok * DN;
    const bf16* kt_v = vbase + (int64_t)kt * DV * kKTok;
    const uint32_t dst = lds0 + (uint32_t)(((kt % kAttBuf) * Dm::kFrag + wave * Dm::kDma) * 1024);
#pragma unroll
    for (int u = 0; u < Dm::kDma; ++u) {
      const bf16* g = kind[u] == 0 ? kt_k : (kind[u] == 1 ? rbase : kt_v);
      dma16(g, voff[u], dst + u * 1024);
    }
  };

  // ---- queries: B operand of k-step s holds dims 16 s + 8 hh .. + 7; the
  // position part is rotated at the query's own position, and the whole
  // query is multiplied by scale * log2(e) before rounding, so the scores
  // come out in log2 units
  bf16x8 qf[Dm::kQS];
  {
    const bf16* src = q + ((int64_t)(q0 + qi) * H + h) * DQ + 8 * hh;
#pragma unroll
    for (int s = 0; s < Dm::kQS; ++s) {
      bf16x8 v = load_bf16x8(src + 16 * s);
      if (16 * s >= DN) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int pair = (16 * s - DN + 8 * hh) / 2 + m;
          float c, sn;
          rope_cos_sin_reduced(pos, freq.theta[pair], &c, &sn);
          const float x0 = to_f32(v[2 * m]), x1 = to_f32(v[2 * m + 1]);
          v[2 * m] = from_f32<bf16>((x0 * c - x1 * sn) * scale_log2e);
          v[2 * m + 1] = from_f32<bf16>((x0 * sn + x1 * c) * scale_log2e);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = from_f32<bf16>(to_f32(v[e]) * scale_log2e);
      }
      qf[s] = v;
    }
  }

  f32x16 O[Dm::kVB];
#pragma unroll
  for (int vb = 0; vb < Dm::kVB; ++vb) O[vb] = zero_f32x16();
  float m_run = -INFINITY, l_run = 0.f;

  issue(0);
  if (nkt > 1) issue(1);
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) wait_dma_ahead(1, Dm::kDma);
    else wait_vmcnt<0>();
    wait_lds();
    __syncthreads();   // tile kt landed for every wave; tile kt-1 fully read
    if (kt + 2 < nkt) issue(kt + 2);
    if (!wave_on || kt * kKTok > wave_last) continue;   // every key past this wave's queries

    const bf16x8* fr = reinterpret_cast<const bf16x8*>(&tiles[kt % kAttBuf][0]);
    // S^T[t][q] for the tile's two 32-token halves
    f32x16 S[2] = {zero_f32x16(), zero_f32x16()};
#pragma unroll
    for (int s = 0; s < Dm::kQS; ++s) {
      const bf16x8 a0 = fr[s * 64 + lane];
      const bf16x8 a1 = fr[(Dm::kQS + s) * 64 + lane];
      S[0] = mfma32(a0, qf[s], S[0]);
      S[1] = mfma32(a1, qf[s], S[1]);
    }
    // online softmax of this lane's query over the 64 keys (log2 units); the
    // running max moves only when a score passes it by kRescaleThreshold
    const int tok0 = kt * kKTok;
    const bool masked = tok0 + kKTok - 1 > pos0 + i0;
    if (masked) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tok0 + 32 * tb + acc_row32(r, lane) > pos) S[tb][r] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) tmax = max_raw(tmax, max_raw(S[tb][r], S[tb][r + 1]));
    {
      const float2 hv = lane_halves(tmax);
      tmax = fmaxf(hv.x, hv.y);
    }
    const float m_new = (tmax > m_run + kRescaleThreshold) ? tmax : m_run;
    const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    bf16x8 pf[4];
    float rs = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(S[tb][r] - m_ref);
        rs += p;
        pf[2 * tb + (r >> 3)][r & 7] = from_f32<bf16>(p);
      }
    {
      const float2 hv = lane_halves(rs);
      rs = hv.x + hv.y;
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int vb = 0; vb < Dm::kVB; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[vb][r] *= alpha;
    }
    // O^T[v][q] += V^T[v][t] P^T[t][q], four 16-token k-steps
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
      for (int vb = 0; vb < Dm::kVB; ++vb)
        O[vb] = mfma32(fr[(Dm::kFragK + vb * 4 + s2) * 64 + lane], pf[s2], O[vb]);
  }

  if (!q_valid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  bf16* dst = out + ((int64_t)(q0 + qi) * H + h) * DV + 4 * hh;
#pragma unroll
  for (int vb = 0; vb < Dm::kVB; ++vb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 v = {from_f32<bf16>(O[vb][4 * j] * inv), from_f32<bf16>(O[vb][4 * j + 1] * inv),
                  from_f32<bf16>(O[vb][4 * j + 2] * inv), from_f32<bf16>(O[vb][4 * j + 3] * inv)};
      *reinterpret_cast<bf16x4*>(dst + 32 * vb + 8 * j) = v;
    }
}

template <int DN, int DV>
void expand_for(const void* cache, const int32_t* seq_lens, const int32_t* page_table, int max_pages,
                int batch, int H, int page_size, int lmax, const void* wukt, const void* wuv,
                void* kexp, void* vexp, hipStream_t st) {
  // heads per workgroup: four when they divide H, else two, else one
  const int nh = H % 4 == 0 ? 4 : (H % 2 == 0 ? 2 : 1);
  const int nblocks = batch * (H / nh) * (lmax / kExpTok);
  expand_kv_kernel<DN, DV><<<nblocks, 64 * kExpWaves, 0, st>>>(
      (const bf16*)cache, seq_lens, page_table, max_pages, batch, H, nh, page_size, lmax,
      (const bf16*)wukt, (const bf16*)wuv, (bf16*)kexp, (bf16*)vexp);
}

template <int DN, int DV>
void attn_for(const void* q, const void* kexp, const void* vexp, const void* cache,
              const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
              int max_pages, int batch, int max_q_len, int H, int page_size, int lmax,
              const RopeFreq& freq, float scale_log2e, void* out, hipStream_t st) {
  const int nqb = (max_q_len + kQBlk - 1) / kQBlk;
  const int nblocks = batch * H * nqb;
  extend_attn_kernel<DN, DV><<<nblocks, 64 * kAttWaves, 0, st>>>(
      (const bf16*)q, (const bf16*)kexp, (const bf16*)vexp, (const bf16*)cache, cu_q, seq_lens,
      page_table, max_pages, batch, H, page_size, lmax, nqb, freq, scale_log2e, (bf16*)out);
}

}  // namespace

bool extend_expanded_supported(int dn, int dv) {
  return (dn == 64 || dn == 128) && (dv == 64 || dv == 128);
}

void launch_expand_kv(const void* cache, const int32_t* seq_lens, const int32_t* page_table,
                      int max_pages, int batch, int H, int dn, int dv, int page_size, int lmax,
                      const void* wukt, const void* wuv, void* kexp, void* vexp, hipStream_t st) {
#define MLA_EXPAND(DN_, DV_)                                                                   \
  if (dn == DN_ && dv == DV_)                                                                  \
    return expand_for<DN_, DV_>(cache, seq_lens, page_table, max_pages, batch, H, page_size,   \
                                lmax, wukt, wuv, kexp, vexp, st);
  MLA_EXPAND(128, 128)
  MLA_EXPAND(64, 64)
  MLA_EXPAND(128, 64)
  MLA_EXPAND(64, 128)
#undef MLA_EXPAND
}

void launch_extend_attn(const void* q, const void* kexp, const void* vexp, const void* cache,
                        const int32_t* cu_q, const int32_t* seq_lens, const int32_t* page_table,
                        int max_pages, int batch, int max_q_len, int H, int dn, int dv,
                        int page_size, int lmax, const RopeFreq& freq, float scale, void* out,
                        hipStream_t st) {
  const float sl2e = scale * 1.4426950408889634f;
#define MLA_ATTN(DN_, DV_)                                                                      \
  if (dn == DN_ && dv == DV_)                                                                   \
    return attn_for<DN_, DV_>(q, kexp, vexp, cache, cu_q, seq_lens, page_table, max_pages,     \
                              batch, max_q_len, H, page_size, lmax, freq, sl2e, out, st);
  MLA_ATTN(128, 128)
  MLA_ATTN(64, 64)
  MLA_ATTN(128, 64)
  MLA_ATTN(64, 128)
#undef MLA_ATTN
}

}  // namespace mla

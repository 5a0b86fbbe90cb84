/*
 * mla.h -- C ABI of the MLA (Multi-head Latent Attention) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * One decode layer in its weight-absorbed form.  Each token's cache entry is
 * one row [c | k_rope]: the d_c-wide latent c = x W_dkv[:, :d_c] and the
 * d_rope-wide position key, rotated at the token's position before caching
 * and shared by every head.  Keys and values are never materialised: the
 * query of head h is folded into latent space (q_lat = W_uk_h q_nope), scored
 * against the cached rows (q_lat . c + rot(q_rope) . k_rope), the softmax
 * weights sum the latents into o_lat, and o_lat is projected out through
 * W_uv_h.
 *
 * Sources (web pages, cited by title and section):
 *   "Multi-head Latent Attention: the KV cache, compressed" (paperfordummies.in)
 *     - "The one formula": what one cached row holds (d_c + d_rope elements).
 *     - "Absorption: the part that makes it free": fold W_uk into the query
 *       side once at load; keys are never built.
 *     - "RoPE, and why the explanations stop here" and "The code"
 *       (decoupled_score): the score is the absorbed content part plus a
 *       rotated position part whose key is cached already rotated.
 *   "Multi-head Latent Attention and KV Cache Compression" (jongkwan.dev),
 *     "The absorption trick and decoupled RoPE": the value-side
 *     up-projection folds onto the output side in the same way.
 *   "Multi-Head Latent Attention (MLA)" (superteams.ai glossary), Hugging Face
 *     config snippet: the field names of mla_config.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named "device" point to GPU memory the CALLER allocated and
 *    owns (e.g. PyTorch tensors).  The library never allocates, frees or
 *    retains device memory; it owns only the small host handle mla_layer.
 *  - Every tensor is stored in cfg.dtype (fp32 or bf16, row-major, densely
 *    packed) unless stated otherwise; index tensors are int32.  Arithmetic
 *    accumulates in fp32; bf16 results are rounded to nearest even.
 *  - Calls enqueue work on `hip_stream` (a hipStream_t; NULL = the default
 *    stream) and return without synchronising.  Faults inside kernels
 *    surface at the caller's next synchronisation as HIP errors.
 *  - Host-checkable problems (null pointers, non-positive sizes, odd d_rope,
 *    unsupported shape/dtype, buffers too small) return a non-OK status
 *    before anything is enqueued.  Values that live in device memory
 *    (lengths, page ids) are trusted: the caller guarantees
 *    1 <= q_len_b <= seq_len_b <= max_seq_len, q_len_b <= max_q_len and
 *    that every page id a sequence touches lies in [0, num_pages).
 *  - The checking build (libmla_debug.so, the same sources compiled with
 *    MLA_DEBUG_CHECKS) verifies those device-resident values before every
 *    append, decode and extend: one single-workgroup kernel checks each
 *    sequence's offsets, lengths and page ids, the call waits for it, and a
 *    failure returns MLA_ERR_INVALID_ARG (mla_last_error() names the first
 *    bad sequence) with nothing else enqueued.  It synchronises the stream,
 *    so it does not check calls made while the stream is being captured.
 *  - Positions are 0-based token indices.  Sequence b's cached token t lives
 *    in row (t % page_size) of page page_table[b * max_pages + t / page_size].
 *  - mla_last_error() returns a thread-local message for the last non-OK
 *    status of the calling thread.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,            /* null pointer, bad size, inconsistent argument */
  MLA_ERR_UNSUPPORTED = 2,            /* valid but not implemented (shape/dtype)      */
  MLA_ERR_HIP = 3,                    /* a HIP runtime call failed                      */
  MLA_ERR_INSUFFICIENT_WORKSPACE = 4  /* workspace or folded buffer too small           */
} mla_status;

typedef enum { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

/* How cache pages store their rows.
 *   MLA_CACHE_DTYPE   rows [c | k_rope] in the layer dtype; a page is
 *                     [page_size][d_c + d_rope] elements.
 *   MLA_CACHE_FP8     (bf16 layers) the latent c of each row is quantized
 *                     to 8-bit floats, OCP E4M3 (1 sign, 4 exponent bits of
 *                     bias 7, 3 mantissa bits, no infinities, largest finite
 *                     448), with one power-of-two scale per row: c ~= 2^e *
 *                     code, e the smallest integer with max|c| <= 448 * 2^e
 *                     (0 for an all-zero latent), codes rounded to nearest
 *                     even.  The rotated rope key stays bf16.  A page is
 *                     page_size rows of 640 bytes (512 codes, then 64 bf16),
 *                     then page_size fp32 scales 2^e: page_size * 644 bytes.
 *                     ("Moving a trained MHA model over" on the "Multi-head
 *                     Latent Attention and KV Cache Compression" page: the
 *                     latent can be quantized further, with scales.) */
typedef enum { MLA_CACHE_DTYPE = 0, MLA_CACHE_FP8 = 1 } mla_cache_format;

/* Shape of one MLA layer.  Field names follow the Hugging Face DeepSeek-V2
 * config.  bf16 layers need kv_lora_rank == 512, qk_rope_head_dim == 64,
 * qk_nope_head_dim (at most 256) and v_head_dim multiples of 32 and d_model a
 * multiple of 256 (the matrix-core path); fp32 layers accept positive sizes with an
 * even qk_rope_head_dim and a kv_lora_rank that is a multiple of 4, at most
 * 1024. */
typedef struct {
  int32_t d_model;              /* hidden size of the tokens appended          */
  int32_t num_attention_heads;  /* H                                           */
  int32_t qk_nope_head_dim;     /* d_nope: content part of one head's query     */
  int32_t qk_rope_head_dim;     /* d_rope: rotated part (even); cached once     */
  int32_t v_head_dim;           /* d_v: output width per head                  */
  int32_t kv_lora_rank;         /* d_c: latent width                           */
  int32_t page_size;            /* tokens per cache page; multiple of 64       */
  float rope_base;              /* rotary base, e.g. 10000                     */
  float softmax_scale;          /* <= 0 selects 1/sqrt(d_nope + d_rope)         */
  mla_dtype dtype;              /* storage dtype of every tensor               */
  int32_t cache_format;         /* an mla_cache_format (0: rows in dtype)       */
} mla_config;

typedef struct mla_layer mla_layer; /* opaque host handle */

/* Bytes of the folded-weight buffer mla_fold_weights fills (0 if cfg is
 * invalid or unsupported): W_dkv, W_uk and W_uv in the kernels' operand
 * layouts, the fold that "Absorption: the part that makes it free" does once
 * at load. */
size_t mla_folded_bytes(const mla_config* cfg);

/* Fold the layer's weights once at load ("Absorption: the part that makes it
 * free": the fold happens once, not per step; rebuilding it in the decode
 * loop is the tax shown under "Now break it").
 *
 *   w_dkv [d_model][d_c + d_rope]   device; columns d_c.. produce k_rope
 *   w_uk  [d_c][H * d_nope]         device; head h = columns h*d_nope ..
 *   w_uv  [d_c][H * d_v]            device; head h = columns h*d_v ..
 *   folded                          device, >= mla_folded_bytes(cfg) bytes,
 *                                   must stay alive and unchanged while the
 *                                   layer is used; 256-byte aligned.
 * The three weights are read by work enqueued on hip_stream and may be freed
 * once that work has completed.  On success *out receives a new handle
 * (release with mla_layer_free).  Errors: INVALID_ARG (null, bad sizes),
 * UNSUPPORTED (shape/dtype), INSUFFICIENT_WORKSPACE (folded too small), HIP. */
mla_status mla_fold_weights(const mla_config* cfg, const void* w_dkv, const void* w_uk,
                            const void* w_uv, void* folded, size_t folded_bytes,
                            void* hip_stream, mla_layer** out);

/* Release the host handle made by mla_fold_weights (the folded buffer stays
 * the caller's).  Null is a no-op. */
void mla_layer_free(mla_layer* layer);

/* Rows of queries x heads one split-KV workgroup attends to in bf16 decode
 * of a layer with rows in the layer dtype: 0 (default) chooses by shape, 64
 * or 128 forces that kernel where it applies (128 needs more than 64 rows
 * per sequence).  Both kernels compute the same attention ("Absorption: the
 * part that makes it free": scores against the cached rows, weights times
 * the latent); the choice moves only rounding and speed.  The split plan of
 * every later decode call of this layer follows it.  Not thread-safe against
 * decode calls of the same layer.  Errors: INVALID_ARG (null layer, another
 * value). */
mla_status mla_layer_set_attention_rows(mla_layer* layer, int32_t rows);

/* Bytes one token occupies in the cache: (d_c + d_rope) * sizeof(dtype)
 * ("The one formula": one latent plus one position key per token and layer,
 * independent of the head count); 644 for MLA_CACHE_FP8 (512 codes, 128
 * bytes of rope key, a 4-byte scale).  A page holds page_size times this.
 * 0 if cfg is invalid. */
size_t mla_cache_bytes_per_token(const mla_config* cfg);

/* Workspace mla_append_latent needs for total_new new tokens. */
size_t mla_append_workspace_bytes(const mla_layer* layer, int32_t total_new);

/* Compute and cache the rows of new tokens ("The code": latent = x W_dkv is
 * the only thing cached; decoupled_score: the rope key is stored already
 * rotated, one copy for all heads).
 *
 *   x            [total_new][d_model]  device; tokens of sequence b are rows
 *                                      cu_new[b] .. cu_new[b+1]-1
 *   cu_new       [batch+1] int32       device; cu_new[0] = 0, nondecreasing,
 *                                      cu_new[batch] = total_new
 *   prefix_lens  [batch]   int32       device; tokens already cached; new token
 *                                      j of b goes to position prefix_lens[b]+j
 *   page_table   [batch][max_pages]    device int32
 *   cache        [num_pages][page_size][d_c + d_rope]  device, updated in place
 *   workspace    device, >= mla_append_workspace_bytes(layer, total_new)
 * Row of a new token: u = x W_dkv (fp32 accumulation), c = u[:d_c],
 * k_rope = rotate(u[d_c:], position); both rounded to dtype.  Only the rows
 * of the new tokens are written.  total_new == 0 is a no-op. */
mla_status mla_append_latent(const mla_layer* layer, const void* x, const int32_t* cu_new,
                             const int32_t* prefix_lens, const int32_t* page_table,
                             int32_t max_pages, int32_t batch, int32_t total_new, void* cache,
                             int64_t num_pages, void* workspace, size_t workspace_bytes,
                             void* hip_stream);

/* Tokens of cache each split-KV work item covers for these bounds
 * (kv_chunk > 0 is validated and returned; 0 picks a value from the batch
 * size, the longest sequence and the GPU's compute-unit count).  Returns -1
 * on invalid arguments. */
int32_t mla_decode_kv_chunk(const mla_layer* layer, int32_t batch, int32_t max_q_len,
                            int32_t max_seq_len, int32_t kv_chunk);

/* Workspace mla_decode needs for these bounds (same kv_chunk meaning): the
 * absorbed queries, each split's partial output and log-sum-exp, and the
 * merged latent output, i.e. the intermediate results of the re-associated
 * attention of "Absorption: the part that makes it free" (0 on invalid
 * arguments). */
size_t mla_decode_workspace_bytes(const mla_layer* layer, int32_t batch, int32_t total_q,
                                  int32_t max_q_len, int32_t max_seq_len, int32_t kv_chunk);

/* One absorbed decode step over a paged latent cache.
 *
 * Defined by "Multi-head Latent Attention: the KV cache, compressed":
 * "Absorption: the part that makes it free" (each head's query is folded
 * through W_uk and scored against the cached latents themselves; the softmax
 * weights sum the latents, and W_uv is applied to that sum, so no per-head key
 * or value is formed) and "RoPE, and why the explanations stop here" with
 * "The code" (decoupled_score: the score adds a position part, the rotated
 * query rope part against the cached, already rotated, shared rope key); and
 * by "Multi-head Latent Attention and KV Cache Compression", "The absorption
 * trick and decoupled RoPE" (one softmax scale over the sum of both parts).
 *
 *   q         [total_q][H][d_nope + d_rope]  device; queries BEFORE rotation;
 *             sequence b owns rows cu_q[b] .. cu_q[b+1]-1
 *   cu_q      [batch+1] int32 device (as cu_new)
 *   seq_lens  [batch] int32 device; cached tokens of b INCLUDING its queries'
 *             own rows (append first).  Query i of b sits at position
 *             seq_lens[b] - q_len_b + i and attends to every position <= it.
 *   page_table, cache   as for mla_append_latent (cache read only)
 *   out       [total_q][H][d_v] device: out = softmax(score) V per head,
 *             computed as (sum_t w_t c_t) W_uv_h; no output projection.
 *   kv_chunk  tokens per split-KV work item, a multiple of 64 up to 8192, or
 *             0 (auto); at most 1024 splits per sequence, and batch x splits
 *             x row groups (64 or 128 rows each) below 2^30 workgroups: a
 *             call past either limit fails with INVALID_ARG (and
 *             mla_decode_workspace_bytes returns 0).
 *             The split plan depends only on host arguments, so results are
 *             run-to-run deterministic.
 *   workspace device, >= mla_decode_workspace_bytes(...) bytes
 * Errors: INVALID_ARG, UNSUPPORTED, INSUFFICIENT_WORKSPACE, HIP. */
mla_status mla_decode(const mla_layer* layer, const void* q, const int32_t* cu_q,
                      const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                      int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                      int32_t kv_chunk, const void* cache, int64_t num_pages, void* out,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* Size of the device scratch mla_decode_no_alloc works in (64 MiB per GPU). */
#define MLA_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* mla_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  Same arguments and results as mla_decode; the
 * workspace is a static device array of MLA_NO_ALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends, looked up on
 * the first call on the current device (which must own q, cache, out and
 * hip_stream).  Nothing is allocated, and nothing in the scratch has to
 * start at zero.  All calls on one GPU share its array: calls that overlap
 * in time on one GPU (two streams, two threads) race and give wrong results;
 * serialize them (one stream).  Errors: as mla_decode, plus
 * INSUFFICIENT_WORKSPACE when mla_decode_workspace_bytes for these bounds
 * exceeds MLA_NO_ALLOC_SCRATCH_BYTES (fewer splits -- a larger kv_chunk -- or
 * a smaller batch fit), HIP if the scratch cannot be found on the device. */
mla_status mla_decode_no_alloc(const mla_layer* layer, const void* q, const int32_t* cu_q,
                               const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                               int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                               int32_t kv_chunk, const void* cache, int64_t num_pages, void* out,
                               void* hip_stream);

/* The three phases of mla_decode, for callers that interleave their own
 * work between them (timing, other streams):
 *   MLA_PHASE_ABSORB  fold each query into latent space and rotate its rope
 *                     part (writes the score operand into the workspace);
 *   MLA_PHASE_ATTEND  split-KV attention over the cache (writes per-split
 *                     partial outputs and log-sum-exps into the workspace);
 *   MLA_PHASE_OUTPUT  merge the splits and project through W_uv into out.
 * mla_decode_phases with the same arguments and workspace, called with the
 * phases in this order (any grouping), is exactly mla_decode; `phases` is a
 * nonzero OR of the flags.  The workspace carries the intermediate results
 * from one call to the next and must not be modified in between. */
typedef enum {
  MLA_PHASE_ABSORB = 1,
  MLA_PHASE_ATTEND = 2,
  MLA_PHASE_OUTPUT = 4,
  MLA_PHASE_ALL = 7
} mla_decode_phase;

mla_status mla_decode_phases(const mla_layer* layer, const void* q, const int32_t* cu_q,
                             const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                             int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                             int32_t kv_chunk, const void* cache, int64_t num_pages, void* out,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             uint32_t phases);

/* A whole decode step of one layer: mla_append_latent of the new tokens'
 * rows (x, cu_new, prefix_lens, total_new as there) followed by mla_decode
 * of the queries (q, cu_q, seq_lens, ... as there; seq_lens count the rows
 * just appended), with the same results bit for bit, in fewer launches: on
 * bf16 layers the query absorb shares a launch with the append's finish (bf16
 * pages: the GEMM runs first, then the finish beside the absorb) or with the
 * append GEMM (FP8 pages) -- work independent of each other ("Multi-head
 * Latent Attention: the KV cache, compressed": section "Store the archive,
 * not the files" for the latent x W_dkv that a step caches, section
 * "Absorption: the part that makes it free" for folding W_uk onto the query;
 * neither needs the other).
 *   workspace  device, 256-byte aligned, >= mla_decode_step_workspace_bytes
 *              (the decode workspace, then the append's)
 * Errors: those of mla_append_latent and mla_decode; nothing is enqueued
 * when a host check fails. */
size_t mla_decode_step_workspace_bytes(const mla_layer* layer, int32_t batch, int32_t total_new,
                                       int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                                       int32_t kv_chunk);
mla_status mla_decode_step(const mla_layer* layer, const void* x, const int32_t* cu_new,
                           const int32_t* prefix_lens, int32_t total_new, const void* q,
                           const int32_t* cu_q, const int32_t* seq_lens,
                           const int32_t* page_table, int32_t max_pages, int32_t batch,
                           int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                           int32_t kv_chunk, void* cache, int64_t num_pages, void* out,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* Prefill and chunked extend: many new query tokens per sequence over the
 * same paged cache ("Multi-head Latent Attention and KV Cache Compression",
 * sections "The absorption trick and decoupled RoPE" and "What separates
 * expressiveness at an equal cache budget": absorption can raise prefill
 * compute; "Multi-head Latent Attention: the KV cache, compressed", section
 * "Absorption: the part that makes it free": at real d_c / head-width ratios
 * the absorbed form is not always fewer multiply-accumulates).
 *
 * Two ways to compute the same result:
 *   MLA_EXTEND_ABSORBED  exactly mla_decode with kv_chunk 0;
 *   MLA_EXTEND_EXPANDED  each head's content keys c W_uk_h and values
 *                        c W_uv_h are built once per cached token into the
 *                        workspace, then causal flash attention runs at width
 *                        d_nope + d_rope (scores) and d_v (values).  bf16
 *                        layers with a bf16 cache (MLA_CACHE_DTYPE) and
 *                        qk_nope_head_dim and v_head_dim each 64 or 128;
 *   MLA_EXTEND_AUTO      the form with less matrix-core work for these
 *                        bounds (see mla_extend_choose_path). */
typedef enum {
  MLA_EXTEND_AUTO = 0,
  MLA_EXTEND_ABSORBED = 1,
  MLA_EXTEND_EXPANDED = 2
} mla_extend_path;

/* The form MLA_EXTEND_AUTO takes for these host bounds: MLA_EXTEND_EXPANDED
 * when it is available for cfg and its estimated matrix-core work,
 *   batch*max_seq_len*H*2*d_c*(d_nope+d_v) + total_q*H*2*(d_nope+d_rope+d_v)*K,
 * is below the absorbed form's,
 *   total_q*H*(2*d_c*(d_nope+d_v) + 2*(2*d_c+d_rope)*K),
 * with K = max_seq_len - max_q_len/2 keys per query; else
 * MLA_EXTEND_ABSORBED.  Host-only (no device call).  -1 on invalid
 * arguments (same bounds as mla_extend). */
int32_t mla_extend_choose_path(const mla_config* cfg, int32_t batch, int32_t total_q,
                               int32_t max_q_len, int32_t max_seq_len);

/* Workspace mla_extend needs for these bounds and path (AUTO resolved as
 * above).  Expanded: batch * H * lmax * (d_nope + d_v) * 2 bytes (plus
 * alignment), lmax = max_seq_len rounded up to a multiple of 256.  0 on
 * invalid arguments or when the path is unavailable for the layer. */
size_t mla_extend_workspace_bytes(const mla_layer* layer, int32_t batch, int32_t total_q,
                                  int32_t max_q_len, int32_t max_seq_len, int32_t path);

/* Attention of every query over its sequence's cache, with the arguments,
 * layout and result of mla_decode (queries before rotation, append first,
 * query i of b at position seq_lens[b] - q_len_b + i, causal).  `path` is an
 * mla_extend_path.  The workspace (>= mla_extend_workspace_bytes for the same
 * path, 256-byte aligned) is scratch for this call only.
 * Errors: INVALID_ARG, UNSUPPORTED (EXPANDED on a layer it does not cover),
 * INSUFFICIENT_WORKSPACE, HIP. */
mla_status mla_extend(const mla_layer* layer, const void* q, const int32_t* cu_q,
                      const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                      int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                      int32_t path, const void* cache, int64_t num_pages, void* out,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * A stack of layers: capacity planning and one page pool for every layer.
 * ("Multi-head Latent Attention: the KV cache, compressed", sections "The
 * one formula": a token costs num_layers * (d_c + d_rope) elements of cache
 * whatever the head count; "Where the saving actually lands": what matters
 * is how many whole sequences of a context fit one cache budget.)
 *
 * Every layer holds the same tokens of the same sequences, so one page table
 * serves all layers: each layer has its own cache tensor
 * [num_pages][page_size][d_c + d_rope] (for example slice l of one
 * [num_layers][num_pages][...] allocation), and page p of a sequence is page
 * p of every layer's tensor.  Host-only calls: nothing here touches the GPU.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t num_layers;
  int32_t page_size;
  int64_t num_pages;        /* pages of each layer's cache                   */
  size_t page_bytes;        /* one page of one layer: page_size * row bytes  */
  size_t layer_bytes;       /* num_pages * page_bytes                        */
  size_t total_bytes;       /* num_layers * layer_bytes, <= the budget       */
  size_t bytes_per_token;   /* num_layers * (d_c + d_rope) * dtype bytes     */
} mla_cache_plan;

/* The most whole pages (the same count in every layer, at most 2^31 - 1)
 * whose caches fit budget_bytes.  Errors: INVALID_ARG (bad cfg, num_layers
 * < 1, out null), INSUFFICIENT_WORKSPACE (not one page of every layer fits). */
mla_status mla_plan_cache(const mla_config* cfg, int32_t num_layers, size_t budget_bytes,
                          mla_cache_plan* out);

/* Whole sequences of `context` tokens that budget_bytes holds across
 * num_layers layers, each taking ceil(context / page_size) pages of every
 * layer: floor(budget / (num_layers * pages * page_bytes)).  -1 on invalid
 * arguments. */
int64_t mla_plan_max_sequences(const mla_config* cfg, int32_t num_layers, size_t budget_bytes,
                               int64_t context);

typedef struct mla_page_pool mla_page_pool; /* opaque host allocator */

/* An allocator of num_pages pages (page ids 0 .. num_pages-1, shared by all
 * layers) for sequence ids 0 .. max_seqs-1 of up to max_pages_per_seq pages
 * each.  A fresh pool hands pages out in ascending order; released pages are
 * handed out again first, the most recently released first, each sequence's
 * pages in their old order.  Not thread safe.  Errors: INVALID_ARG. */
mla_status mla_pool_create(int64_t num_pages, int32_t page_size, int32_t max_seqs,
                           int32_t max_pages_per_seq, mla_page_pool** out);
void mla_pool_destroy(mla_page_pool* pool);

/* Grow sequence `seq` to hold `length` tokens: pages are added at its end,
 * never removed or moved (rows already cached stay where they are).
 * INVALID_ARG for a bad id or a length beyond max_pages_per_seq * page_size;
 * INSUFFICIENT_WORKSPACE when the free pages do not cover the growth (the
 * pool is then unchanged). */
mla_status mla_pool_reserve(mla_page_pool* pool, int32_t seq, int64_t length);

/* Return every page of `seq` to the pool; its reserved length becomes 0. */
mla_status mla_pool_release(mla_page_pool* pool, int32_t seq);

/* Free pages, and the tokens reserved for `seq` (-1 on bad arguments). */
int64_t mla_pool_free_pages(const mla_page_pool* pool);
int64_t mla_pool_length(const mla_page_pool* pool, int32_t seq);

/* The page-table rows of n sequences, ready to copy to the device for
 * mla_append_latent / mla_decode / mla_extend of any layer: table is a HOST
 * buffer [n][max_pages_per_seq] int32, row i = the pages of seqs[i] in token
 * order, then -1.  Errors: INVALID_ARG. */
mla_status mla_pool_page_table(const mla_page_pool* pool, const int32_t* seqs, int32_t n,
                               int32_t* table);

/* ---------------------------------------------------------------------------
 * Layer output with the output projection W_o, the value up-projection kept
 * apart or folded into it ("Multi-head Latent Attention and KV Cache
 * Compression", section "The absorption trick and decoupled RoPE": W_uv can
 * be pre-multiplied into W_o just as W_uk is pre-multiplied into the query
 * side).
 *   MLA_OUTPUT_UNFOLDED  y = concat_h(o_lat_h W_uv_h) . W_o
 *                        (weights H*d_v*(d_c + d_model) elements)
 *   MLA_OUTPUT_FOLDED    y = concat_h(o_lat_h) . W_uvo, W_uvo_h = W_uv_h W_o_h
 *                        folded once at load (H*d_c*d_model elements)
 *   MLA_OUTPUT_AUTO      mla_output_choose_form(cfg, 1)
 * bf16 layers with num_attention_heads * v_head_dim a multiple of 256.
 * ------------------------------------------------------------------------- */
typedef enum {
  MLA_OUTPUT_AUTO = 0,
  MLA_OUTPUT_UNFOLDED = 1,
  MLA_OUTPUT_FOLDED = 2
} mla_output_form;

/* The form with the smaller estimated time for total_q query tokens, each
 * form's time the larger of its weight bytes / 8 TB/s and its matrix-core
 * flops / 2.5 PFLOP/s.  Folding wins only when d_model < d_c d_v / (d_c - d_v)
 * (for d_c > d_v): never for the shapes the kernels take.  Host only; -1 on
 * an invalid config or total_q < 1. */
int32_t mla_output_choose_form(const mla_config* cfg, int32_t total_q);

/* Bytes of the buffer mla_fold_output fills for a form (0 if unsupported). */
size_t mla_output_folded_bytes(const mla_config* cfg, int32_t form);

/* Attach the output projection to a layer.
 *   w_uv  [d_c][H * d_v]       device, the same W_uv given to mla_fold_weights
 *                              (read for MLA_OUTPUT_FOLDED only; may be null otherwise)
 *   w_o   [H * d_v][d_model]   device; head h = rows h*d_v ..
 *   folded                     device, >= mla_output_folded_bytes(cfg, form),
 *                              256-byte aligned, kept and read by later calls
 * The inputs are read by work enqueued on hip_stream.  Errors: INVALID_ARG,
 * UNSUPPORTED (fp32 layer, H * d_v not a multiple of 256),
 * INSUFFICIENT_WORKSPACE, HIP. */
mla_status mla_fold_output(mla_layer* layer, const void* w_uv, const void* w_o, int32_t form,
                           void* folded, size_t folded_bytes, void* hip_stream);

/* Workspace bytes of mla_decode_project for these host bounds, by the form
 * the layer was folded with (0 when no output projection is folded or the
 * sizes are invalid). */
size_t mla_decode_project_workspace_bytes(const mla_layer* layer, int32_t batch, int32_t total_q,
                                          int32_t max_q_len, int32_t max_seq_len);

/* mla_decode (kv_chunk 0) followed by the output projection: y [total_q][d_model]
 * (layer dtype) = concat_h out[t][h] . W_o, by the form the layer was folded
 * with.  Same arguments and contract as mla_decode otherwise; the workspace is
 * scratch for this call only.  Errors as mla_decode, and INVALID_ARG when no
 * output projection was folded. */
mla_status mla_decode_project(const mla_layer* layer, const void* q, const int32_t* cu_q,
                              const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                              int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                              const void* cache, int64_t num_pages, void* y, void* workspace,
                              size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Queries from the layer input, with the key up-projection kept apart or
 * folded into the query projection ("Multi-head Latent Attention: the KV
 * cache, compressed", section "Store the archive, not the files": the score
 * (x W_q)(c W_uk)^T equals x (W_q W_uk^T) c^T, so W_abs = W_q W_uk^T is formed
 * once at load and no key is ever built).
 *   MLA_QUERY_UNFOLDED  q = x . W_q, then mla_decode's own absorb
 *                       (weights H*(d_nope + d_rope)*d_model + H*d_nope*d_c elements)
 *   MLA_QUERY_FOLDED    per head [q_lat | q_rope] = x . [W_q_h^nope W_uk_h^T | W_q_h^rope],
 *                       folded once at load (H*(d_c + d_rope)*d_model elements)
 *   MLA_QUERY_AUTO      mla_query_choose_form(cfg, 1)
 * bf16 layers.  x is whatever the query projection reads (the token's hidden
 * state, width d_model).
 * ------------------------------------------------------------------------- */
typedef enum {
  MLA_QUERY_AUTO = 0,
  MLA_QUERY_UNFOLDED = 1,
  MLA_QUERY_FOLDED = 2
} mla_query_form;

/* The form with the smaller estimated time for total_q query tokens, each
 * form's time the larger of its weight bytes / 8 TB/s and its matrix-core
 * flops / 2.5 PFLOP/s.  Both scale with the weight element counts, so
 * folding wins when d_model < d_c d_nope / (d_c - d_nope): at d_model 256 for
 * d_nope >= 192 (d_c 512), never for d_nope 128.  Host only; -1 on an
 * invalid config or total_q < 1. */
int32_t mla_query_choose_form(const mla_config* cfg, int32_t total_q);

/* Bytes of the buffer mla_fold_query fills for a form (0 if unsupported). */
size_t mla_query_folded_bytes(const mla_config* cfg, int32_t form);

/* Attach the query projection to a layer.
 *   w_q   [d_model][H * (d_nope + d_rope)]  device; head h owns the columns
 *                              h*(d_nope + d_rope) .., content part first
 *   w_uk  [d_c][H * d_nope]    device, the same W_uk given to mla_fold_weights
 *                              (read for MLA_QUERY_FOLDED only; may be null otherwise)
 *   folded                     device, >= mla_query_folded_bytes(cfg, form),
 *                              256-byte aligned, kept and read by later calls
 * The inputs are read by work enqueued on hip_stream.  Errors: INVALID_ARG,
 * UNSUPPORTED (fp32 layer), INSUFFICIENT_WORKSPACE, HIP. */
mla_status mla_fold_query(mla_layer* layer, const void* w_q, const void* w_uk, int32_t form,
                          void* folded, size_t folded_bytes, void* hip_stream);

/* Workspace bytes of mla_decode_hidden for these host bounds, by the form the
 * layer was folded with (0 when no query projection is folded or the sizes
 * are invalid). */
size_t mla_decode_hidden_workspace_bytes(const mla_layer* layer, int32_t batch, int32_t total_q,
                                         int32_t max_q_len, int32_t max_seq_len);

/* mla_decode (kv_chunk 0) with its queries projected from the layer input:
 * x [total_q][d_model] (bf16) in the token order of cu_q, projected by the
 * form the layer was folded with (mla_fold_query); out [total_q][H][d_v] as
 * mla_decode.  Same arguments and contract as mla_decode otherwise; the
 * workspace is scratch for this call only.  Errors as mla_decode, and
 * INVALID_ARG when no query projection was folded. */
mla_status mla_decode_hidden(const mla_layer* layer, const void* x, const int32_t* cu_q,
                             const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                             int32_t batch, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                             const void* cache, int64_t num_pages, void* out, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* Status bookkeeping (no passage defines it): the name of a status code,
 * and the calling thread's message for its last non-OK status -- in the
 * checking build, also which sequence, length or page id failed the check of
 * device-resident arguments. */
const char* mla_status_string(mla_status s);
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */

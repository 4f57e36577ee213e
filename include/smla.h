/*
 * smla.h -- C ABI of the MI355X (gfx950) sparse MLA prefill attention library.
 *
 * The operation is the FP8-KV sparse MLA prefill described on the Modular
 * kernel API page "mla_sm100_prefill_sparse_fp8" (function description,
 * Parameters and Args), with the shared-latent K/V of the page
 * "mla_prefill_sparse_qkv_fp8": for every query token t and head h,
 *
 *   rows   : the token's first L = min(topk_lengths[t], topk) listed slots,
 *            each a logical position idx in the token's sequence, mapped to a
 *            physical row page_table[b, idx / page_size] * page_size
 *            + idx % page_size of the paged FP8 e4m3fn latent cache;
 *   k_j    : the 576-wide dequantised latent row (unit scale, one scale per
 *            row, or one scale per scale_block_size columns);
 *   v_j    : its first 512 columns (the same gathered row, no second gather);
 *   s_j    = scale * <q[t,h,:], k_j>;
 *   out    = sum_j exp(s_j) v_j / (sum_j exp(s_j) + [sink] exp(sink[h])).
 *
 * Layouts are dense row-major.  All data pointers are DEVICE pointers owned
 * by the caller; they must stay valid until the enqueued work completes.
 * `dims` is a HOST pointer read during the call.  The library allocates no
 * device memory, keeps no per-call global state (the one exception is the
 * fixed scratch array of sparse_mla_prefill_split_noalloc), never
 * synchronises, and enqueues its kernels on `stream` (a hipStream_t; NULL =
 * default stream).
 * Every check runs on the host before anything is enqueued; a non-zero status
 * means nothing was enqueued (except SMLA_ERR_LAUNCH, reported by the HIP
 * runtime after a launch).  Data-dependent conditions are not errors: a slot
 * whose index or page id is out of range is skipped (weight 0), lengths above
 * topk are clamped, and a token with no valid slot gets out = 0.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define SMLA_API __attribute__((visibility("default")))
#else
#define SMLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_NULL = 1,         /* a required pointer is NULL                          */
  SMLA_ERR_SHAPE = 2,        /* a size is negative, zero where it may not be, or
                                inconsistent (e.g. qk_depth != 576)                 */
  SMLA_ERR_UNSUPPORTED = 3,  /* valid input the library does not run (head count,
                                scale_block_size, a latent pool of 2^32 rows or
                                more, a scale table of 4 GiB or more)               */
  SMLA_ERR_MISALIGNED = 4,   /* q / out / kv_pages not 16-byte aligned, or a 4-byte
                                array not 4-byte aligned                            */
  SMLA_ERR_LAUNCH = 5,       /* the HIP runtime rejected a kernel launch            */
  SMLA_ERR_SCRATCH_LIMIT = 6 /* the split partials of a no-allocation call do not fit
                                its fixed scratch buffer                            */
} smla_status;

/* Sizes of one call.  Query tokens are packed by sequence (cu_seqlens_q). */
typedef struct {
  int32_t num_tokens;         /* T: total query tokens ("total_q_tokens")            */
  int32_t num_heads;          /* H: query heads; multiple of 16, 16..128             */
  int32_t qk_depth;           /* must be 576 (512 latent + 64 rope)                  */
  int32_t v_depth;            /* must be 512                                         */
  int32_t topk;               /* K: indices row stride ("indices_stride"), >= 0      */
  int32_t num_seqs;           /* B >= 1                                              */
  int32_t page_size;          /* rows per KV page, >= 1                              */
  int32_t max_pages_per_seq;  /* page_table row stride, >= 1                         */
  int64_t num_pages;          /* physical pages in kv_pages, >= 1                    */
} smla_dims;

/*
 * sparse_mla_prefill -- the attention (page "mla_sm100_prefill_sparse_fp8").
 *
 *   out           bf16  [T, H, 512]                written
 *   q             bf16  [T, H, 576]
 *   kv_pages      e4m3fn bytes [num_pages, page_size, 576]; fewer than
 *                 2^32 rows (pools of 4 GiB and more are read through
 *                 64-bit row addresses)
 *   page_table    int32 [B, max_pages_per_seq]     physical page ids
 *   cu_seqlens_q  int32 [B + 1]                    token offsets, non-decreasing,
 *                                                  cu[0] = 0, cu[B] = T
 *   scales        f32   [num_pages * page_size, ncols], indexed by PHYSICAL row
 *                 (below 4 GiB);
 *                 ncols = 1 if scale_block_size >= 576, else
 *                 ceil(576 / scale_block_size); may be NULL iff
 *                 scale_block_size == 0 ("scales_ptr", Parameters:
 *                 scale_block_size).  Dequantisation factors: finite and
 *                 > 0.  The kernels choose their power-of-two working ranges
 *                 from the largest scale of a tile, so zero, negative or
 *                 non-finite scales give unspecified outputs (device data:
 *                 not checked)
 *   indices       uint32 [T, topk]   logical positions inside the token's sequence
 *   topk_lengths  uint32 [T]         effective top-k count per token
 *   sink          f32 [H] or NULL    per-head logit added to the softmax
 *                                    denominator only ("attn_sink_ptr")
 *   scale         softmax scale multiplying the dot product (finite, > 0;
 *                 SMLA_ERR_SHAPE otherwise)
 *   scale_block_size  0: unit scale; >= 576: one scale per row; otherwise a
 *                     multiple of 16 below 576: blockwise (K uses all ncols
 *                     blocks, V the first ceil(512 / scale_block_size))
 *   dims          host pointer to the sizes above
 *   stream        hipStream_t
 */
SMLA_API smla_status sparse_mla_prefill(void* out, const void* q, const void* kv_pages,
                               const int32_t* page_table, const int32_t* cu_seqlens_q,
                               const float* scales, const uint32_t* indices,
                               const uint32_t* topk_lengths, const float* sink, float scale,
                               int32_t scale_block_size, const smla_dims* dims, void* stream);

/*
 * sparse_mla_prefill_split -- the same attention with each token's listed
 * slots cut into num_splits runs of ceil(ceil(topk / 64) / num_splits) 64-slot
 * tiles, one workgroup per run, and a second kernel that merges the runs'
 * partial results with log-sum-exp weights (the correction step of the page
 * "SM100MLA"; the page "sparse_index_fp8_sm100", Grid, slices an underfilled
 * grid the same way).  For few query tokens (decode, multi-token prediction)
 * this spreads the work over all CUs.  The result equals sparse_mla_prefill's
 * up to rounding (the run results are kept in f32).
 *
 *   num_splits       1..64; 1 runs exactly sparse_mla_prefill (workspace
 *                    unused, may be NULL); runs past the last listed slot are
 *                    empty and cost one small workgroup each
 *   workspace        device memory of at least
 *                    sparse_mla_split_workspace_bytes(dims, num_splits) bytes,
 *                    256-byte aligned, owned by the caller; its contents on
 *                    entry do not matter and it may be reused once the
 *                    stream's work is done
 *   workspace_bytes  its size (SMLA_ERR_SHAPE if too small)
 * Other arguments and errors as for sparse_mla_prefill.
 */
SMLA_API smla_status sparse_mla_prefill_split(void* out, const void* q, const void* kv_pages,
                               const int32_t* page_table, const int32_t* cu_seqlens_q,
                               const float* scales, const uint32_t* indices,
                               const uint32_t* topk_lengths, const float* sink, float scale,
                               int32_t scale_block_size, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, const smla_dims* dims, void* stream);

/*
 * sparse_mla_prefill_single_pass -- sparse_mla_prefill_split with q and the
 * softmax probabilities P each rounded to ONE FP8 e4m3 operand (per-head
 * power-of-two scale) before the two products, as the page
 * "mla_prefill_sparse_qkv_fp8" runs them (module description: Q, K, V and P
 * all FP8).  Half the matrix-core work of the default path, which carries q
 * and P as two FP8 terms each; the price is accuracy: the relative output
 * error is that of 3-bit mantissas (a few percent of an output's scale, not
 * the default path's bf16-level error).  Opt-in only.
 * scale_block_size below 576 (blockwise) is SMLA_ERR_UNSUPPORTED; all other
 * arguments, results and errors as for sparse_mla_prefill_split.
 */
SMLA_API smla_status sparse_mla_prefill_single_pass(void* out, const void* q, const void* kv_pages,
                               const int32_t* page_table, const int32_t* cu_seqlens_q,
                               const float* scales, const uint32_t* indices,
                               const uint32_t* topk_lengths, const float* sink, float scale,
                               int32_t scale_block_size, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, const smla_dims* dims, void* stream);

/*
 * sparse_mla_prefill_split_noalloc -- sparse_mla_prefill_split for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The run partials go to a
 * scratch array the library holds in device memory, one per GPU, for the
 * life of the process (sparse_mla_noalloc_scratch_bytes() bytes, 80 MiB);
 * nothing is allocated and nothing is synchronised.  The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress).
 *
 *   num_splits  1..64; 1 needs no scratch.  A call whose partials,
 *               sparse_mla_split_workspace_bytes(dims, num_splits), exceed
 *               the scratch size returns SMLA_ERR_SCRATCH_LIMIT and enqueues
 *               nothing (about T * num_splits * H <= 40,800 partial rows).
 * The scratch array keeps the last call's contents; every partial a call
 * reads is written by the same call first, so nothing needs clearing.  Calls
 * that overlap on one GPU (different streams or host threads with work in
 * flight at once) share the array and RACE: serialise them.  Other
 * arguments, results and errors as for sparse_mla_prefill_split.
 */
SMLA_API smla_status sparse_mla_prefill_split_noalloc(void* out, const void* q, const void* kv_pages,
                               const int32_t* page_table, const int32_t* cu_seqlens_q,
                               const float* scales, const uint32_t* indices,
                               const uint32_t* topk_lengths, const float* sink, float scale,
                               int32_t scale_block_size, int32_t num_splits, const smla_dims* dims,
                               void* stream);

/* Size of the fixed scratch array of sparse_mla_prefill_split_noalloc. */
SMLA_API size_t sparse_mla_noalloc_scratch_bytes(void);

/* Workspace bytes sparse_mla_prefill_split needs (0 for num_splits <= 1):
 * T * num_splits * H * (512 + 2) floats, in two 256-byte aligned parts. */
SMLA_API size_t sparse_mla_split_workspace_bytes(const smla_dims* dims, int32_t num_splits);

/* A run count that gives at least one workgroup per MI355X CU (256), with at
 * least two tiles per run (1 for large token counts).  More runs than that
 * cost more than they gain: each run re-reads q and writes a partial result. */
SMLA_API int32_t sparse_mla_auto_splits(const smla_dims* dims, int32_t scale_block_size);

/*
 * sparse_mla_gather_debug -- the gather stage alone, for bit-exact checks of
 * the index -> page -> row translation and of the LDS staging (the top-k
 * gather of the page "mla_prefill_sparse_qkv_fp8").  Runs the same
 * translation and the same swizzled global->LDS staging as the attention and
 * copies each staged tile back out in logical order:
 *
 *   rows_out   uint8 [T, topk, 576]  written; slot j of token t holds the raw
 *              latent bytes of its row, or zeros when the slot is not read
 *              (j >= min(topk_lengths[t], topk), index or page out of range).
 * Other arguments as for sparse_mla_prefill (num_heads is not used).
 */
SMLA_API smla_status sparse_mla_gather_debug(uint8_t* rows_out, const void* kv_pages,
                                    const int32_t* page_table, const int32_t* cu_seqlens_q,
                                    const uint32_t* indices, const uint32_t* topk_lengths,
                                    const smla_dims* dims, void* stream);

/*
 * ---------------------------------------------------------------- indexer
 * FP8 lightning indexer (page "sparse_index_fp8_sm100") and the top-k stage
 * that turns its score buffer into the index lists sparse_mla_prefill reads.
 */
typedef struct {
  int32_t num_tokens;         /* T: query tokens, packed by sequence                  */
  int32_t num_heads;          /* indexer heads: 32, 64, 96 or 128                     */
  int32_t depth;              /* must be 128                                          */
  int32_t num_seqs;           /* B >= 1                                               */
  int32_t page_size;          /* rows per key page, >= 1                              */
  int32_t max_pages_per_seq;  /* page_table row stride, >= 1                          */
  int64_t num_pages;          /* physical pages in k_pages, >= 1                      */
  int32_t score_stride;       /* columns of the score buffer, >= 1                    */
  int32_t topk;               /* K: indices row stride, >= 0                          */
} smla_index_dims;

/*
 * sparse_mla_index_scores -- the indexer's score buffer (page
 * "sparse_index_fp8_sm100", module description):
 *   scores[t, j] = k_scale[row_j] * sum_h relu(q[t,h,:] . k[row_j,:]) * q_scale[t,h]
 * for the keys j < n_t of token t's causal prefix, and -inf for n_t <= j <
 * score_stride.  Query token i of sequence b sits at position
 * seq_lens_k[b] - q_len_b + i and sees keys 0..position (n_t = position + 1,
 * 0 when negative, at most score_stride); row_j = page_table[b, j / P] * P +
 * j % P, and a page id outside [0, num_pages) gives the key -inf.
 *
 *   scores        f32 [T, score_stride]          written
 *   q             e4m3fn bytes [T, num_heads, 128]   (16-byte aligned)
 *   q_scale       f32 [T, num_heads]                 (16-byte aligned)
 *   k_pages       e4m3fn bytes [num_pages, page_size, 128] (16-byte aligned)
 *   k_scale       f32 [num_pages * page_size], indexed by physical row
 *   page_table    int32 [B, max_pages_per_seq]
 *   cu_seqlens_q  int32 [B + 1]   token offsets, non-decreasing, cu[0] = 0, cu[B] = T
 *   seq_lens_k    int32 [B]       keys of each sequence
 * Device pointers owned by the caller; checks, errors and stream behaviour as
 * for sparse_mla_prefill (pool bytes num_pages * page_size * 128 below 4 GiB).
 */
SMLA_API smla_status sparse_mla_index_scores(float* scores, const void* q, const float* q_scale,
                                    const void* k_pages, const float* k_scale, const int32_t* page_table,
                                    const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                    const smla_index_dims* dims, void* stream);

/*
 * sparse_mla_index_topk -- the top-k stage the indexer page leaves to a later
 * step, in its plain reading: for token t, the L = min(topk, n_t) keys of
 * scores[t, 0:n_t] with the largest scores, ties going to the lower key index
 * (NaN below -inf, -0 equal to +0), written to indices[t, 0:L] in ascending
 * key order; indices[t, L:topk] = 0xFFFFFFFF and topk_lengths[t] = L.  n_t is
 * the causal count defined for sparse_mla_index_scores.  The output feeds
 * sparse_mla_prefill (indices / topk_lengths, indices_stride = topk).
 *
 *   indices       uint32 [T, topk]  written (may be NULL iff topk == 0)
 *   topk_lengths  uint32 [T]        written
 *   scores        f32 [T, score_stride]
 * Other arguments as for sparse_mla_index_scores (q and k sizes are not used).
 */
SMLA_API smla_status sparse_mla_index_topk(uint32_t* indices, uint32_t* topk_lengths, const float* scores,
                                  const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                  const smla_index_dims* dims, void* stream);

/* ------------------------------------------------------------------ dense */

/* Sizes of a dense MLA prefill call (host struct). */
typedef struct {
  int32_t num_seqs;           /* B >= 1                                                */
  int32_t max_prompt_len;     /* S >= 1: rows per sequence in q and out (padded)       */
  int32_t num_heads;          /* H >= 1                                                */
  int32_t num_kv_heads;       /* K_nope / V heads, >= 1, dividing H                    */
  int32_t nope_depth;         /* must be 128                                           */
  int32_t rope_depth;         /* must be 64                                            */
  int32_t v_depth;            /* must be 128                                           */
  int32_t page_size;          /* rows per page, >= 1                                   */
  int32_t max_pages_per_seq;  /* page_table row stride; max_pages_per_seq * page_size
                                 must cover max_prompt_len                             */
  int64_t num_pages;          /* physical pages in each cache, >= 1                    */
  int32_t causal;             /* 1: key j visible to row i iff j <= i; 0: all keys     */
} smla_dense_dims;

/*
 * mla_dense_prefill -- dense MLA prefill with a block-scaled FP8 K_rope (page
 * "mla_sm100_prefill_blockscale", function description, Parameters and Args;
 * the 64-wide rope part of K from the "SM100MLA" page, comptime members).
 * With L_b = min(valid_length[b], S), row i < L_b of sequence b and head h
 * (kv head h / (H / num_kv_heads)) attend over the keys j < L_b of the
 * sequence (j <= i when causal):
 *   k_j = [k_nope[row_j, hk, 0:128], fp8(k_rope[row_j, 0:64]) * sigma(row_j, c)]
 *   out[b*S + i, h, :] = sum_j softmax_j(scale * q[b*S + i, h, :] . k_j) v[row_j, hk, :]
 * with row_j = page_table[b, j / P] * P + j % P (one table for the three
 * caches); a page id outside [0, num_pages) masks its keys.  sigma follows
 * scale_block_size: 0 = 1 (k_rope_scales NULL), >= 64 = k_rope_scales[row, 0],
 * 16, 32 or 48 = k_rope_scales[row, c / sbs] (ceil(64 / sbs) columns).  As
 * the page describes, K_rope is turned into BF16 before the BF16 matrix
 * products.  Rows i >= L_b and rows with no visible key are written as 0.
 *
 *   out            bf16 [B * S, H, 128]            written
 *   q              bf16 [B * S, H, 192]  (nope 128 | rope 64)
 *   k_nope         bf16 [num_pages, P, num_kv_heads, 128]
 *   v              bf16 [num_pages, P, num_kv_heads, 128]
 *   k_rope         e4m3fn bytes [num_pages, P, 64]
 *   k_rope_scales  f32 [num_pages * P, ncols] or NULL (scale_block_size 0)
 *   page_table     int32 [B, max_pages_per_seq]
 *   valid_length   uint32 [B]
 * scale is the softmax scale (finite, > 0).  Device pointers owned by the
 * caller, 16-byte aligned (page_table, valid_length, k_rope_scales: 4);
 * dims is a host pointer.  Checks run on the host before anything is
 * enqueued and fail with SMLA_ERR_NULL, _SHAPE (sizes, a page table shorter
 * than max_prompt_len, a bad scale), _UNSUPPORTED (depths other than
 * 128 / 64 / 128, scale_block_size not 0, >= 64, 16, 32 or 48, a K_nope / V
 * cache of 2 GiB or more) or _MISALIGNED; the work is enqueued on
 * `stream` (a hipStream_t, NULL = default stream) and nothing synchronises.
 */
SMLA_API smla_status mla_dense_prefill(void* out, const void* q, const void* k_nope, const void* v,
                                       const void* k_rope, const float* k_rope_scales,
                                       const int32_t* page_table, const uint32_t* valid_length, float scale,
                                       int32_t scale_block_size, const smla_dense_dims* dims, void* stream);

/* Static text for a status code. */
SMLA_API const char* smla_status_string(smla_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
SMLA_API int32_t smla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */

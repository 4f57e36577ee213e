// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

struct AttnParams {
  uint16_t* out;              // bf16 [T, H, 512]
  const uint16_t* q;          // bf16 [T, H, 576]
  const uint8_t* kv;          // e4m3fn [num_pages, P, 576]
  const int32_t* page_table;  // [B, max_pages]
  const int32_t* cu_seqlens;  // [B + 1]
  const float* scales;        // [num_pages * P, ncols] or null
  const uint32_t* indices;    // [T, K]
  const uint32_t* lengths;    // [T]
  const float* sink;          // [H] or null
  float scale_log2;           // softmax scale * log2(e)
  uint32_t num_rows;          // num_pages * P (< 2^32)
  uint32_t kv_bytes;          // num_rows * 576 when below 4 GiB - 1 KiB, else 0
  int wide_pool;              // 1: the pool is 4 GiB - 1 KiB or more (64-bit row addresses)
  uint32_t scale_bytes;       // num_pages * P * ncols * 4
  int T, H, K, B, P, max_pages, num_pages;
  int sbs;                    // 0 unit, >= 576 one scale per row, else block size
  int scale_cols;             // columns of the scale table (0, 1 or ceil(576 / sbs))
  // split top-k: each token's slots are cut into `splits` runs of
  // `split_tiles` 64-slot tiles, one workgroup each; with splits > 1 the
  // workgroups write partial results that smla_combine turns into `out`.
  int splits;                 // >= 1
  int split_tiles;            // tiles per run
  float* part_o;              // [T, splits, H, 512] numerators, in units of 2^-m (splits > 1)
  float* part_ml;             // [T, splits, H, 2]: running max m (log2 domain), row sum l
  int single_pass;            // 1: q and P as one FP8 term each (fp8 path only)
};

// FP8 lightning indexer: scores and their top-k selection.
struct IndexParams {
  float* scores;              // [T, stride]
  const uint8_t* q;           // e4m3fn [T, H, 128]
  const float* q_scale;       // [T, H]
  const uint8_t* k;           // e4m3fn [num_pages, P, 128]
  const float* k_scale;       // [num_pages * P]
  const int32_t* page_table;  // [B, max_pages]
  const int32_t* cu_seqlens;  // [B + 1]
  const int32_t* seq_lens_k;  // [B]
  uint32_t* indices;          // [T, K] (top-k)
  uint32_t* lengths;          // [T]    (top-k)
  uint32_t k_bytes;           // num_pages * P * 128
  uint32_t ks_bytes;          // num_pages * P * 4
  int T, H, B, P, max_pages, num_pages, stride, K;
};
hipError_t launch_index_scores(const IndexParams& p, hipStream_t stream);
hipError_t launch_index_topk(const IndexParams& p, hipStream_t stream);

// Dense MLA prefill with a block-scaled FP8 K_rope (BF16 MFMA).
struct DenseParams {
  uint16_t* out;                 // bf16 [B * S, H, 128]
  const uint16_t* q;             // bf16 [B * S, H, 192]
  const uint8_t* k_nope;         // bf16 [num_pages, P, Hkv, 128]
  const uint8_t* v;              // bf16 [num_pages, P, Hkv, 128]
  const uint8_t* k_rope;         // e4m3fn [num_pages, P, 64]
  const float* rope_scales;      // [num_pages * P, scale_cols] or null
  const int32_t* page_table;     // [B, max_pages]
  const uint32_t* valid_length;  // [B]
  float scale_log2;              // softmax scale * log2(e)
  uint32_t kn_bytes, v_bytes;    // sizes of the K_nope and V caches (< 2^31)
  uint32_t kr_bytes, sc_bytes;   // sizes of the K_rope cache and its scale table
  int B, S, H, Hkv, P, max_pages, num_pages;
  int P_log2;                    // log2(P) when P is a power of two, else -1
  int sbs;                       // 0 unit, >= 64 one scale per row, else 16, 32 or 48
  int scale_cols;                // 0, 1 or 64 / sbs rounded up
  int causal;                    // 1: key j visible to row i iff j <= i
  int row_blocks;                // blocks of query rows per sequence (set by launch_dense)
};
hipError_t launch_dense(const DenseParams& p, hipStream_t stream);

// FP8 MFMA path (unit and one-scale-per-row modes).
hipError_t launch_fp8x2(const AttnParams& p, hipStream_t stream);
// The same, 64 heads per workgroup as two pairs of waves (pipelined softmax).
hipError_t launch_fp8pair(const AttnParams& p, hipStream_t stream);
// FP16 MFMA path (blockwise scales: dequantised once per tile in LDS), one
// workgroup per (token, 64 heads), 16 heads per wave.
hipError_t launch_f16_block(const AttnParams& p, hipStream_t stream);
// The same with one workgroup per token for up to 128 heads, 32 heads per wave.
hipError_t launch_f16_wide(const AttnParams& p, hipStream_t stream);
// Combine the partial results of a split launch into out (sink in the denominator).
hipError_t launch_combine(const AttnParams& p, hipStream_t stream);
// Gather-only debug path.
hipError_t launch_gather_debug(uint8_t* rows_out, const AttnParams& p, hipStream_t stream);

}  // namespace smla

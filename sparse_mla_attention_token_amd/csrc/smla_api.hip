// C ABI of the sparse MLA prefill library: host-side validation, dispatch to
// the gfx950 kernels, and the gather-only debug kernel.
//
// The argument set follows the page "mla_sm100_prefill_sparse_fp8"
// (output, q, paged FP8 kv_cache, indices, topk_lengths, optional
// attn_sink_ptr, scales_ptr, scale, scale_block_size) with the paged cache
// spelled out as kv_pages + page_table and the packed query tokens described
// by cu_seqlens_q.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/smla.h"
#include "smla_device.h"
#include "smla_gather.h"
#include "smla_kernels.h"

namespace smla {
namespace {

// One workgroup (4 waves) per token: translate each tile synchronously, stage
// it through the same swizzled global->LDS path as the attention, and copy it
// back out in logical (row, column) order.
template <bool WIDE>
__global__ __launch_bounds__(256, 1) void smla_gather_debug_kernel(uint8_t* rows_out, AttnParams p) {
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(1024))) uint8_t tile[kTileBytes];
  __shared__ u32 rowid[kBK];
  __shared__ u32 vmask[2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int b = token_sequence(p.cu_seqlens, p.B, t);
  TokenSlots ts;
  ts.L = 0;
  ts.idx_row = p.indices + (size_t)t * p.K;
  ts.pt_row = p.page_table + (size_t)(b < p.B ? b : 0) * p.max_pages;
  if (b < p.B) {
    u32 len = p.lengths[t];
    ts.L = len < (u32)p.K ? len : (u32)p.K;
  }
  GatherArgs ga;
  ga.kv = p.kv;
  ga.page_table = p.page_table;
  ga.indices = p.indices;
  ga.num_rows = p.num_rows;
  ga.kv_bytes = p.kv_bytes;
  const v4i kv_rsrc = make_rsrc(p.kv, p.kv_bytes);
  ga.K = p.K;
  ga.P = p.P;
  ga.max_pages = p.max_pages;
  ga.num_pages = p.num_pages;
  uint8_t* dst = rows_out + (size_t)t * p.K * kQK;
  const int ntiles_all = (p.K + kBK - 1) / kBK;  // every slot of the row is written
  for (int tl = 0; tl < ntiles_all; ++tl) {
    if (wave == 0) {
      u32 ix = slot_index(ts, tl, lane);
      int pg = slot_page(ts, ga, tl, lane, ix);
      publish_slots(ga, ix, pg, rowid, vmask, lane);
    }
    __syncthreads();
    gather_tile<NW, WIDE>(kv_rsrc, ga, rowid, tile, wave, lane);
    wait_vmem_all();
    __syncthreads();
    for (u32 s = threadIdx.x; s < (u32)(kBK * kRowGranules); s += blockDim.x) {
      const u32 row = s / kRowGranules, gl = s % kRowGranules;
      const u32 j = (u32)tl * kBK + row;
      if (j < (u32)p.K) {
        const v4i v = *(const v4i*)(tile + tile_off(row, gl));
        *(v4i*)(dst + (size_t)j * kQK + 16u * gl) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gather_debug(uint8_t* rows_out, const AttnParams& p, hipStream_t stream) {
  if (p.wide_pool) hipLaunchKernelGGL(smla_gather_debug_kernel<true>, dim3(p.T), dim3(256), 0, stream, rows_out, p);
  else hipLaunchKernelGGL(smla_gather_debug_kernel<false>, dim3(p.T), dim3(256), 0, stream, rows_out, p);
  return hipGetLastError();
}

}  // namespace smla

namespace {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// Shape and support checks shared by both entry points.
smla_status check_dims(const smla_dims* dims, bool need_heads) {
  if (!dims) return SMLA_ERR_NULL;
  const smla_dims& d = *dims;
  if (d.num_tokens < 0 || d.topk < 0 || d.num_seqs < 1 || d.page_size < 1 || d.max_pages_per_seq < 1 ||
      d.num_pages < 1)
    return SMLA_ERR_SHAPE;
  if (d.qk_depth != smla::kQK || d.v_depth != smla::kV) return SMLA_ERR_SHAPE;
  if (need_heads) {
    if (d.num_heads < 1) return SMLA_ERR_SHAPE;
    if (d.num_heads % 16 != 0 || d.num_heads > 128) return SMLA_ERR_UNSUPPORTED;
  }
  // pool rows are 32-bit ids (the gather itself uses 64-bit addresses); the
  // id num_pages * page_size marks a slot that is not read
  const long double rows = (long double)d.num_pages * (long double)d.page_size;
  if (rows > (long double)0xFFFFFFFFull) return SMLA_ERR_UNSUPPORTED;
  if (d.num_pages > INT_MAX) return SMLA_ERR_UNSUPPORTED;
  return SMLA_OK;
}

smla::AttnParams make_params(const smla_dims& d) {
  smla::AttnParams p{};
  p.T = d.num_tokens;
  p.H = d.num_heads;
  p.K = d.topk;
  p.B = d.num_seqs;
  p.P = d.page_size;
  p.max_pages = d.max_pages_per_seq;
  p.num_pages = (int)d.num_pages;
  p.num_rows = (uint32_t)(d.num_pages * d.page_size);
  const uint64_t pool = (uint64_t)p.num_rows * (uint64_t)smla::kQK;
  p.wide_pool = pool > 0xFFFFFFFFull - 1024ull ? 1 : 0;
  p.kv_bytes = p.wide_pool ? 0u : (uint32_t)pool;
  return p;
}

constexpr int kMaxSplits = 64;                 // runs per token
constexpr long long kSplitTargetWorkgroups = 256;  // one per CU

// More than 64 heads and fewer tokens than CUs, yet one workgroup per
// (token, 64-head group) covers every CU: the FP8 path then runs the paired
// kernel over the head groups in one run.
bool fp8_heads_fill(long long T, long long H) {
  const long long groups = (H + 63) / 64;
  return H > 64 && T < kSplitTargetWorkgroups && T * groups >= kSplitTargetWorkgroups;
}

// Workspace of a split launch: partial numerators [T, S, H, 512] f32, then
// (m, l) pairs [T, S, H, 2] f32, each 256-byte aligned.
struct SplitLayout {
  size_t o_offset, ml_offset, total;
};

SplitLayout split_layout(const smla_dims& d, int S) {
  const size_t rows = (size_t)d.num_tokens * (size_t)S * (size_t)d.num_heads;
  SplitLayout l;
  l.o_offset = 0;
  l.ml_offset = (rows * smla::kV * 4 + 255) & ~(size_t)255;
  l.total = l.ml_offset + ((rows * 2 * 4 + 255) & ~(size_t)255);
  return l;
}

}  // namespace

extern "C" {

smla_status sparse_mla_prefill(void* out, const void* q, const void* kv_pages, const int32_t* page_table,
                               const int32_t* cu_seqlens_q, const float* scales, const uint32_t* indices,
                               const uint32_t* topk_lengths, const float* sink, float scale,
                               int32_t scale_block_size, const smla_dims* dims, void* stream) {
  return sparse_mla_prefill_split(out, q, kv_pages, page_table, cu_seqlens_q, scales, indices, topk_lengths, sink,
                                  scale, scale_block_size, 1, nullptr, 0, dims, stream);
}

size_t sparse_mla_split_workspace_bytes(const smla_dims* dims, int32_t num_splits) {
  if (!dims || num_splits <= 1 || dims->num_tokens <= 0 || dims->num_heads <= 0) return 0;
  return split_layout(*dims, num_splits).total;
}

int32_t sparse_mla_auto_splits(const smla_dims* dims, int32_t scale_block_size) {
  if (!dims || dims->num_tokens <= 0 || dims->topk <= 0) return 1;
  const bool block = scale_block_size > 0 && scale_block_size < smla::kQK;
  if (!block && fp8_heads_fill(dims->num_tokens, dims->num_heads)) return 1;  // head groups, one run
  const long long groups = 1;  // workgroups per token and run (every path takes all heads of a token)
  const long long wgs = (long long)dims->num_tokens * groups;
  const long long tiles = ((long long)dims->topk + smla::kBK - 1) / smla::kBK;
  long long s = (kSplitTargetWorkgroups + wgs - 1) / wgs;         // one workgroup per CU
  const long long max_s = tiles / 2 > 0 ? tiles / 2 : 1;          // at least two tiles per run
  if (s > max_s) s = max_s;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int32_t)s;
}

}  // extern "C"

namespace {

// FP8 path.  Up to 64 heads, the paired-wave kernel (two waves share 32 heads
// and split each tile's keys and output columns) keeps all four waves of a
// workgroup busy; with more heads, one workgroup per token and 32 heads per
// wave does less exchange per key.  The exception is a launch of one run
// whose tokens alone would leave CUs idle while their 64-head groups fill
// them (decode-sized batches): there the paired kernel over the head groups
// beats split runs of the one-workgroup kernel plus their combine.
hipError_t launch_fp8(const smla::AttnParams& p, hipStream_t s) {
  const bool pair = p.H <= 64 || (p.splits == 1 && fp8_heads_fill(p.T, p.H));
  return pair ? smla::launch_fp8pair(p, s) : smla::launch_fp8x2(p, s);
}

// ------------------------------------------------------------ fixed scratch
// Partial results of split launches for callers that cannot allocate
// (sparse_mla_prefill_split_noalloc).  The array lives in the code object:
// every GPU the library runs on holds its own copy until the process ends.
// Host code never uses the array's name as an address (on the host it names
// a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(80) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (set up on the
// first call on that device); nullptr when HIP reports an error.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Blockwise path.  More than 64 heads: one workgroup per token, 32 heads per
// wave, so each tile is gathered and dequantised once for all heads; up to 64
// heads, one workgroup per token with 16 heads per wave keeps all four waves
// busy.
bool blockwise_wide(int H) { return H > 64; }

hipError_t launch_blockwise(const smla::AttnParams& p, hipStream_t s) {
  return blockwise_wide(p.H) ? smla::launch_f16_wide(p, s) : smla::launch_f16_block(p, s);
}

// Body shared by the two-pass, the single-pass and the no-allocation entry
// points.  use_scratch: the split partials go to the fixed scratch array
// instead of `workspace` (which is then ignored).
smla_status run_prefill(void* out, const void* q, const void* kv_pages, const int32_t* page_table,
                        const int32_t* cu_seqlens_q, const float* scales, const uint32_t* indices,
                        const uint32_t* topk_lengths, const float* sink, float scale, int32_t scale_block_size,
                        int32_t num_splits, void* workspace, size_t workspace_bytes, const smla_dims* dims,
                        void* stream, bool single_pass, bool use_scratch = false) {
  smla_status st = check_dims(dims, true);
  if (st != SMLA_OK) return st;
  const smla_dims d = *dims;
  const int sbs = scale_block_size;
  if (sbs < 0) return SMLA_ERR_SHAPE;
  if (sbs > 0 && sbs < smla::kQK && sbs % 16 != 0) return SMLA_ERR_UNSUPPORTED;
  if (single_pass && sbs > 0 && sbs < smla::kQK) return SMLA_ERR_UNSUPPORTED;  // fp8 kernel modes only
  if (!(scale > 0.0f) || scale == __builtin_huge_valf()) return SMLA_ERR_SHAPE;  // softmax scale: finite, > 0
  if (num_splits < 1 || num_splits > kMaxSplits) return SMLA_ERR_SHAPE;
  if (d.num_tokens == 0) return SMLA_OK;
  if (!out || !q || !kv_pages || !page_table || !cu_seqlens_q || !topk_lengths) return SMLA_ERR_NULL;
  if (d.topk > 0 && !indices) return SMLA_ERR_NULL;
  if (sbs != 0 && !scales) return SMLA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(kv_pages, 16)) return SMLA_ERR_MISALIGNED;
  if (!aligned(page_table, 4) || !aligned(cu_seqlens_q, 4) || !aligned(indices, 4) || !aligned(topk_lengths, 4) ||
      !aligned(scales, 4) || !aligned(sink, 4))
    return SMLA_ERR_MISALIGNED;
  SplitLayout lay{};
  if (num_splits > 1 && use_scratch) {
    lay = split_layout(d, num_splits);
    if (lay.total > kScratchBytes) return SMLA_ERR_SCRATCH_LIMIT;
    workspace = scratch_for_current_device();
    if (!workspace) return SMLA_ERR_LAUNCH;
    workspace_bytes = kScratchBytes;
  }
  if (num_splits > 1) {
    if (!workspace) return SMLA_ERR_NULL;
    if (!aligned(workspace, 256)) return SMLA_ERR_MISALIGNED;
    lay = split_layout(d, num_splits);
    if (workspace_bytes < lay.total) return SMLA_ERR_SHAPE;
  }

  smla::AttnParams p = make_params(d);
  p.out = static_cast<uint16_t*>(out);
  p.q = static_cast<const uint16_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_pages);
  p.page_table = page_table;
  p.cu_seqlens = cu_seqlens_q;
  p.indices = indices;
  p.lengths = topk_lengths;
  p.sink = sink;
  p.scales = sbs != 0 ? scales : nullptr;
  p.scale_log2 = scale * smla::kLog2e;
  p.sbs = sbs;
  p.scale_cols = sbs == 0 ? 0 : (sbs >= smla::kQK ? 1 : (smla::kQK + sbs - 1) / sbs);
  const uint64_t rows = (uint64_t)d.num_pages * (uint64_t)d.page_size;
  const uint64_t sbytes = rows * (uint64_t)p.scale_cols * 4ull;
  if (sbytes > 0xFFFFFFFFull - 1024ull) return SMLA_ERR_UNSUPPORTED;
  p.scale_bytes = (uint32_t)sbytes;
  const int tiles = (d.topk + smla::kBK - 1) / smla::kBK;
  p.splits = num_splits;
  p.split_tiles = tiles > 0 ? (tiles + num_splits - 1) / num_splits : 1;
  if (num_splits > 1) {
    p.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + lay.o_offset);
    p.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + lay.ml_offset);
  }
  p.single_pass = single_pass ? 1 : 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the check below sees only this launch
  hipError_t e = (sbs == 0 || sbs >= smla::kQK) ? launch_fp8(p, s) : launch_blockwise(p, s);
  if (e == hipSuccess && num_splits > 1) e = smla::launch_combine(p, s);
  if (e == hipErrorNotSupported) return SMLA_ERR_UNSUPPORTED;
  return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

smla_status sparse_mla_prefill_split(void* out, const void* q, const void* kv_pages, const int32_t* page_table,
                                     const int32_t* cu_seqlens_q, const float* scales, const uint32_t* indices,
                                     const uint32_t* topk_lengths, const float* sink, float scale,
                                     int32_t scale_block_size, int32_t num_splits, void* workspace,
                                     size_t workspace_bytes, const smla_dims* dims, void* stream) {
  return run_prefill(out, q, kv_pages, page_table, cu_seqlens_q, scales, indices, topk_lengths, sink, scale,
                     scale_block_size, num_splits, workspace, workspace_bytes, dims, stream, false);
}

smla_status sparse_mla_prefill_split_noalloc(void* out, const void* q, const void* kv_pages,
                                             const int32_t* page_table, const int32_t* cu_seqlens_q,
                                             const float* scales, const uint32_t* indices,
                                             const uint32_t* topk_lengths, const float* sink, float scale,
                                             int32_t scale_block_size, int32_t num_splits, const smla_dims* dims,
                                             void* stream) {
  return run_prefill(out, q, kv_pages, page_table, cu_seqlens_q, scales, indices, topk_lengths, sink, scale,
                     scale_block_size, num_splits, nullptr, 0, dims, stream, false, true);
}

size_t sparse_mla_noalloc_scratch_bytes(void) { return kScratchBytes; }

smla_status sparse_mla_prefill_single_pass(void* out, const void* q, const void* kv_pages,
                                           const int32_t* page_table, const int32_t* cu_seqlens_q,
                                           const float* scales, const uint32_t* indices,
                                           const uint32_t* topk_lengths, const float* sink, float scale,
                                           int32_t scale_block_size, int32_t num_splits, void* workspace,
                                           size_t workspace_bytes, const smla_dims* dims, void* stream) {
  return run_prefill(out, q, kv_pages, page_table, cu_seqlens_q, scales, indices, topk_lengths, sink, scale,
                     scale_block_size, num_splits, workspace, workspace_bytes, dims, stream, true);
}

smla_status sparse_mla_gather_debug(uint8_t* rows_out, const void* kv_pages, const int32_t* page_table,
                                    const int32_t* cu_seqlens_q, const uint32_t* indices,
                                    const uint32_t* topk_lengths, const smla_dims* dims, void* stream) {
  smla_status st = check_dims(dims, false);
  if (st != SMLA_OK) return st;
  const smla_dims d = *dims;
  if (d.num_tokens == 0 || d.topk == 0) return SMLA_OK;
  if (!rows_out || !kv_pages || !page_table || !cu_seqlens_q || !indices || !topk_lengths) return SMLA_ERR_NULL;
  if (!aligned(rows_out, 16) || !aligned(kv_pages, 16)) return SMLA_ERR_MISALIGNED;
  if (!aligned(page_table, 4) || !aligned(cu_seqlens_q, 4) || !aligned(indices, 4) || !aligned(topk_lengths, 4))
    return SMLA_ERR_MISALIGNED;
  smla::AttnParams p = make_params(d);
  p.kv = static_cast<const uint8_t*>(kv_pages);
  p.page_table = page_table;
  p.cu_seqlens = cu_seqlens_q;
  p.indices = indices;
  p.lengths = topk_lengths;
  (void)hipGetLastError();
  hipError_t e = smla::launch_gather_debug(rows_out, p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

smla_status check_index_dims(const smla_index_dims* dims, smla::IndexParams* p) {
  if (!dims) return SMLA_ERR_NULL;
  const smla_index_dims& d = *dims;
  if (d.num_tokens < 0 || d.num_seqs < 1 || d.page_size < 1 || d.max_pages_per_seq < 1 || d.num_pages < 1 ||
      d.score_stride < 1 || d.topk < 0 || d.num_heads < 1)
    return SMLA_ERR_SHAPE;
  if (d.depth != 128) return SMLA_ERR_SHAPE;
  if (d.num_heads % 32 != 0 || d.num_heads > 128) return SMLA_ERR_UNSUPPORTED;
  // 32-bit byte offsets into the key pool and its scale table
  const long double pool = (long double)d.num_pages * (long double)d.page_size * 128.0L;
  if (pool > (long double)(0xFFFFFFFFull - 1024ull) || d.num_pages > INT_MAX) return SMLA_ERR_UNSUPPORTED;
  *p = smla::IndexParams{};
  p->T = d.num_tokens;
  p->H = d.num_heads;
  p->B = d.num_seqs;
  p->P = d.page_size;
  p->max_pages = d.max_pages_per_seq;
  p->num_pages = (int)d.num_pages;
  p->stride = d.score_stride;
  p->K = d.topk;
  p->k_bytes = (uint32_t)(d.num_pages * d.page_size * 128);
  p->ks_bytes = (uint32_t)(d.num_pages * d.page_size * 4);
  return SMLA_OK;
}

}  // namespace

extern "C" {

smla_status sparse_mla_index_scores(float* scores, const void* q, const float* q_scale, const void* k_pages,
                                    const float* k_scale, const int32_t* page_table, const int32_t* cu_seqlens_q,
                                    const int32_t* seq_lens_k, const smla_index_dims* dims, void* stream) {
  smla::IndexParams p;
  smla_status st = check_index_dims(dims, &p);
  if (st != SMLA_OK) return st;
  if (p.T == 0) return SMLA_OK;
  if (!scores || !q || !q_scale || !k_pages || !k_scale || !page_table || !cu_seqlens_q || !seq_lens_k)
    return SMLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(q_scale, 16)) return SMLA_ERR_MISALIGNED;
  if (!aligned(scores, 4) || !aligned(k_scale, 4) || !aligned(page_table, 4) || !aligned(cu_seqlens_q, 4) ||
      !aligned(seq_lens_k, 4))
    return SMLA_ERR_MISALIGNED;
  p.scores = scores;
  p.q = static_cast<const uint8_t*>(q);
  p.q_scale = q_scale;
  p.k = static_cast<const uint8_t*>(k_pages);
  p.k_scale = k_scale;
  p.page_table = page_table;
  p.cu_seqlens = cu_seqlens_q;
  p.seq_lens_k = seq_lens_k;
  (void)hipGetLastError();
  const hipError_t e = smla::launch_index_scores(p, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return SMLA_ERR_UNSUPPORTED;
  return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

smla_status sparse_mla_index_topk(uint32_t* indices, uint32_t* topk_lengths, const float* scores,
                                  const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                  const smla_index_dims* dims, void* stream) {
  smla::IndexParams p;
  smla_status st = check_index_dims(dims, &p);
  if (st != SMLA_OK) return st;
  if (p.T == 0) return SMLA_OK;
  if (!topk_lengths || !scores || !cu_seqlens_q || !seq_lens_k || (p.K > 0 && !indices)) return SMLA_ERR_NULL;
  if (!aligned(indices, 4) || !aligned(topk_lengths, 4) || !aligned(scores, 4) || !aligned(cu_seqlens_q, 4) ||
      !aligned(seq_lens_k, 4))
    return SMLA_ERR_MISALIGNED;
  p.indices = indices;
  p.lengths = topk_lengths;
  p.scores = const_cast<float*>(scores);
  p.cu_seqlens = cu_seqlens_q;
  p.seq_lens_k = seq_lens_k;
  (void)hipGetLastError();
  const hipError_t e = smla::launch_index_topk(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

smla_status mla_dense_prefill(void* out, const void* q, const void* k_nope, const void* v, const void* k_rope,
                              const float* k_rope_scales, const int32_t* page_table, const uint32_t* valid_length,
                              float scale, int32_t scale_block_size, const smla_dense_dims* dims, void* stream) {
  if (!dims) return SMLA_ERR_NULL;
  const smla_dense_dims& d = *dims;
  if (d.num_seqs < 1 || d.max_prompt_len < 1 || d.num_heads < 1 || d.num_kv_heads < 1 || d.page_size < 1 ||
      d.max_pages_per_seq < 1 || d.num_pages < 1 || (d.causal != 0 && d.causal != 1))
    return SMLA_ERR_SHAPE;
  if (d.num_heads % d.num_kv_heads != 0) return SMLA_ERR_SHAPE;
  if (d.nope_depth != 128 || d.rope_depth != 64 || d.v_depth != 128) return SMLA_ERR_UNSUPPORTED;
  if ((long long)d.max_pages_per_seq * d.page_size < d.max_prompt_len) return SMLA_ERR_SHAPE;
  if (!(scale > 0.0f) || scale == __builtin_huge_valf()) return SMLA_ERR_SHAPE;  // softmax scale: finite, > 0
  const int sbs = scale_block_size;
  if (sbs < 0 || (sbs > 0 && sbs < 64 && sbs % 16 != 0)) return SMLA_ERR_UNSUPPORTED;
  const int ncols = sbs == 0 ? 0 : (sbs >= 64 ? 1 : (64 + sbs - 1) / sbs);
  const long long rows = d.num_pages * (long long)d.page_size;
  const long long cache_bytes = rows * d.num_kv_heads * 128 * 2;
  const long long q_rows = (long long)d.num_seqs * d.max_prompt_len;
  if (cache_bytes >= (1ll << 31) || rows * 64 >= (1ll << 31) || q_rows * d.num_heads * 192 >= (1ll << 40))
    return SMLA_ERR_UNSUPPORTED;
  if ((long long)d.num_seqs * d.num_heads * ((d.max_prompt_len + 127) / 128) >= (1ll << 31)) return SMLA_ERR_UNSUPPORTED;
  if (!out || !q || !k_nope || !v || !k_rope || !page_table || !valid_length || (sbs != 0 && !k_rope_scales))
    return SMLA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_nope, 16) || !aligned(v, 16) || !aligned(k_rope, 16) ||
      !aligned(page_table, 4) || !aligned(valid_length, 4) || (k_rope_scales && !aligned(k_rope_scales, 4)))
    return SMLA_ERR_MISALIGNED;
  smla::DenseParams p;
  p.out = static_cast<uint16_t*>(out);
  p.q = static_cast<const uint16_t*>(q);
  p.k_nope = static_cast<const uint8_t*>(k_nope);
  p.v = static_cast<const uint8_t*>(v);
  p.k_rope = static_cast<const uint8_t*>(k_rope);
  p.rope_scales = sbs == 0 ? nullptr : k_rope_scales;
  p.page_table = page_table;
  p.valid_length = valid_length;
  p.scale_log2 = scale * smla::kLog2e;
  p.kn_bytes = (uint32_t)cache_bytes;
  p.v_bytes = (uint32_t)cache_bytes;
  p.kr_bytes = (uint32_t)(rows * 64);
  p.sc_bytes = (uint32_t)(rows * ncols * 4);
  p.B = d.num_seqs;
  p.S = d.max_prompt_len;
  p.H = d.num_heads;
  p.Hkv = d.num_kv_heads;
  p.P = d.page_size;
  p.P_log2 = (d.page_size & (d.page_size - 1)) == 0 ? __builtin_ctz((unsigned)d.page_size) : -1;
  p.max_pages = d.max_pages_per_seq;
  p.num_pages = (int)d.num_pages;
  p.sbs = sbs;
  p.scale_cols = ncols;
  p.causal = d.causal;
  p.row_blocks = 0;
  (void)hipGetLastError();
  const hipError_t e = smla::launch_dense(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

const char* smla_status_string(smla_status status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_NULL: return "a required pointer is NULL";
    case SMLA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case SMLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SMLA_ERR_MISALIGNED: return "misaligned pointer";
    case SMLA_ERR_LAUNCH: return "kernel launch failed";
    case SMLA_ERR_SCRATCH_LIMIT: return "request exceeds the fixed scratch buffer of the no-allocation entry point";
  }
  return "unknown status";
}

int32_t smla_version(void) { return 100; }

}  // extern "C"

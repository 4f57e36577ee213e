// Index translation and the swizzled global->LDS row gather, shared by the
// attention kernels and the gather-only debug kernel so that the bytes the
// debug entry point returns are the bytes the attention consumes.
//
// Source: the "mla_sm100_prefill_sparse_fp8" page (Args: indices are
// per-query uint32 slots, topk_lengths the effective count, the KV cache is
// paged, scales live in physical-row space) and the "mla_prefill_sparse_qkv_fp8"
// page (rows are gathered 64 at a time into one K/V buffer).  Reading of the
// index space: a slot holds a logical position in the token's sequence and
// is mapped through the sequence's page-table row.
#pragma once

#include "smla_device.h"

namespace smla {

struct GatherArgs {
  const uint8_t* kv;          // [num_pages, P, 576]
  const int32_t* page_table;  // [B, max_pages]
  const u32* indices;         // [T, K]
  u32 num_rows;               // num_pages * P (< 2^32); a row id >= num_rows marks a slot not read
  u32 kv_bytes;               // num_rows * 576 below 4 GiB - 1 KiB (buffer path), else 0
  int K, P, max_pages, num_pages;
};

// What a slot that is not read stages: a row of zeros (never written), so a
// masked key enters the products as zeros, never as whatever bytes a pool row
// would hold (an e4m3fn NaN times a zero weight is NaN).
static __device__ __align__(64) const uint8_t kZeroRow[kQK] = {};

// Per-token state of the translation pipeline (lives in wave 0).
struct TokenSlots {
  const u32* idx_row;     // indices + t * K
  const int32_t* pt_row;  // page_table + b * max_pages
  u32 L;                  // effective slot count, already clamped to K
};

// The slots of run sp of token t (sequence b; b == B when t is not covered):
// slots [sp * split_tiles * 64, ...) of the token's effective list, at most
// split_tiles tiles of them.  With one run this is the whole list.
template <class Params>
__device__ __forceinline__ void token_run(const Params& p, int t, int sp, int b, TokenSlots& ts) {
  ts.L = 0;
  ts.idx_row = p.indices + (size_t)t * p.K;
  ts.pt_row = p.page_table + (size_t)(b < p.B ? b : 0) * p.max_pages;
  if (b < p.B) {
    u32 len = p.lengths[t];
    len = len < (u32)p.K ? len : (u32)p.K;
    const u32 cap = (u32)p.split_tiles * (u32)kBK;
    const u32 s0 = (u32)sp * cap;
    const u32 rem = len > s0 ? len - s0 : 0u;
    ts.L = rem < cap ? rem : cap;
    if (ts.L) ts.idx_row += s0;
  }
}

// token_run with the token's length word already loaded (len = lengths[t]),
// so a prologue can issue that load together with its other first loads.
template <class Params>
__device__ __forceinline__ void token_run_len(const Params& p, int t, int sp, int b, u32 len, TokenSlots& ts) {
  ts.L = 0;
  ts.idx_row = p.indices + (size_t)t * p.K;
  ts.pt_row = p.page_table + (size_t)(b < p.B ? b : 0) * p.max_pages;
  if (b < p.B) {
    len = len < (u32)p.K ? len : (u32)p.K;
    const u32 cap = (u32)p.split_tiles * (u32)kBK;
    const u32 s0 = (u32)sp * cap;
    const u32 rem = len > s0 ? len - s0 : 0u;
    ts.L = rem < cap ? rem : cap;
    if (ts.L) ts.idx_row += s0;
  }
}

// Load the logical index of slot tile*64 + lane (0 when the slot is not read).
__device__ __forceinline__ u32 slot_index(const TokenSlots& ts, int tile, int lane) {
  u32 j = (u32)tile * kBK + (u32)lane;
  return j < ts.L ? ts.idx_row[j] : 0u;
}

// Physical page of that slot, or -1 when the slot is not read or its logical
// page lies outside the page-table row.
__device__ __forceinline__ int slot_page(const TokenSlots& ts, const GatherArgs& ga, int tile, int lane, u32 idx) {
  u32 j = (u32)tile * kBK + (u32)lane;
  u32 page = idx / (u32)ga.P;
  bool ok = j < ts.L && page < (u32)ga.max_pages;
  return ok ? ts.pt_row[page] : -1;
}

// slot_page with the page-table load issued unconditionally, from a page
// clamped into the row, and the result selected afterwards.  A load under a
// divergent branch makes the compiler wait for every outstanding load where
// the branch ends, which serialises the prologue's page loads behind each
// other and behind the q loads.  Used by the blockwise kernel's prologue
// (measured faster there); the FP8 kernels keep slot_page, whose register
// allocation of the tile loop this change disturbed.
__device__ __forceinline__ int slot_page_unbranched(const TokenSlots& ts, const GatherArgs& ga, int tile, int lane,
                                                    u32 idx) {
  const u32 j = (u32)tile * kBK + (u32)lane;
  const u32 page = idx / (u32)ga.P;
  const bool in_row = page < (u32)ga.max_pages;
  const int v = ts.pt_row[in_row ? page : 0u];
  return j < ts.L && in_row ? v : -1;
}

// Physical row of the slot inside the pool; num_rows (its scales and its
// bytes read as zeros) when the slot is not read.
__device__ __forceinline__ u32 slot_row(const GatherArgs& ga, u32 idx, int pg, bool* ok_out) {
  bool ok = pg >= 0 && pg < ga.num_pages;
  *ok_out = ok;
  return ok ? (u32)pg * (u32)ga.P + idx % (u32)ga.P : ga.num_rows;
}

// Write one tile's physical rows and its 64-bit validity mask to LDS (wave 0).
__device__ __forceinline__ void publish_slots(const GatherArgs& ga, u32 idx, int pg, u32* rowid_lds,
                                              u32* mask_lds, int lane) {
  bool ok;
  u32 row = slot_row(ga, idx, pg, &ok);
  unsigned long long m = __ballot(ok);
  rowid_lds[lane] = row;
  if (lane == 0) {
    mask_lds[0] = (u32)m;
    mask_lds[1] = (u32)(m >> 32);
  }
}

// Translate slots [tile0 * 64, tile0 * 64 + ntiles * 64) of a token with the
// whole workgroup (NW waves): rowid_lds[64 * i + lane] and mask_lds[2 * i ..]
// describe tile tile0 + i.  Each wave takes every NW-th tile; the two
// dependent loads (index, then page) of all its tiles are issued before any is
// consumed.
template <int NW, int MAXT>
__device__ __forceinline__ void translate_chunk(const TokenSlots& ts, const GatherArgs& ga, int tile0, int ntiles,
                                                u32* rowid_lds, u32* mask_lds, int wave, int lane) {
  constexpr int PER = (MAXT + NW - 1) / NW;  // tiles per wave
  constexpr int BATCH = PER < 8 ? PER : 8;   // loads in flight per batch
  for (int r0 = 0; r0 < PER; r0 += BATCH) {
    u32 ix[BATCH];
    int pg[BATCH];
#pragma unroll
    for (int r = 0; r < BATCH; ++r) {
      const int i = wave + (r0 + r) * NW;
      ix[r] = i < ntiles ? slot_index(ts, tile0 + i, lane) : 0u;
    }
#pragma unroll
    for (int r = 0; r < BATCH; ++r) {
      const int i = wave + (r0 + r) * NW;
      pg[r] = i < ntiles ? slot_page(ts, ga, tile0 + i, lane, ix[r]) : -1;
    }
#pragma unroll
    for (int r = 0; r < BATCH; ++r) {
      const int i = wave + (r0 + r) * NW;
      if (i < ntiles) publish_slots(ga, ix[r], pg[r], rowid_lds + kBK * i, mask_lds + 2 * i, lane);
    }
  }
}

// Gather one 64-row tile into `tile_lds` (36864 bytes) with four waves.  Wave
// w stages row group w (rows 16 w .. 16 w + 15): copy ch fills block 4 ch + w,
// lane i fetching row 16 w + i / 4, granule 4 ch + ((i % 4) ^ h(i / 4)), so
// each lane needs a single row.  gather_lane_src() is that lane's source of
// copy 0, gather_chunk() issues copy ch (64 bytes further per chunk).
//
// Two ways to name the source.  WIDE: a 64-bit address, so the pool may be
// of any size (a slot not read copies kZeroRow).  Otherwise a 32-bit byte
// offset through a raw buffer descriptor over the pool, for pools below
// 4 GiB - 1 KiB (a slot not read gets an offset past the pool, which reads as
// zeros): one register instead of two in the kernels that keep it live
// across a tile, which their register allocation needs.
template <bool WIDE> struct RowSrcT { using type = u32; };
template <> struct RowSrcT<true> { using type = uint64_t; };
template <bool WIDE> using RowSrc = typename RowSrcT<WIDE>::type;

template <bool WIDE>
__device__ __forceinline__ RowSrc<WIDE> gather_lane_src(const GatherArgs& ga, const u32* rowid_lds, int wave,
                                                        int lane) {
  const u32 l = (u32)lane;
  const u32 q = l >> 2;
  const u32 row = rowid_lds[16u * (u32)wave + q];
  const u32 g = 16u * ((l & 3u) ^ tile_h(q));
  if constexpr (WIDE) {
    const uint8_t* src = row < ga.num_rows ? ga.kv + (uint64_t)row * (uint64_t)kQK : kZeroRow;
    return reinterpret_cast<uint64_t>(src) + g;
  } else {
    return (row < ga.num_rows ? row * (u32)kQK : ga.kv_bytes) + g;
  }
}

// Source of a copy that stages nothing anyone reads (zeros).
template <bool WIDE>
__device__ __forceinline__ RowSrc<WIDE> gather_no_src() {
  if constexpr (WIDE) return reinterpret_cast<uint64_t>(kZeroRow);
  else return 0xFFFFFC00u;  // at or past any pool the buffer path accepts
}

// Copy ch of a lane's row into the tile at LDS byte address tile_lds_addr
// (wave-uniform).  kv_rsrc: raw descriptor over the pool (buffer path only).
template <bool WIDE>
__device__ __forceinline__ void gather_chunk_at(v4i kv_rsrc, u32 tile_lds_addr, int wave, RowSrc<WIDE> src, int ch) {
  const u32 lds = __builtin_amdgcn_readfirstlane(tile_lds_addr + 1024u * (4u * (u32)ch + (u32)wave));
  if constexpr (WIDE) load_global_to_lds_at(lds, src + 64u * (u32)ch);
  else load_to_lds_at<16>(kv_rsrc, lds, src + 64u * (u32)ch);
}

template <int NW, bool WIDE>
__device__ __forceinline__ void gather_tile(v4i kv_rsrc, const GatherArgs& ga, const u32* rowid_lds, uint8_t* tile_lds,
                                            int wave, int lane) {
  static_assert(NW == 4, "one row group per wave");
  const RowSrc<WIDE> src = gather_lane_src<WIDE>(ga, rowid_lds, wave, lane);
  const u32 base = lds_addr_of(tile_lds);
#pragma unroll
  for (int ch = 0; ch < kRowGranules / 4; ++ch) gather_chunk_at<WIDE>(kv_rsrc, base, wave, src, ch);
}

}  // namespace smla

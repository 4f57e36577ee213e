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
  u32 kv_bytes;               // num_pages * P * 576 (< 2^32 - 1024)
  int K, P, max_pages, num_pages;
};

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

// Byte offset of the slot's row inside the pool; kv_bytes (out of range, so
// buffer loads return zeros) when the slot is not read.
__device__ __forceinline__ u32 slot_row_offset(const GatherArgs& ga, u32 idx, int pg, bool* ok_out) {
  bool ok = pg >= 0 && pg < ga.num_pages;
  *ok_out = ok;
  return ok ? ((u32)pg * (u32)ga.P + idx % (u32)ga.P) * (u32)kQK : ga.kv_bytes;
}

// Write one tile's row offsets and its 64-bit validity mask to LDS (wave 0).
__device__ __forceinline__ void publish_slots(const GatherArgs& ga, u32 idx, int pg, u32* rowoff_lds,
                                              u32* mask_lds, int lane) {
  bool ok;
  u32 off = slot_row_offset(ga, idx, pg, &ok);
  unsigned long long m = __ballot(ok);
  rowoff_lds[lane] = off;
  if (lane == 0) {
    mask_lds[0] = (u32)m;
    mask_lds[1] = (u32)(m >> 32);
  }
}

// Translate slots [tile0 * 64, tile0 * 64 + ntiles * 64) of a token with the
// whole workgroup (NW waves): rowoff_lds[64 * i + lane] and mask_lds[2 * i ..]
// describe tile tile0 + i.  Each wave takes every NW-th tile; the two
// dependent loads (index, then page) of all its tiles are issued before any is
// consumed.
template <int NW, int MAXT>
__device__ __forceinline__ void translate_chunk(const TokenSlots& ts, const GatherArgs& ga, int tile0, int ntiles,
                                                u32* rowoff_lds, u32* mask_lds, int wave, int lane) {
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
      if (i < ntiles) publish_slots(ga, ix[r], pg[r], rowoff_lds + kBK * i, mask_lds + 2 * i, lane);
    }
  }
}

// Gather one 64-row tile into `tile_lds` (36864 bytes) with four waves.  Wave
// w stages row group w (rows 16 w .. 16 w + 15): copy ch fills block 4 ch + w,
// lane i fetching row 16 w + i / 4, granule 4 ch + ((i % 4) ^ h(i / 4)), so
// each lane needs the offset of a single row.  gather_lane_offset() is that
// lane's source offset of copy 0, gather_chunk() issues copy ch.
__device__ __forceinline__ u32 gather_lane_offset(const u32* rowoff_lds, int wave, int lane) {
  const u32 l = (u32)lane;
  const u32 q = l >> 2;
  return rowoff_lds[16u * (u32)wave + q] + 16u * ((l & 3u) ^ tile_h(q));
}

__device__ __forceinline__ void gather_chunk(v4i kv_rsrc, uint8_t* tile_lds, int wave, u32 ro, int ch) {
  load_to_lds<16>(kv_rsrc, (SMLA_LDS void*)(tile_lds + 1024u * (4u * (u32)ch + (u32)wave)), ro + 64u * (u32)ch);
}

// gather_chunk with the tile's LDS byte address given wave-uniform.
__device__ __forceinline__ void gather_chunk_at(v4i kv_rsrc, u32 tile_lds_addr, int wave, u32 ro, int ch) {
  load_to_lds_at<16>(kv_rsrc, tile_lds_addr + 1024u * (4u * (u32)ch + (u32)wave), ro + 64u * (u32)ch);
}

template <int NW>
__device__ __forceinline__ void gather_tile(v4i kv_rsrc, const u32* rowoff_lds, uint8_t* tile_lds, int wave, int lane) {
  static_assert(NW == 4, "one row group per wave");
  const u32 ro = gather_lane_offset(rowoff_lds, wave, lane);
#pragma unroll
  for (int ch = 0; ch < kRowGranules / 4; ++ch) gather_chunk(kv_rsrc, tile_lds, wave, ro, ch);
}

}  // namespace smla

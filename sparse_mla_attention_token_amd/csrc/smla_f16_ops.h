// FP16 building blocks of the blockwise-scale kernels: the dequantised FP16
// tile layout in LDS, its transposed reads, and the per-tile dequantisation of
// a staged FP8 tile with its block scales.
//
// Blockwise scales (page "mla_sm100_prefill_sparse_fp8", Parameters:
// scale_block_size, and the scales_ptr argument) give every physical row one
// f32 per scale_block_size columns: k[c] = fp8(kv[row, c]) * scales[row, c /
// sbs], and V uses the first 512 columns of the same dequantised row.
#pragma once

#include "smla_device.h"

namespace smla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kMaxScaleCols = 36;          // ceil(576 / 16): smallest block size is 16
constexpr int kHTileBytes = kBK * kQK * 2;  // 73728: one dequantised FP16 tile

// FP16 tile: row r (key), 8-column granule G (16 bytes) at
//   G * 1024 + 16 * (r ^ 12 (G & 1)).
// Reads of 16 or 32 consecutive rows of one granule (K operands) and the
// transposed V reads (4 rows x 2 adjacent granules per 16 lanes, the odd
// granule's rows XORed with 12) are free of bank conflicts for 32 and 64
// banks: each 16-lane group covers two distinct 64-byte segments of a 128-byte
// window, two groups four distinct segments of a 256-byte window.
__device__ __forceinline__ u32 ht_swz(u32 G) { return 12u * (G & 1u); }
__device__ __forceinline__ u32 ht_off(u32 r, u32 G) { return G * 1024u + 16u * (r ^ ht_swz(G)); }

// Transposed 16-bit read: within each 16-lane group, lane 4k + c supplies
// the address of 4 consecutive halves (row k of a 4 x 16 block, columns
// 4c .. 4c + 3); lane j receives column j of the block, element k from row k.
__device__ __forceinline__ s16x4 lds_read_tr16(const SMLA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS s16x4*)p);
}

// Largest of 64 non-negative floats, one per lane, returned to every lane:
// DPP steps inside each 16-lane row (quad swaps, then the half-row and row
// mirrors), then the four row results through scalar registers.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = dpp_max<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_max<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_max<0x141>(x);  // row_half_mirror
  x = dpp_max<0x140>(x);  // row_mirror
  const u32 a = (u32)__builtin_amdgcn_readlane(__float_as_int(x), 0);
  const u32 b = (u32)__builtin_amdgcn_readlane(__float_as_int(x), 16);
  const u32 c = (u32)__builtin_amdgcn_readlane(__float_as_int(x), 32);
  const u32 d = (u32)__builtin_amdgcn_readlane(__float_as_int(x), 48);
  // non-negative floats order like their bit patterns
  return __uint_as_float(max(max(a, b), max(c, d)));
}

// two f32 -> two fp16 (round to nearest even) in one dword
__device__ __forceinline__ u32 pack_h2(float a, float b) {
  return __builtin_bit_cast(u32, __builtin_convertvector((v2f){a, b}, f16x2));
}

// Stage the block scales of a tile's 64 rows next to the rows, one padded row
// per slot: copy k fills ssc[64 k .. 64 k + 63], lane i the float 64 k + i =
// slot s, column c (x / pitch = x * magic >> 20 for x < 64 pitch).  Rows that
// are not read and the padding fetch zeros.  NW waves share the pitch copies.
template <int NW>
__device__ __forceinline__ void stage_block_scales(v4i sc_rsrc, const u32* rowid, float* ssc, int pitch, u32 pitch_magic,
                                                   int ncols, u32 num_rows, u32 scale_bytes, int wave, int lane) {
  for (int k = wave; k < pitch; k += NW) {
    const u32 i = 64u * (u32)k + (u32)lane;
    const u32 s = (i * pitch_magic) >> 20, c = i - s * (u32)pitch;
    const u32 row = rowid[s];
    const bool ok = row < num_rows && c < (u32)ncols;
    const u32 soff = ok ? (row * (u32)ncols + c) * 4u : scale_bytes;
    load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&ssc[64 * k], soff);
  }
}

// Tile factor 2^ek: 448 (largest |e4m3fn|) times the largest block scale of
// the tile's 64 staged rows lands in [128, 256).  Every wave reduces the whole
// table itself (no barrier needed): lane s takes the maximum of its slot's
// row (16 bytes per read, five reads per step so they are in flight
// together), then the wave reduces the 64 row maxima.
__device__ __forceinline__ int tile_exponent(const float* ssc, int pitch, int lane) {
  float smax = 0.f;
  const int nv = pitch >> 2;
  const SMLA_LDS float* myrow = (const SMLA_LDS float*)&ssc[lane * pitch];
  for (int m0 = 0; m0 < nv; m0 += 5) {
    v4f v[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) v[k] = *(const SMLA_LDS v4f*)(myrow + 4 * (m0 + k < nv ? m0 + k : nv - 1));
    __builtin_amdgcn_sched_barrier(0);  // all five reads before any use
#pragma unroll
    for (int k = 0; k < 5; ++k) smax = fmaxf(smax, fmaxf(fmaxf(v[k][0], v[k][1]), fmaxf(v[k][2], v[k][3])));
  }
  smax = wave_max_nonneg(smax);
  int ek = fit_exponent(448.0f * smax);
  return ek < -100 ? -100 : (ek > 100 ? 100 : ek);
}

// Dequantise the staged FP8 tile s8 into the FP16 tile kt: lane = row slot,
// FP8 granules wave + NW rep (16 columns each -> FP16 granules 2 gl and
// 2 gl + 1), element = fp16(fp8 * fp16(scale * 2^ek)): the FP8 code widened
// to fp16 exactly (the conversion's scale operand applies only its exponent,
// so 1 keeps the code as it is), one rounding in the packed fp16 multiply.
// All the lane's bytes and scales are read before any is converted, so the
// LDS latencies overlap.  scol[rep]: scale column of granule wave + NW rep.
template <int NW>
__device__ __forceinline__ void dequant_tile(const uint8_t* s8, uint8_t* kt, const float* ssc, int pitch,
                                             const int* scol, int ek, int wave, int lane) {
  constexpr int REPS = kRowGranules / NW;
  const SMLA_LDS float* srow = (const SMLA_LDS float*)&ssc[lane * pitch];
  v4i raw[REPS];
  float sc[REPS];
#pragma unroll
  for (int rep = 0; rep < REPS; ++rep) {
    raw[rep] = lds_read_b128((const SMLA_LDS uint8_t*)s8 + tile_off((u32)lane, (u32)(wave + NW * rep)));
    sc[rep] = srow[scol[rep]];
  }
#pragma unroll
  for (int rep = 0; rep < REPS; ++rep) {
    const u32 gl = (u32)(wave + NW * rep);
    const _Float16 sh = (_Float16)__builtin_amdgcn_ldexpf(sc[rep], ek);
    const f16x2 s2 = {sh, sh};
    u32 w[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[rep][d], 1.0f, false) * s2;
      const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[rep][d], 1.0f, true) * s2;
      w[2 * d] = __builtin_bit_cast(u32, lo);
      w[2 * d + 1] = __builtin_bit_cast(u32, hi);
    }
    *(SMLA_LDS v4i*)(kt + ht_off((u32)lane, 2u * gl)) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    *(SMLA_LDS v4i*)(kt + ht_off((u32)lane, 2u * gl + 1u)) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
  }
}

}  // namespace smla

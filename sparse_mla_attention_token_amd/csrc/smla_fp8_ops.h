// Operand reads of a staged 64-row KV tile for the FP8 MFMA kernels
// (32x32x64 f8f6f4 fragments: a lane holds row / column l % 32 and the
// contraction bytes 16 g .. 16 g + 15 and 32 + 16 g .. of its half g).
#pragma once

#include "smla_device.h"

namespace smla {

// Lane-dependent base offsets of the operand reads inside a staged tile
// (closed forms of offset(r, G) for the rows and granules each lane reads).
//   K operand, contraction step ks, M-block mb, granule half u:
//     row 32 mb + hl, granule 4 ks + 2 g + u   ->  kbase(u) + 4096 ks + 2048 mb
//   V^T operand, output block nb, transposed read q:
//     lane 2k + c of 16-lane group (g, half) points at row
//       key(g, 8q + k) = 16 q + 8 (k / 4) + 4 g + k % 4,
//     granule 2 nb + half, byte 8c  ->  vbase(nb % 2) + 4096 (nb / 2) + 1024 q
__device__ __forceinline__ u32 k_base(int lane, int u) {
  const u32 hl = (u32)lane & 31u, g = (u32)lane >> 5;
  const u32 q = hl & 15u;
  return 1024u * (hl >> 4) + 64u * q + 16u * ((2u * g + (u32)u) ^ tile_h(q));
}

__device__ __forceinline__ u32 v_base(int lane, int par) {
  const u32 i = (u32)lane & 15u, k = i >> 1, c = i & 1u, g = (u32)lane >> 5, half = ((u32)lane >> 4) & 1u;
  const u32 q = 8u * (k >> 2) + 4u * g + (k & 3u);
  return 64u * q + 16u * ((2u * (u32)par + half) ^ tile_h(q)) + 8u * c;
}

__device__ __forceinline__ v8i read_k(const SMLA_LDS uint8_t* tb, u32 kb0, u32 kb1, int ks, int mb) {
  const u32 o = 4096u * (u32)ks + 2048u * (u32)mb;
  v4i a0 = lds_read_b128(tb + kb0 + o), a1 = lds_read_b128(tb + kb1 + o);
  return v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
}

__device__ __forceinline__ v8i read_vt(const SMLA_LDS uint8_t* tb, u32 vb, int nb) {
  v8i a;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v2i r = lds_read_tr8(tb + vb + 4096u * (u32)(nb >> 1) + 1024u * (u32)q);
    a[2 * q] = r[0];
    a[2 * q + 1] = r[1];
  }
  return a;
}


}  // namespace smla

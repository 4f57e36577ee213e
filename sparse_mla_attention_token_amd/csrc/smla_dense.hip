// Dense MLA prefill attention on gfx950 BF16 MFMA, with a block-scaled FP8
// K_rope.
//
// What is computed: the attention of the page "mla_sm100_prefill_blockscale"
// (function description, Parameters and Args), with the 64-wide rope part of
// K of the "SM100MLA" page (comptime members).  For query row i of sequence b
// and head h (kv head hk = h / group):
//   k_j = [K_nope[j, hk, 0:128], fp8(K_rope[j, 0:64]) * sigma(j, c)]
//   out[i, h, :] = sum_{j visible} softmax_j(scale * q[i, h, :] . k_j) V[j, hk, :]
// with the keys j = 0 .. L_b - 1 of the sequence (L_b = min(valid_length[b],
// max_prompt_len)), visible when j <= i under the causal mask, read through
// one page table shared by the three paged caches.  As the page describes,
// the FP8 K_rope is turned into BF16 (times its block scale, rounded to
// nearest even) before the products, which run on v_mfma_f32_16x16x32_bf16
// with f32 accumulation; P is rounded to BF16 for the P.V product.
//
// Work decomposition: one workgroup per (sequence, head, block of 256 query
// rows), eight waves of 32 rows (two per SIMD); blocks with the longest
// causal key range are dispatched first.  Each 64-key tile goes through a
// three-stage LDS ring (45 KiB a stage) with the copies two tiles ahead of
// the compute: K_nope, V, the FP8 K_rope bytes and their scales are copied
// straight from global memory into LDS (buffer loads with the LDS flag), and
// the rope is dequantised to BF16 in LDS once the tile has landed.  Page ids
// of pages of 64 rows or more come through the scalar cache, so no vector
// load the compiler tracks waits on the copies in flight.  Per wave and tile:
//   * S^T[64 keys x 32 rows] = K . Q^T (keys on M), q held in registers as
//     the B operand, 48 MFMAs;
//   * online exp2 softmax with a lazy rescale (O moves to a new running max
//     only when a tile exceeds it by more than 2^8);
//   * O^T[128 columns x 32 rows] += V^T . P^T, V^T read from the tile with
//     ds_read_b64_tr_b16, 32 MFMAs.
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
#define SMLA_CONST __attribute__((address_space(4)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kDn = 128;                 // K_nope width
constexpr int kDr = 64;                  // K_rope width
constexpr int kDq = kDn + kDr;           // 192
constexpr int kDv = 128;                 // V / output width
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWG = 32 * kWaves;     // query rows per workgroup: 256
constexpr int kNS = 3;                   // LDS stages; copies run two tiles ahead
constexpr u32 kKBytes = (kDq / 8) * 1024u;   // 24 granule columns of 64 keys (bf16)
constexpr u32 kVBytes = (kDv / 8) * 1024u;   // 16
constexpr u32 kRawOff = kKBytes + kVBytes;   // fp8 rope bytes, [key][64]
constexpr u32 kScOff = kRawOff + 64u * kDr;  // rope scales, [column][key] (up to 4 columns)
constexpr u32 kStageBytes = kScOff + 4u * 256u;  // 46080
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazy = 8.0f;            // log2 headroom before O is rescaled
constexpr u32 kNoRow = 0x80000000u;      // offset past every buffer: reads zeros

// BF16 tile: key r, 8-column granule G (16 bytes) at G * 1024 + 16 (r ^ 12 (G & 1)).
// One granule column (64 keys) is 1024 contiguous bytes, the destination of
// one wave-wide copy; the K operand reads (16 consecutive keys, one granule
// per 16-lane group) and the transposed V reads are free of bank conflicts.
__device__ __forceinline__ u32 tile_at(u32 r, u32 G) { return G * 1024u + 16u * (r ^ (12u * (G & 1u))); }

__device__ __forceinline__ v4f mfma_bf16(bf16x8 a, bf16x8 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// K operand, key block mb (keys 16 mb + r), contraction step ks (granule
// 4 ks + g), r = lane % 16, g = lane / 16  ->  kbase + 4096 ks + 256 mb.
__device__ __forceinline__ u32 k_base(int lane) {
  const u32 r = (u32)lane & 15u, g = (u32)lane >> 4;
  return g * 1024u + 16u * (r ^ (12u * (g & 1u)));
}

__device__ __forceinline__ bf16x8 read_k(const SMLA_LDS uint8_t* tb, u32 kb, int ks, int mb) {
  return __builtin_bit_cast(bf16x8, lds_read_b128(tb + kb + 4096u * (u32)ks + 256u * (u32)mb));
}

// Transposed 16-bit read: within each 16-lane group, lane 4k + c supplies the
// address of 4 consecutive halves (row k of a 4 x 16 block, columns
// 4c .. 4c + 3); lane j receives column j of the block, element k from row k.
__device__ __forceinline__ s16x4 lds_read_tr16(const SMLA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS s16x4*)p);
}

// V^T operand for output block nb (columns 16 nb .. +15) and key block kb:
// MFMA slot s of lane (n, g) holds key 32 kb + 16 (s / 4) + 4 g + s % 4, the
// order of the P^T operand assembled from the S^T accumulators.  Half hh
// (slots 4 hh .. 4 hh + 3): lane 4k + c of group g points at key
// 32 kb + 16 hh + 4 g + k, columns 16 nb + 4 c .. +3.
__device__ __forceinline__ u32 v_base(int lane) {
  const u32 i = (u32)lane & 15u, k = i >> 2, c = i & 3u, g = (u32)lane >> 4;
  const u32 key = 4u * g + k;
  const u32 G = c >> 1;
  return G * 1024u + 16u * (key ^ (12u * G)) + 8u * (c & 1u);
}

__device__ __forceinline__ bf16x8 read_vt(const SMLA_LDS uint8_t* tb, u32 vb, int nb, int kb) {
  const u32 o = 2048u * (u32)nb + 512u * (u32)kb;
  const s16x4 a = lds_read_tr16(tb + vb + o), b = lds_read_tr16(tb + vb + o + 256u);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}


// x of lane i ^ m through the LDS crossbar.  The lane-swap form of the other
// kernels (v_permlane16/32_swap) measured 5% slower here, so this kernel keeps
// ds_bpermute.
__device__ __forceinline__ float bperm_xor(float x, u32 m) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ m) << 2), __float_as_int(x)));
}

// reductions over the four lanes holding one query row (n, n+16, n+32, n+48)
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, bperm_xor(x, 16u));
  return fmaxf(x, bperm_xor(x, 32u));
}
__device__ __forceinline__ float row_sum(float x) {
  x += bperm_xor(x, 16u);
  return x + bperm_xor(x, 32u);
}

__global__ __launch_bounds__(kThreads, 1) void smla_dense_kernel(DenseParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[kNS][kStageBytes];

  const int lane = (int)(threadIdx.x & 63u);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g = lane >> 4, n = lane & 15;

  // ---- work item: blocks of the longest causal range first
  const int total = p.B * p.H * p.row_blocks;
  const int wid = xcd_token((int)blockIdx.x, total);
  const int rbi = wid % p.row_blocks;
  const int bh = wid / p.row_blocks;
  const int h = bh % p.H, b = bh / p.H;
  const int rb = p.row_blocks - 1 - rbi;
  const int hk = h / (p.H / p.Hkv);
  const int vl = (int)(p.valid_length[b] < (uint32_t)p.S ? p.valid_length[b] : (uint32_t)p.S);
  const int L = __builtin_amdgcn_readfirstlane(vl);
  const int q0 = rb * kRowsWG;
  const int i0w = q0 + 32 * wave;          // first row of this wave

  const size_t out_row0 = (size_t)b * (size_t)p.S;
  if (q0 >= L) {
    // padding rows only: zeros
    for (int r = (int)(threadIdx.x >> 4); r < kRowsWG; r += kThreads / 16) {
      const int i = q0 + r;
      if (i >= p.S) break;
      uint16_t* orow = p.out + ((out_row0 + (size_t)i) * (size_t)p.H + (size_t)h) * kDv + 8 * (threadIdx.x & 15u);
      *(v4i*)orow = v4i{0, 0, 0, 0};
    }
    return;
  }
  const int kend = p.causal ? (q0 + kRowsWG < L ? q0 + kRowsWG : L) : L;
  const int ntiles = (kend + 63) / 64;

  const v4i kn_rsrc = make_rsrc(p.k_nope, p.kn_bytes);
  const v4i v_rsrc = make_rsrc(p.v, p.v_bytes);
  const v4i kr_rsrc = make_rsrc(p.k_rope, p.kr_bytes);
  const v4i sc_rsrc = make_rsrc(p.rope_scales, p.sc_bytes);
  const u32 lds0 = lds_addr_of(tiles);
  const int32_t* ptab = p.page_table + (size_t)b * (size_t)p.max_pages;
  // the same table through the scalar cache (read-only here): uniform page ids
  const SMLA_CONST int32_t* ptab_s = (const SMLA_CONST int32_t*)ptab;
  const bool wide_pages = p.P >= 64;      // a tile spans at most two pages

  // ---- copies of tile t into stage st, all global->LDS: the rope bytes and
  // their scales first, then the K_nope / V granule columns (the last four
  // copies of every wave), so that "at most 4 in flight" means everything but
  // the K_nope / V columns of the newest tile has landed.
  auto issue = [&](int t, int st) -> unsigned long long {
    const int k0 = 64 * t;
    int ra, rx;
    {
      const int j = k0 + lane, jx = k0 + (lane ^ 12);
      if (wide_pages) {
        const int pi0 = p.P_log2 >= 0 ? (k0 >> p.P_log2) : k0 / p.P;
        const int pg0 = ptab_s[pi0];
        const int pg1 = ptab_s[pi0 + 1 < p.max_pages ? pi0 + 1 : pi0];
        // page size a power of two (the usual case): shifts instead of divisions
        const int qa = p.P_log2 >= 0 ? (j >> p.P_log2) : j / p.P;
        const int qx = p.P_log2 >= 0 ? (jx >> p.P_log2) : jx / p.P;
        const int pa = qa == pi0 ? pg0 : pg1, px = qx == pi0 ? pg0 : pg1;
        ra = (j < L && pa >= 0 && pa < p.num_pages) ? pa * p.P + (j - qa * p.P) : -1;
        rx = (jx < L && px >= 0 && px < p.num_pages) ? px * p.P + (jx - qx * p.P) : -1;
      } else {
        auto row_of = [&](int jj) -> int {
          if (jj >= L) return -1;
          const int pg = ptab[jj / p.P];
          if (pg < 0 || pg >= p.num_pages) return -1;
          return pg * p.P + jj % p.P;
        };
        ra = row_of(j);
        rx = row_of(jx);
      }
    }
    const u32 sbase = lds0 + (u32)st * kStageBytes;
    if (wave < 4) {
      // rope bytes: copy `wave` takes keys 16 wave .. +15, lane -> (key 16 wave + lane / 4,
      // 16-byte quarter lane % 4); the key's row was found by lane 16 wave + lane / 4
      const int rr = __builtin_amdgcn_ds_bpermute((16 * wave + (lane >> 2)) << 2, ra);
      const u32 off = rr < 0 ? kNoRow : (u32)rr * (u32)kDr + 16u * (u32)(lane & 3);
      load_to_lds_at<16>(kr_rsrc, sbase + kRawOff + 1024u * (u32)wave, off);
    } else if (wave - 4 < p.scale_cols) {
      // scale column wave - 4 of the 64 keys, one dword per lane
      const u32 col = (u32)(wave - 4);
      const u32 off = ra < 0 ? kNoRow : ((u32)ra * (u32)p.scale_cols + col) * 4u;
      load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&tiles[st][kScOff + 256u * col], off);
    }
    const u32 hkb = (u32)hk * (u32)(kDn * 2);
    const u32 oa = ra < 0 ? kNoRow : (u32)ra * (u32)p.Hkv * (u32)(kDn * 2) + hkb;
    const u32 ox = rx < 0 ? kNoRow : (u32)rx * (u32)p.Hkv * (u32)(kDn * 2) + hkb;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const u32 G = 2u * (u32)wave + (u32)gi;
      const u32 off = ((G & 1u) ? ox : oa) + 16u * G;
      load_to_lds_at<16>(kn_rsrc, sbase + G * 1024u, off);
      load_to_lds_at<16>(v_rsrc, sbase + kKBytes + G * 1024u, off);
    }
    return __ballot(ra >= 0);
  };
  // rope of the tile in stage st: fp8 x block scale -> bf16 granules 16 .. 23
  // (threads 0 .. 255: key tid / 4, columns 16 (tid % 4) .. +15)
  auto convert_rope = [&](int st) {
    if (threadIdx.x >= 256u) return;
    uint8_t* kt = &tiles[st][0];
    const u32 r = threadIdx.x >> 2, c = threadIdx.x & 3u;
    const v4i raw = *(const SMLA_LDS v4i*)(kt + kRawOff + 64u * r + 16u * c);
    float sc = 1.0f;
    if (p.sbs != 0) {
      const u32 col = p.sbs >= kDr ? 0u : (16u * c) / (u32)p.sbs;
      sc = *(const SMLA_LDS float*)(kt + kScOff + 256u * col + 4u * r);
    }
    u32 w[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const v2f lo = fp8x2_to_f32<false>(raw[d]), hi = fp8x2_to_f32<true>(raw[d]);
      w[2 * d] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
      w[2 * d + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
    }
    const u32 G = 16u + 2u * c;
    *(SMLA_LDS v4i*)(kt + tile_at(r, G)) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    *(SMLA_LDS v4i*)(kt + tile_at(r, G + 1u)) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
  };

  unsigned long long vm0 = issue(0, 0), vm1 = 0, vm2 = 0;
  if (ntiles > 1) vm1 = issue(1, 1);

  // ---- q rows of this wave as the B operand: row i0w + 16 nb + n, depth
  // granule 4 ks + g
  bf16x8 qreg[2][6];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int i = i0w + 16 * nb + n;
    const uint16_t* qrow = p.q + ((out_row0 + (size_t)(i < p.S ? i : 0)) * (size_t)p.H + (size_t)h) * kDq + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      v4i v = i < p.S ? *(const v4i*)(qrow + 32 * ks) : v4i{0, 0, 0, 0};
      qreg[nb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  wait_vmem_all();
  __syncthreads();
  convert_rope(0);
  __syncthreads();

  float m_run[2] = {kNegInf, kNegInf}, l_part[2] = {0.f, 0.f};
  v4f o[8][2];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) o[c][nb] = v4f{0.f, 0.f, 0.f, 0.f};
  const float c2 = p.scale_log2;
  const u32 kb = k_base(lane);

  int st = 0;
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = 64 * t;
    const int st1 = st == kNS - 1 ? 0 : st + 1, st2 = st1 == kNS - 1 ? 0 : st1 + 1;
    if (t + 2 < ntiles) vm2 = issue(t + 2, st2);

    // a wave whose rows all precede the tile's first key has nothing to add
    if (!p.causal || k0 <= i0w + 31) {
      const SMLA_LDS uint8_t* tb = (const SMLA_LDS uint8_t*)&tiles[st][0];
      // (1) S^T = K . Q^T
      v4f s[2][4];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) s[nb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
      bf16x8 kr[2][4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) kr[0][mb] = read_k(tb, kb, 0, mb);
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        if (ks + 1 < 6) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) kr[(ks + 1) & 1][mb] = read_k(tb, kb, ks + 1, mb);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          s[0][mb] = mfma_bf16(kr[ks & 1][mb], qreg[0][ks], s[0][mb]);
          s[1][mb] = mfma_bf16(kr[ks & 1][mb], qreg[1][ks], s[1][mb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // (2) online softmax.  Lane (row n, quarter g) holds in register ii of
      // block mb the score of key k0 + 16 mb + 4 g + ii for row i0w + 16 nb + n.
      const bool masked = (vm0 != ~0ull) || (p.causal && k0 + 63 > i0w);  // wave-uniform
      bf16x8 pv[2][2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int i = i0w + 16 * nb + n;
        float tmax = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int jj = 16 * mb + 4 * g + ii;
            float x = s[nb][mb][ii];
            if (masked) {
              const bool vis = ((vm0 >> jj) & 1ull) && (!p.causal || k0 + jj <= i);
              x = vis ? x : kNegInf;
            }
            s[nb][mb][ii] = x;
            tmax = fmaxf(tmax, x);
          }
        tmax = row_max(tmax) * c2;
        const bool upd = tmax > m_run[nb] + kLazy;
        if (__any(upd)) {
          const float m_new = upd ? tmax : m_run[nb];
          const float alpha = upd ? __builtin_amdgcn_exp2f(m_run[nb] - m_new) : 1.0f;
          m_run[nb] = m_new;
          l_part[nb] *= alpha;
#pragma unroll
          for (int c = 0; c < 8; ++c) o[c][nb] *= alpha;
        }
        const float msub = m_run[nb] == kNegInf ? 0.f : m_run[nb];
        float lsum = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          u32 w[4];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int mb = 2 * kb2 + hh;
            float y[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              y[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][mb][ii], c2, -msub));
              lsum += y[ii];
            }
            w[2 * hh] = pack_bf16x2(y[0], y[1]);
            w[2 * hh + 1] = pack_bf16x2(y[2], y[3]);
          }
          pv[nb][kb2] = __builtin_bit_cast(bf16x8, v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
        }
        l_part[nb] += lsum;
      }

      // (3) O^T += V^T . P^T; the empty asm keeps the transposed reads below
      // the softmax
      const SMLA_LDS uint8_t* vt = tb + kKBytes;
      u32 vb = v_base(lane);
      asm volatile("" : "+v"(vb) : "v"(pv[0][0]), "v"(pv[0][1]), "v"(pv[1][0]), "v"(pv[1][1]));
      bf16x8 va[2][2];
      va[0][0] = read_vt(vt, vb, 0, 0);
      va[0][1] = read_vt(vt, vb, 0, 1);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c + 1 < 8) {
          va[(c + 1) & 1][0] = read_vt(vt, vb, c + 1, 0);
          va[(c + 1) & 1][1] = read_vt(vt, vb, c + 1, 1);
        }
        o[c][0] = mfma_bf16(va[c & 1][0], pv[0][0], o[c][0]);
        o[c][1] = mfma_bf16(va[c & 1][0], pv[1][0], o[c][1]);
        o[c][0] = mfma_bf16(va[c & 1][1], pv[0][1], o[c][0]);
        o[c][1] = mfma_bf16(va[c & 1][1], pv[1][1], o[c][1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // (4) tile t + 1 has landed (only the K_nope / V copies of tile t + 2 may
    // still be in flight) and every wave is done with stage st; then its rope
    // is dequantised, and the next tile may start once that is visible
    if (t + 1 < ntiles) {
      if (t + 2 < ntiles) wait_vmem_le<4>();
      else wait_vmem_all();
      __syncthreads();
      convert_rope(st1);
      __syncthreads();
    }
    vm0 = vm1;
    vm1 = vm2;
    st = st1;
  }

  // ---- epilogue: O / l to bf16; rows past the length are zeros
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l_tot = row_sum(l_part[nb]);
    const int i = i0w + 16 * nb + n;
    if (i >= p.S) continue;
    const float inv = (i < L && l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    uint16_t* orow = p.out + ((out_row0 + (size_t)i) * (size_t)p.H + (size_t)h) * kDv + 4 * g;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const v2i w = {(int)pack_bf16x2(o[c][nb][0] * inv, o[c][nb][1] * inv),
                     (int)pack_bf16x2(o[c][nb][2] * inv, o[c][nb][3] * inv)};
      *(v2i*)(orow + 16 * c) = w;
    }
  }
}

}  // namespace

hipError_t launch_dense(const DenseParams& params, hipStream_t stream) {
  DenseParams p = params;
  p.row_blocks = (p.S + kRowsWG - 1) / kRowsWG;
  const long long blocks = (long long)p.B * p.H * p.row_blocks;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(smla_dense_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla

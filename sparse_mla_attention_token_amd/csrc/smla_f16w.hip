// Sparse MLA prefill attention on gfx950 FP16 MFMA, blockwise scales, one
// workgroup per query token for up to 128 heads.
//
// What is computed is the attention of the page "mla_sm100_prefill_sparse_fp8"
// (function description, Parameters and Args) with blockwise scales: k_j[c] =
// fp8(kv[row, c]) * scales[row, c / sbs] over the 576 latent columns, v_j the
// first 512 of the same dequantised row (the shared K/V latent of the page
// "mla_prefill_sparse_qkv_fp8"), softmax with an optional per-head sink logit
// in the denominator.
//
// Work decomposition.  One workgroup takes a token and all of its heads, four
// waves of 32 heads, so each 64-row tile is gathered from L2 / HBM once and
// dequantised once for every head of the token (the FP8 path shares its tile
// the same way).  Per tile:
//   * the FP8 rows and their block scales are copied global->LDS one tile
//     ahead of the compute (the gather of the FP8 kernels);
//   * the whole workgroup dequantises the staged tile into an FP16 copy in
//     LDS: fp16(fp8 * fp16(scale * 2^ek)), with a power-of-two tile factor
//     2^ek that puts 448 * (largest block scale of the tile) in [128, 256);
//   * S^T[64 keys x 32 heads] = K . Q^T on v_mfma_f32_32x32x16_f16 (keys on
//     M, q held in registers as fp16 scaled per head by 2^eq), so each K
//     operand read from LDS feeds 32 heads;
//   * online exp2 softmax with a lazy rescale, O kept in units of 2^-E and
//     P formed as exp2(s - m + E - ek) so every tile lands in those units;
//   * O^T[512 x 32 heads] += V^T . P^T on the same MFMA, V^T read from the
//     FP16 tile with ds_read_b64_tr_b16.
// Why FP16 and a dequantised copy rather than folding the scales into FP8
// operands: a block scale varies along the contraction of both products and
// is not a power of two, so it cannot ride on the FP8 MFMA's E8M0 operand
// scales; and converting in registers costs one VALU operation per element
// and wave, as many VALU cycles as the matrix pipe needs for the tile at 32
// heads per wave, where dequantising once per workgroup costs a quarter of
// that.  FP16 keeps fp8 * scale, q and P within 2^-12 relative (BF16's 2^-9
// on K alone doubles the output error).
#include "smla_device.h"
#include "smla_f16_ops.h"
#include "smla_gather.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyRescale = 8.0f;   // log2 headroom before O is rescaled
constexpr int kUnitDrift = 4;          // binades E may trail or lead a tile's ek
constexpr int kChunkTiles = 32;        // 2048 slots translated at a time
constexpr int kWaves = 4;
constexpr int kHeadsPerWave = 32;

// D[32x32] += A[32x16] * B[16x32] in fp16 with f32 accumulation.  Lane l
// holds row (A) / column (B) l % 32 and eight contraction elements of half
// l / 32; D lane l holds column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4.
__device__ __forceinline__ v16f mfma32_f16(f16x8 a, f16x8 b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The same MFMA for the score accumulators, written as an instruction so
// that they stay in VGPRs (the softmax reads them there) while the P.V
// accumulators, 256 values, take the AGPRs.  The wait states the compiler
// would insert around it are covered by hand: consecutive MFMAs on one
// accumulator chain in hardware, and the VALU reads the scores only after
// mfma_fence().
__device__ __forceinline__ void mfma32_f16_v(v16f& acc, f16x8 a, f16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_f16_v0(v16f& acc, f16x8 a, f16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}

// max(a, b, c) in one v_max3_f32 (the operands are finite or -inf, so no
// NaN quieting is needed, which fmaxf would add for values the compiler
// cannot prove canonical)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Wait states between the last MFMA that wrote a register and a VALU access
// of it (a 16-pass MFMA needs 18).
__device__ __forceinline__ void mfma_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// K operand, key block mb (keys 32 mb + r), contraction step ks (columns
// 16 ks + 8 g .. +7 = granule 2 ks + g): ht_off(32 mb + r, 2 ks + g) =
// kbase + 2048 ks + 512 mb (the row swizzle only touches bits 2 and 3).
__device__ __forceinline__ u32 k_base32(int lane) {
  const u32 r = (u32)lane & 31u, g = (u32)lane >> 5;
  return g * 1024u + 16u * (r ^ ht_swz(g));
}

__device__ __forceinline__ f16x8 read_k32(const SMLA_LDS uint8_t* tb, u32 kb, int ks, int mb) {
  return __builtin_bit_cast(f16x8, lds_read_b128(tb + kb + 2048u * (u32)ks + 512u * (u32)mb));
}

// V^T operand, output block nb (columns 32 nb .. +31), P.V step kk: element e
// of lane (n, g) is key 16 kk + 8 (e / 4) + 4 g + e % 4, the order in which
// the S^T accumulators hold the keys (register 8 (kk % 2) + e of key block
// kk / 2), so P^T is those eight registers.  Read h of the pair (elements
// 4h .. 4h+3): lane 4k + c of the 16-lane group (nh, g) points at key
// 16 kk + 8 h + 4 g + k, columns 32 nb + 16 nh + 4 c .. +3, i.e. granule
// 4 nb + 2 nh + c / 2, byte 8 (c % 2)  ->  vbase(h) + 4096 nb + 256 kk.
__device__ __forceinline__ u32 v_base32(int lane, int h) {
  const u32 j = (u32)lane & 15u, k = j >> 2, c = j & 3u, nh = ((u32)lane >> 4) & 1u, g = (u32)lane >> 5;
  const u32 G = 2u * nh + (c >> 1);          // granule modulo 4 (4 nb is added per block)
  const u32 key = 8u * (u32)h + 4u * g + k;  // low four bits of the key
  return G * 1024u + 16u * (key ^ ht_swz(G)) + 8u * (c & 1u);
}

__device__ __forceinline__ f16x8 read_vt32(const SMLA_LDS uint8_t* tb, u32 vb0, u32 vb1, int nb, int kk) {
  const u32 o = 4096u * (u32)nb + 256u * (u32)kk;
  const s16x4 a = lds_read_tr16(tb + vb0 + o), b = lds_read_tr16(tb + vb1 + o);
  const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(f16x8, ab);
}

template <bool SINK>
__global__ __launch_bounds__(kWaves * 64, 1) void smla_f16_wide_kernel(AttnParams p) {
  constexpr int NW = kWaves;
  constexpr int CT = kChunkTiles;
  __shared__ __attribute__((aligned(1024))) uint8_t kt[kHTileBytes];   // dequantised fp16 tile
  __shared__ __attribute__((aligned(1024))) uint8_t s8[kTileBytes];    // staged fp8 tile
  __shared__ __attribute__((aligned(16))) float ssc[kBK * kMaxScaleCols];  // its block scales
  __shared__ u32 rowid[CT * kBK];
  __shared__ u32 vmask[CT * 2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  const int u = xcd_token(blockIdx.x, p.T * p.splits);  // (token, run of slots)
  const int t = u / p.splits;
  const int sp = u - t * p.splits;

  // ---- Prologue.  The loads that need only the token number go out first
  // (sequence bounds, length word, the index words of the first chunk), the
  // page loads as soon as those land, then q, so that waiting for the pages
  // (issued before q; loads retire in order) does not wait for q, and q's
  // latency runs under the translation and the first gather.
  // lane i: cu_seqlens[1 + i] (sequences 0..63), loaded from a clamped
  // address; the value is selected only where it is used (see slot_index)
  const int cu_raw = p.cu_seqlens[1 + lane <= p.B ? 1 + lane : p.B];
  const int cu_first = p.cu_seqlens[0];
  const u32 len = p.lengths[t];
  constexpr int kPer = CT / NW;  // first-chunk tiles per wave
  u32 ix0[kPer];
  {
    const u32 cap = (u32)p.split_tiles * (u32)kBK;
    const u32 s0 = (u32)sp * cap;
    const u32 run = (u32)p.K > s0 ? ((u32)p.K - s0 < cap ? (u32)p.K - s0 : cap) : 0u;
    const u32* row = run > 0 ? p.indices + (size_t)t * p.K + s0 : p.lengths + t;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const u32 j = (u32)(wave + NW * r) * (u32)kBK + (u32)lane;
      const u32 v = row[j < run ? j : 0u];
      ix0[r] = j < run ? v : 0u;
    }
  }
  // the ballot runs whatever B is, so the load above is used unconditionally
  // and stays where it is issued
  const int cnt64 = __popcll(__ballot((1 + lane <= p.B ? cu_raw : 0x7fffffff) <= t));
  int b;
  if (p.B <= 64) {
    b = t < cu_first ? p.B : cnt64;
  } else {
    b = token_sequence(p.cu_seqlens, p.B, t);
  }
  TokenSlots ts;
  token_run_len(p, t, sp, b, len, ts);
  const int ntiles = (int)((ts.L + kBK - 1) / kBK);

  GatherArgs ga;
  ga.kv = p.kv;
  ga.page_table = p.page_table;
  ga.indices = p.indices;
  ga.num_rows = p.num_rows;
  ga.kv_bytes = p.kv_bytes;
  ga.K = p.K;
  ga.P = p.P;
  ga.max_pages = p.max_pages;
  ga.num_pages = p.num_pages;
  const v4i sc_rsrc = make_rsrc(p.scales, p.scale_bytes);
  const int ncols = p.scale_cols;
  const int pitch = (ncols + 3) & ~3;  // <= kMaxScaleCols
  const u32 pitch_magic = ((1u << 20) + (u32)pitch - 1u) / (u32)pitch;

  const int hl = lane & 31;  // head within the wave (MFMA N column)
  const int g = lane >> 5;   // contraction half held by this lane
  const int head = wave * kHeadsPerWave + hl;
  const bool head_ok = head < p.H;
  const bool wave_active = wave * kHeadsPerWave < p.H;  // wave-uniform

  // pages of the first chunk (the same translation as translate_chunk)
  const int n0 = ntiles < CT ? ntiles : CT;
  int pg0[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = wave + NW * r;
    pg0[r] = slot_page_unbranched(ts, ga, i, lane, ix0[r]);  // -1 past the list
  }

  // q: lane (hl, g) holds q[head][16 ks + 8 g .. +7]
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order of the loads above and below
  v4i raw[36];
  {
    const uint16_t* qrow = p.q + ((size_t)t * p.H + (head_ok ? head : 0)) * kQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const v4i v = *(const v4i*)(qrow + 16 * ks);  // a lane without a head reads head 0
      raw[ks] = head_ok ? v : v4i{0, 0, 0, 0};
    }
  }

#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = wave + NW * r;
    if (i < n0) {
      const u32 j = (u32)i * (u32)kBK + (u32)lane;
      publish_slots(ga, j < ts.L ? ix0[r] : 0u, pg0[r], rowid + kBK * i, vmask + 2 * i, lane);
    }
  }
  __syncthreads();
  if (ntiles > 0) {
    gather_tile<NW, true>(v4i{}, ga, rowid, s8, wave, lane);
    stage_block_scales<NW>(sc_rsrc, rowid, ssc, pitch, pitch_magic, ncols, p.num_rows, p.scale_bytes, wave, lane);
  }

  // ---- Q as the B operand, scaled by 2^eq (largest |q| of the head in
  // [128, 256)) and held in fp16, which represents every bf16 value of that
  // range exactly.
  f16x8 qreg[36];
  float c2h;  // softmax scale * log2(e) * 2^-eq
  {
    u32 mbits = 0;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32 two = (u32)raw[ks][w];
        mbits = max(mbits, max(two & 0x7FFFu, (two >> 16) & 0x7FFFu));
      }
    float amax = __uint_as_float(mbits << 16);
    amax = fmaxf(amax, shfl_xor32(amax));
    int eq = fit_exponent(amax);
    eq = eq < -100 ? -100 : (eq > 100 ? 100 : eq);
    const float up = __builtin_amdgcn_ldexpf(1.0f, eq);
    c2h = __builtin_amdgcn_ldexpf(p.scale_log2, -eq);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      v4i h;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32 two = (u32)raw[ks][w];
        h[w] = (int)pack_h2(__uint_as_float(two << 16) * up, __uint_as_float(two & 0xffff0000u) * up);
      }
      qreg[ks] = __builtin_bit_cast(f16x8, h);
    }
  }

  // scale column of each fp8 granule this lane dequantises (granules wave + 4 rep)
  int scol[9];
#pragma unroll
  for (int rep = 0; rep < 9; ++rep) scol[rep] = (16 * (wave + NW * rep)) / p.sbs;

  // Per tile, every wave: (1) tile factor 2^ek, (2) the FP16 copy of the
  // staged tile, barrier, (3) the gather of tile + 1 (a new chunk of slots is
  // translated first).  Returns ek; mk0 / mk1 get the tile's validity mask.
  // (Issuing the copies between the next QK^T's MFMAs instead measured
  // slower: the copy issue then holds up the MFMA issue.)
  auto stage = [&](int tile, u32& mk0, u32& mk1) {
    const int ek = tile_exponent(ssc, pitch, lane);
    dequant_tile<NW>(s8, kt, ssc, pitch, scol, ek, wave, lane);
    mk0 = __builtin_amdgcn_readfirstlane(vmask[2 * (tile % CT)]);
    mk1 = __builtin_amdgcn_readfirstlane(vmask[2 * (tile % CT) + 1]);
    __syncthreads();  // fp16 tile complete; the fp8 stage and scales are free
    if (tile + 1 < ntiles) {
      const int tg = tile + 1;
      if (tg % CT == 0) {
        translate_chunk<NW, CT>(ts, ga, tg, ntiles - tg < CT ? ntiles - tg : CT, rowid, vmask, wave, lane);
        wait_vmem_all();
        __syncthreads();
      }
      gather_tile<NW, true>(v4i{}, ga, rowid + kBK * (tg % CT), s8, wave, (int)opaque((u32)lane));
      stage_block_scales<NW>(sc_rsrc, rowid + kBK * (tg % CT), ssc, pitch, pitch_magic, ncols, p.num_rows,
                             p.scale_bytes, wave, lane);
    }
    return ek;
  };

  wait_vmem_all();
  __syncthreads();

  // A wave without heads (H < 128) helps with the staging only; it takes
  // part in every barrier of the waves that compute, in the same order.
  if (!wave_active) {
    for (int tile = 0; tile < ntiles; ++tile) {
      u32 mk0, mk1;
      (void)stage(tile, mk0, mk1);
      wait_vmem_all();
      __syncthreads();
    }
    if (p.splits == 1) {
      for (int k = 0; k < 4; ++k) __syncthreads();  // the two rounds of output staging
    }
    return;
  }

  float m_run = kNegInf;  // running max, log2 domain
  float l_part = 0.f;     // partial row sum of p = exp2(s - m_run) over this lane's keys
  int E = 0;              // O holds the output numerator in units of 2^-E
  bool e_set = false;
  v16f o[16];
#pragma unroll
  for (int nb = 0; nb < 16; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nb][i] = 0.f;

  const u32 kb = k_base32(lane);
  const u32 vb0 = v_base32(lane, 0), vb1 = v_base32(lane, 1);

  for (int tile = 0; tile < ntiles; ++tile) {
    u32 mk0, mk1;
    const int ek = stage(tile, mk0, mk1);
    const SMLA_LDS uint8_t* tb = (const SMLA_LDS uint8_t*)kt;

    // (4) S^T = K . Q^T: two 32-key blocks, 36 contraction steps of 16,
    // operands read one step ahead
    v16f s0, s1;
    const u32 kbo = opaque(kb);
    f16x8 ka0 = read_k32(tb, kbo, 0, 0), ka1 = read_k32(tb, kbo, 0, 1);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      f16x8 kn0, kn1;
      if (ks < 35) {
        kn0 = read_k32(tb, kbo, ks + 1, 0);
        kn1 = read_k32(tb, kbo, ks + 1, 1);
      }
      if (ks == 0) {
        mfma32_f16_v0(s0, ka0, qreg[0]);
        mfma32_f16_v0(s1, ka1, qreg[0]);
      } else {
        mfma32_f16_v(s0, ka0, qreg[ks]);
        mfma32_f16_v(s1, ka1, qreg[ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (ks < 35) {
        ka0 = kn0;
        ka1 = kn1;
      }
    }
    mfma_fence();  // the softmax reads the scores next

    // (5) online softmax.  Lane (head hl, half g) holds, in register i of
    // key block mb, the score of key 32 mb + 8 (i / 4) + 4 g + i % 4, in
    // units of 2^(eq + ek).  Scores go to the log2 domain first, so the
    // largest one minus the running max is exactly 0 (a single listed key
    // gets p = 1 exactly).
    const float c2t = __builtin_amdgcn_ldexpf(c2h, -ek);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] *= c2t;
      s1[i] *= c2t;
    }
    // slots not read get -inf; the branch is wave-uniform and taken only by
    // ragged tiles
    if ((mk0 & mk1) != 0xFFFFFFFFu) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int bit = 8 * (i >> 2) + 4 * g + (i & 3);
        s0[i] = ((mk0 >> bit) & 1u) ? s0[i] : kNegInf;
        s1[i] = ((mk1 >> bit) & 1u) ? s1[i] : kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = max3f(tmax, s0[i], s1[i]);
    tmax = fmaxf(tmax, shfl_xor32(tmax));
    const bool upd = tmax > m_run + kLazyRescale;
    // O's unit follows ek when they drift apart (wave-uniform: ek is)
    const bool move_e = !e_set || E - ek > kUnitDrift || ek - E > kUnitDrift;
    if (__any(upd) || move_e) {
      const bool o_live = e_set;  // wave-uniform: a P.V has run
      const float m_new = upd ? tmax : m_run;
      const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      const float beta = move_e && e_set ? __builtin_amdgcn_ldexpf(1.0f, ek - E) : 1.0f;
      m_run = m_new;
      l_part *= alpha;
      if (move_e) {
        E = ek;
        e_set = true;
      }
      const float f = alpha * beta;
      // O lives in AGPRs; the multiply goes through a VGPR one value at a
      // time (a plain C++ multiply made the compiler move all of O to VGPRs
      // and spill q).  The last MFMA that wrote O is a whole QK^T back.
      // Before the first tile's P.V, O is zero and needs no rescale.
      if (o_live) {
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float tmp;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(o[nb][i]), "=&v"(tmp) : "v"(f));
          }
        }
      }
    }
    const float msub = (m_run == kNegInf) ? 0.f : m_run;
    // P in O's units: exp2(s - m + E - ek); its row sum is scaled back to p units
    const float bias = (float)(E - ek) - msub;
    f16x8 pv[4];
    float lsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const v16f& sb = (kk >> 1) ? s1 : s0;
      v4i w;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int i0 = 8 * (kk & 1) + 2 * d;
        const float y0 = __builtin_amdgcn_exp2f(sb[i0] + bias), y1 = __builtin_amdgcn_exp2f(sb[i0 + 1] + bias);
        lsum += y0 + y1;
        w[d] = (int)pack_h2(y0, y1);
      }
      pv[kk] = __builtin_bit_cast(f16x8, w);
    }
    l_part += __builtin_amdgcn_ldexpf(lsum, ek - E);

    // (6) O^T += V^T . P^T: sixteen 32-column output blocks, four 16-key
    // steps each, operands read one step ahead.  The empty asm ties the read
    // bases to P so the transposed reads are not hoisted above the softmax.
    u32 v0 = vb0, v1 = vb1;
    asm volatile("" : "+v"(v0), "+v"(v1) : "v"(pv[0]), "v"(pv[1]), "v"(pv[2]), "v"(pv[3]));
    f16x8 va = read_vt32(tb, v0, v1, 0, 0);
#pragma unroll
    for (int st = 0; st < 64; ++st) {
      const int nb = st >> 2, kk = st & 3;
      f16x8 vn;
      if (st < 63) vn = read_vt32(tb, v0, v1, (st + 1) >> 2, (st + 1) & 3);
      o[nb] = mfma32_f16(va, pv[kk], o[nb]);
      __builtin_amdgcn_sched_barrier(0);
      if (st < 63) va = vn;
    }

    // (7) tile + 1 landed; every wave is done with the fp16 tile
    wait_vmem_all();
    __syncthreads();
  }

  // ---- epilogue: normalise (sink in the denominator only) and store bf16,
  // or hand the unnormalised run result (O in units of 2^-m) to the combine
  const float l_tot = l_part + shfl_xor32(l_part);
  if (p.splits > 1) {
    if (head_ok) {
      const size_t row = (size_t)u * p.H + head;
      float* po = p.part_o + row * kV;
      const float f = __builtin_amdgcn_ldexpf(1.0f, -E);
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(v4f*)(po + 32 * nb + 8 * j + 4 * g) =
              v4f{o[nb][4 * j], o[nb][4 * j + 1], o[nb][4 * j + 2], o[nb][4 * j + 3]} * f;
      if (g == 0) *(float2*)(p.part_ml + 2 * row) = float2{m_run, l_tot};
    }
    return;
  }
  float den = l_tot;
  if (SINK && head_ok && m_run != kNegInf) den += __builtin_amdgcn_exp2f(p.sink[head] * kLog2e - m_run);
  const float inv = (m_run != kNegInf && den > 0.f) ? __builtin_amdgcn_ldexpf(1.0f / den, -E) : 0.f;
  // bf16 rows through LDS (the fp16 tile is free): 16 heads of a wave at a
  // time, rows 1040 bytes apart, then one coalesced 1 KiB store per head row
  constexpr u32 kPitch = 1040;
  static_assert(NW * 16 * kPitch <= kHTileBytes, "output staging room");
  uint8_t* const stage_out = kt + (u32)wave * 16u * kPitch;
  const int rows = p.H - wave * kHeadsPerWave < kHeadsPerWave ? p.H - wave * kHeadsPerWave : kHeadsPerWave;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((hl >> 4) == half) {
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32 n = 32u * (u32)nb + 8u * (u32)j + 4u * (u32)g;
          const v2i w = {(int)pack_bf16x2(o[nb][4 * j] * inv, o[nb][4 * j + 1] * inv),
                         (int)pack_bf16x2(o[nb][4 * j + 2] * inv, o[nb][4 * j + 3] * inv)};
          *(SMLA_LDS v2i*)((SMLA_LDS uint8_t*)stage_out + (u32)(hl & 15) * kPitch + 2u * n) = w;
        }
    }
    __syncthreads();
    uint16_t* const obase = p.out + ((size_t)t * p.H + (size_t)wave * kHeadsPerWave + 16 * half) * kV + 8 * lane;
    const int r1 = rows - 16 * half < 16 ? rows - 16 * half : 16;  // wave-uniform, a multiple of 16
    for (int r0 = 0; r0 < r1; r0 += 4) {
      v4i v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[r] = lds_read_b128((const SMLA_LDS uint8_t*)stage_out + (u32)(r0 + r) * kPitch + 16u * (u32)lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) store_stream(obase + (size_t)(r0 + r) * kV, v[r]);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_f16_wide(const AttnParams& p, hipStream_t stream) {
  if (p.scales == nullptr || p.scale_cols < 1 || p.scale_cols > kMaxScaleCols) return hipErrorNotSupported;
  if (p.sbs < kQK && p.sbs % 16 != 0) return hipErrorNotSupported;
  if (p.H > kWaves * kHeadsPerWave) return hipErrorNotSupported;
  dim3 grid(p.T * p.splits), block(kWaves * 64);
  if (p.sink == nullptr) hipLaunchKernelGGL((smla_f16_wide_kernel<false>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((smla_f16_wide_kernel<true>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla

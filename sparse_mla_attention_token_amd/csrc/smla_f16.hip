// Sparse MLA prefill attention on gfx950 FP16 MFMA: the blockwise-scale path.
//
// What is computed is the same as on the FP8 path (page
// "mla_sm100_prefill_sparse_fp8", function description, Parameters and Args):
// out[t,h,:] = sum_j softmax_j(scale * q[t,h,:] . k_j) v_j with an optional
// per-head sink logit in the denominator, where k_j is the 576-wide latent row
// dequantised with its block scales, k_j[c] = fp8(kv[row, c]) * scales[row,
// c / sbs] (the "scale_block_size" and "scales_ptr" arguments: one f32 per
// sbs-wide column block of a physical row), and v_j its first 512 columns
// (so V uses the first 512 / sbs blocks of the same scales).
//
// A block scale is an arbitrary f32 that varies along the contraction of both
// products, so it cannot ride on the MFMA's power-of-two operand scales.  Each
// gathered tile is therefore dequantised once, by the whole workgroup, into an
// FP16 copy in LDS, and both products run on v_mfma_f32_16x16x32_f16:
//   * S^T[64 keys x 16 heads] = K . Q^T per wave (keys on M, as on the FP8
//     path), q held in registers as the B operand;
//   * online exp2 softmax with the lazy rescale of the FP8 path;
//   * O^T[512 x 16 heads] += V^T . P^T, P in fp16, V^T read from the same
//     FP16 tile with ds_read_b64_tr_b16.
// FP16 rather than BF16: the 11-bit significand keeps fp8 * scale, q and P
// within 2^-12 relative, where BF16's 2^-9 on K alone doubles the output
// error.  FP16's narrow exponent range is managed with powers of two: q is
// scaled per head so its largest magnitude sits in [128, 256); a tile is
// dequantised with a factor 2^ek that brings 448 * (largest block scale of the
// tile) into [128, 256) -- an element becomes fp16(fp8 * fp16(scale * 2^ek)):
// the FP8 code widened to fp16 exactly, times the block scale held in fp16,
// one rounding -- O is kept in units of 2^-E, and P is formed as
// exp2(s - m + E - ek) so every tile lands in those units; E follows ek
// (rescaling O) only when they drift more than 4 binades apart.
//
// Work decomposition: one workgroup per (token, group of 64 heads), four waves
// of 16 heads.  The FP8 rows are staged with the shared gather (one stage,
// one tile ahead of the compute), the block scales of the 64 rows next to
// them.
#include "smla_device.h"
#include "smla_gather.h"
#include "smla_kernels.h"

namespace smla {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyRescale = 8.0f;   // log2 headroom before O is rescaled
constexpr int kUnitDrift = 4;          // binades E may trail or lead a tile's ek
constexpr int kChunkTiles = 32;        // 2048 slots translated at a time
constexpr int kHeadsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kHeadsPerGroup = kHeadsPerWave * kWaves;  // 64
constexpr int kMaxScaleCols = 36;      // ceil(576 / 16): smallest block size is 16
constexpr int kHTileBytes = kBK * kQK * 2;              // 73728

// FP16 tile: row r (key), 8-column granule G (16 bytes) at
//   G * 1024 + 16 * (r ^ 12 (G & 1)).
// K operand reads (16 consecutive rows, one granule per 16-lane group) and
// the transposed V reads (4 rows x 2 adjacent granules per 16 lanes, the odd
// granule's rows XORed with 12) are free of bank conflicts for 32 and 64
// banks: each 16-lane group covers two distinct 64-byte segments of a 128-byte
// window, two groups four distinct segments of a 256-byte window.
__device__ __forceinline__ u32 ht_off(u32 r, u32 G) { return G * 1024u + 16u * (r ^ (12u * (G & 1u))); }

__device__ __forceinline__ v4f mfma_f16(f16x8 a, f16x8 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Transposed 16-bit read: within each 16-lane group, lane 4k + c supplies
// the address of 4 consecutive halves (row k of a 4 x 16 block, columns
// 4c .. 4c + 3); lane j receives column j of the block, element k from row k.
__device__ __forceinline__ s16x4 lds_read_tr16(const SMLA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMLA_LDS s16x4*)p);
}


// Reductions over the four lanes that hold one head (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float head_max(float x) {
  x = fmaxf(x, shfl_xor16(x));
  return fmaxf(x, shfl_xor32(x));
}
__device__ __forceinline__ float head_sum(float x) {
  x += shfl_xor16(x);
  return x + shfl_xor32(x);
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

// K operand for key block mb, contraction step ks: rows 16 mb + r, granule
// 4 ks + g (r = lane % 16, g = lane / 16)  ->  kbase + 4096 ks + 256 mb.
__device__ __forceinline__ u32 k_base16(int lane) {
  const u32 r = (u32)lane & 15u, g = (u32)lane >> 4;
  return g * 1024u + 16u * (r ^ (12u * (g & 1u)));
}

// V^T operand for output block nb (columns 16 nb .. +15) and key block kb:
// MFMA slot s of lane (n, g) holds key 32 kb + 16 (s / 4) + 4 g + s % 4, so
// that it matches the P^T operand built from the S^T accumulators.  Read
// half h (slots 4h .. 4h+3): lane 4k + c of group g points at key
// 32 kb + 16 h + 4 g + k, columns 16 nb + 4 c .. +3  ->  vbase + 2048 nb + 512 kb + 256 h.
__device__ __forceinline__ u32 v_base16(int lane) {
  const u32 i = (u32)lane & 15u, k = i >> 2, c = i & 3u, g = (u32)lane >> 4;
  const u32 key = 4u * g + k;          // row within the 16-row group
  const u32 G = c >> 1;                // granule 2 nb + c / 2
  return G * 1024u + 16u * (key ^ (12u * G)) + 8u * (c & 1u);
}

__device__ __forceinline__ f16x8 read_k16(const SMLA_LDS uint8_t* tb, u32 kb, int ks, int mb) {
  const u32 o = 4096u * (u32)ks + 256u * (u32)mb;
  return __builtin_bit_cast(f16x8, lds_read_b128(tb + kb + o));
}

__device__ __forceinline__ f16x8 read_vt16(const SMLA_LDS uint8_t* tb, u32 vb, int nb, int kb) {
  const u32 o = 2048u * (u32)nb + 512u * (u32)kb;
  const s16x4 a = lds_read_tr16(tb + vb + o), b = lds_read_tr16(tb + vb + o + 256u);
  const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(f16x8, ab);
}

// two f32 -> two fp16 (round to nearest even) in one dword
__device__ __forceinline__ u32 pack_h2(float a, float b) {
  return __builtin_bit_cast(u32, __builtin_convertvector((v2f){a, b}, f16x2));
}

template <bool SINK>
__global__ __launch_bounds__(kWaves * 64, 1) void smla_f16_block_kernel(AttnParams p) {
  constexpr int NW = kWaves;
  constexpr int CT = kChunkTiles;
  __shared__ __attribute__((aligned(1024))) uint8_t kt[kHTileBytes];   // dequantised fp16 tile
  __shared__ __attribute__((aligned(1024))) uint8_t s8[kTileBytes];    // staged fp8 tile
  // block scales of the staged rows: slot s at ssc[s * pitch ..], the row's
  // ncols scales then zeros up to a multiple of four
  __shared__ __attribute__((aligned(16))) float ssc[kBK * kMaxScaleCols];
  __shared__ u32 rowid[CT * kBK];
  __shared__ u32 vmask[CT * 2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  const int HG = (p.H + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int u = xcd_token(blockIdx.x, p.T * p.splits * HG);  // (token, run of slots, head group)
  const int ur = u / HG;                                      // (token, run)
  const int hg = u - ur * HG;
  const int t = ur / p.splits;
  const int b = token_sequence(p.cu_seqlens, p.B, t);

  TokenSlots ts;
  token_run(p, t, ur - t * p.splits, b, ts);
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

  const int r = lane & 15;   // head within the wave (MFMA N column)
  const int g = lane >> 4;   // contraction quarter held by this lane
  const int head = hg * kHeadsPerGroup + wave * kHeadsPerWave + r;
  const bool head_ok = head < p.H;
  const bool wave_active = hg * kHeadsPerGroup + wave * kHeadsPerWave < p.H;  // wave-uniform

  // Stage the block scales of a tile's 64 rows, one padded row per slot:
  // copy k fills ssc[64 k .. 64 k + 63], lane i the float 64 k + i = slot s,
  // column c.  Rows that are not read and the padding fetch zeros.
  const int pitch = (ncols + 3) & ~3;                        // <= kMaxScaleCols
  const u32 pitch_magic = ((1u << 20) + (u32)pitch - 1u) / (u32)pitch;  // x / pitch = x * magic >> 20 for x < 64 pitch
  auto gather_scales = [&](const u32* rid) {
    for (int k = wave; k < pitch; k += NW) {
      const u32 i = 64u * (u32)k + (u32)lane;
      const u32 s = (i * pitch_magic) >> 20, c = i - s * (u32)pitch;
      const u32 row = rid[s];
      const bool ok = row < p.num_rows && c < (u32)ncols;
      const u32 soff = ok ? (row * (u32)ncols + c) * 4u : p.scale_bytes;
      load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&ssc[64 * k], soff);
    }
  };

  // ---- translation of the first chunk, gather of tile 0
  translate_chunk<NW, CT>(ts, ga, 0, ntiles < CT ? ntiles : CT, rowid, vmask, wave, lane);
  __syncthreads();
  if (ntiles > 0) {
    gather_tile<NW, true>(v4i{}, ga, rowid, s8, wave, lane);
    gather_scales(rowid);
  }

  // ---- Q as the B operand: lane (r, g) holds q[head][32 ks + 8 g .. +7],
  // scaled by 2^eq (largest |q| of the head in [128, 256)) and held in fp16,
  // which represents every bf16 value of that range exactly.
  f16x8 qreg[18];
  float c2h;  // softmax scale * log2(e) * 2^-eq
  {
    const uint16_t* qrow = p.q + ((size_t)t * p.H + (head_ok ? head : 0)) * kQK + 8 * g;
    v4i raw[18];
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) raw[ks] = head_ok ? *(const v4i*)(qrow + 32 * ks) : v4i{0, 0, 0, 0};
    u32 mbits = 0;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32 two = (u32)raw[ks][w];
        mbits = max(mbits, max(two & 0x7FFFu, (two >> 16) & 0x7FFFu));
      }
    const float amax = head_max(__uint_as_float(mbits << 16));
    int eq = fit_exponent(amax);
    eq = eq < -100 ? -100 : (eq > 100 ? 100 : eq);
    const float up = __builtin_amdgcn_ldexpf(1.0f, eq);
    c2h = __builtin_amdgcn_ldexpf(p.scale_log2, -eq);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
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
  for (int rep = 0; rep < 9; ++rep) {
    const int gl = wave + NW * rep;
    scol[rep] = p.sbs >= kQK ? 0 : (16 * gl) / p.sbs;
  }

  float m_run = kNegInf;  // running max, log2 domain
  float l_part = 0.f;     // partial row sum of p = exp2(s - m_run) over this lane's keys
  int E = 0;              // O holds the output numerator in units of 2^-E
  bool e_set = false;
  v4f o[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};

  wait_vmem_all();
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    // (1) tile factor 2^ek: 448 (largest |e4m3fn|) times the largest block
    // scale of the 64 rows lands in [128, 256).  Every wave reduces the whole
    // table itself, so no extra barrier is needed: lane s takes the maximum
    // of its slot's row (16 bytes per read, five reads per step so they are
    // in flight together; a vector read twice changes nothing), then the
    // wave reduces the 64 row maxima.
    float smax = 0.f;
    {
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
    }
    smax = wave_max_nonneg(smax);
    int ek = fit_exponent(448.0f * smax);
    ek = ek < -100 ? -100 : (ek > 100 ? 100 : ek);

    // (2) dequantise: lane = row slot, wave + 4 rep = fp8 granule (16 columns
    // -> fp16 granules 2 gl and 2 gl + 1): fp16(fp8 * fp16(scale * 2^ek)),
    // two codes per conversion (exact: every e4m3fn value is an fp16 value)
    // and two products per packed fp16 multiply.  The bytes and the scale of
    // granule rep + 1 are read while granule rep is converted.
    v4i raw_n = lds_read_b128((const SMLA_LDS uint8_t*)s8 + tile_off((u32)lane, (u32)wave));
    const SMLA_LDS float* srow = (const SMLA_LDS float*)&ssc[lane * pitch];
    float sc_n = srow[scol[0]];
#pragma unroll
    for (int rep = 0; rep < 9; ++rep) {
      const u32 gl = (u32)(wave + NW * rep);
      const v4i raw = raw_n;
      const _Float16 sh = (_Float16)__builtin_amdgcn_ldexpf(sc_n, ek);
      const f16x2 s2 = {sh, sh};
      if (rep < 8) {
        raw_n = lds_read_b128((const SMLA_LDS uint8_t*)s8 + tile_off((u32)lane, gl + (u32)NW));
        sc_n = srow[scol[rep + 1]];
      }
      u32 w[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // the conversion's scale operand only applies its exponent; 1 keeps
        // the codes as they are
        const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[d], 1.0f, false) * s2;
        const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[d], 1.0f, true) * s2;
        w[2 * d] = __builtin_bit_cast(u32, lo);
        w[2 * d + 1] = __builtin_bit_cast(u32, hi);
      }
      *(SMLA_LDS v4i*)(kt + ht_off((u32)lane, 2u * gl)) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *(SMLA_LDS v4i*)(kt + ht_off((u32)lane, 2u * gl + 1u)) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
    const u32 mk0 = vmask[2 * (tile % CT)], mk1 = vmask[2 * (tile % CT) + 1];
    __syncthreads();  // fp16 tile complete; the fp8 stage and scales are free

    // (3) stage tile + 1 (a new chunk of slots is translated first)
    if (tile + 1 < ntiles) {
      const int tg = tile + 1;
      if (tg % CT == 0) {
        translate_chunk<NW, CT>(ts, ga, tg, ntiles - tg < CT ? ntiles - tg : CT, rowid, vmask, wave, lane);
        wait_vmem_all();
        __syncthreads();
      }
      gather_tile<NW, true>(v4i{}, ga, rowid + kBK * (tg % CT), s8, wave, (int)opaque((u32)lane));
      gather_scales(rowid + kBK * (tg % CT));
    }

    if (wave_active) {
      const SMLA_LDS uint8_t* tb = (const SMLA_LDS uint8_t*)kt;
      // (4) S^T = K . Q^T: four 16-key blocks, 18 contraction steps of 32.
      // Operands are read two steps ahead (a ring of three) so the LDS
      // latency hides behind the four MFMAs of a step.
      const u32 kb = k_base16((int)opaque((u32)lane));
      v4f s[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) s[mb] = v4f{0.f, 0.f, 0.f, 0.f};
      f16x8 kr[3][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) kr[j][mb] = read_k16(tb, kb, j, mb);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ks + 2 < 18) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) kr[(ks + 2) % 3][mb] = read_k16(tb, kb, ks + 2, mb);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) s[mb] = mfma_f16(kr[ks % 3][mb], qreg[ks], s[mb]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // (5) online softmax.  Lane (head r, quarter g) holds, in register i of
      // block mb, the score of key 16 mb + 4 g + i, in units of 2^(eq + ek).
      // Scores are taken to the log2 domain first, so the largest one minus
      // the running max is exactly 0 (a single listed key gets p = 1 exactly).
      const float c2t = __builtin_amdgcn_ldexpf(c2h, -ek);
      const bool full = (mk0 & mk1) == 0xFFFFFFFFu;  // wave-uniform
      float tmax = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const u32 mk = (mb < 2) ? mk0 : mk1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int bit = 16 * (mb & 1) + 4 * g + i;
          float sv = s[mb][i] * c2t;
          if (!full) sv = ((mk >> bit) & 1u) ? sv : kNegInf;
          s[mb][i] = sv;
          tmax = fmaxf(tmax, sv);
        }
      }
      tmax = head_max(tmax);
      const bool upd = tmax > m_run + kLazyRescale;
      // O's unit follows ek when they drift apart (wave-uniform: ek is)
      const bool move_e = !e_set || E - ek > kUnitDrift || ek - E > kUnitDrift;
      if (__any(upd) || move_e) {
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
#pragma unroll
        for (int nb = 0; nb < 32; ++nb) {
          o[nb] *= f;
          if ((nb & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
      }
      const float msub = (m_run == kNegInf) ? 0.f : m_run;
      // P in O's units: exp2(s - m + E - ek); its row sum is scaled back to p units
      const float bias = (float)(E - ek) - msub;
      f16x8 pv[2];
      float lsum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        v4i w;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int mb = 2 * kb2 + h;
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            y[i] = __builtin_amdgcn_exp2f(s[mb][i] + bias);
            lsum += y[i];
          }
          w[2 * h] = (int)pack_h2(y[0], y[1]);
          w[2 * h + 1] = (int)pack_h2(y[2], y[3]);
        }
        pv[kb2] = __builtin_bit_cast(f16x8, w);
      }
      l_part += __builtin_amdgcn_ldexpf(lsum, ek - E);

      // (6) O^T += V^T . P^T, two output blocks per step (their MFMAs
      // interleaved so no two dependent ones are adjacent), operands read two
      // steps ahead.  The empty asm ties the read base to P so the transposed
      // reads are not hoisted above the softmax.
      u32 vb = v_base16(lane);
      asm volatile("" : "+v"(vb) : "v"(pv[0]), "v"(pv[1]));
      f16x8 vr[3][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) vr[j][q] = read_vt16(tb, vb, 2 * j + (q >> 1), q & 1);
#pragma unroll
      for (int pr = 0; pr < 16; ++pr) {
        if (pr + 2 < 16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) vr[(pr + 2) % 3][q] = read_vt16(tb, vb, 2 * (pr + 2) + (q >> 1), q & 1);
        }
        const int sl = pr % 3;
        o[2 * pr] = mfma_f16(vr[sl][0], pv[0], o[2 * pr]);
        o[2 * pr + 1] = mfma_f16(vr[sl][2], pv[0], o[2 * pr + 1]);
        o[2 * pr] = mfma_f16(vr[sl][1], pv[1], o[2 * pr]);
        o[2 * pr + 1] = mfma_f16(vr[sl][3], pv[1], o[2 * pr + 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }  // wave_active

    // (7) tile + 1 landed; every wave is done with the fp16 tile
    wait_vmem_all();
    __syncthreads();
  }

  // ---- epilogue: normalise (sink in the denominator only) and store bf16,
  // or hand the unnormalised run result (O in units of 2^-m) to the combine
  float l_tot = head_sum(l_part);
  if (p.splits > 1) {
    if (head_ok) {
      const size_t row = (size_t)ur * p.H + head;
      float* po = p.part_o + row * kV + 4 * g;
      const float f = __builtin_amdgcn_ldexpf(1.0f, -E);
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) *(v4f*)(po + 16 * nb) = o[nb] * f;
      if (g == 0) *(float2*)(p.part_ml + 2 * row) = float2{m_run, l_tot};
    }
    return;
  }
  if (SINK && head_ok && m_run != kNegInf) l_tot += __builtin_amdgcn_exp2f(p.sink[head] * kLog2e - m_run);
  const float inv = (m_run != kNegInf && l_tot > 0.f) ? __builtin_amdgcn_ldexpf(1.0f / l_tot, -E) : 0.f;
  if (head_ok) {
    uint16_t* orow = p.out + ((size_t)t * p.H + head) * kV + 4 * g;
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) {
      uint2 w;
      w.x = pack_bf16x2(o[nb][0] * inv, o[nb][1] * inv);
      w.y = pack_bf16x2(o[nb][2] * inv, o[nb][3] * inv);
      *(uint2*)(orow + 16 * nb) = w;
    }
  }
}

}  // namespace

hipError_t launch_f16_block(const AttnParams& p, hipStream_t stream) {
  if (p.scales == nullptr || p.scale_cols < 1 || p.scale_cols > kMaxScaleCols) return hipErrorNotSupported;
  if (p.sbs < kQK && p.sbs % 16 != 0) return hipErrorNotSupported;
  const int HG = (p.H + kHeadsPerGroup - 1) / kHeadsPerGroup;
  dim3 grid(p.T * p.splits * HG), block(kWaves * 64);
  if (p.sink == nullptr) hipLaunchKernelGGL((smla_f16_block_kernel<false>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((smla_f16_block_kernel<true>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla

// Sparse MLA prefill attention on gfx950 FP8 MFMA, paired-wave variant
// (unit scale and one scale per KV row; the same numerics as smla_fp8x2).
//
// What is computed is the attention of the page "mla_sm100_prefill_sparse_fp8"
// (function description, Parameters and Args) over the shared latent of the
// page "mla_prefill_sparse_qkv_fp8"; see smla_fp8x2.hip for the numerics (q
// and P as two FP8 terms on v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Why a second decomposition.  With one workgroup per token and 32 heads per
// wave, a wave's 512-column accumulator fills all its accumulation
// registers, q_lo has to live in LDS, only two KV stages fit, and the softmax
// of a tile runs while the matrix pipe idles.  Here a workgroup takes one
// token and 64 heads (two workgroups per token at 128 heads), as two pairs of
// waves.  The two waves of a pair share 32 heads and split the scores of a
// tile: wave m of the pair computes keys 32 m .. 32 m + 31.  For P.V every
// wave takes output columns 128 w .. 128 w + 127 of all 64 heads, so each
// transposed V^T fragment it reads feeds four MFMAs (two head blocks, hi and
// lo) and the workgroup reads V once per tile.  Its accumulator is a quarter
// of the workgroup's output, q (hi and lo) stays in registers, and three KV
// stages fit.  That buys the pipelining the pages get from separate softmax
// warps ("SM100MLA" page: softmax and correction roles): each iteration
// issues the next tile's QK^T MFMAs and runs this tile's softmax on the VALU
// in the same instruction stream, then every wave publishes its P quarter
// (its heads x its keys) through LDS, reads all four, and runs P.V.
// The exchange and the barrier it needs cost more than the pipelining gains
// when a token has 128 heads, so the library launches this kernel for up to
// 64 heads, where one workgroup per token would leave two of its four waves
// without heads (on MI355X: 3.0 ms instead of 4.3 ms for 8192 tokens x 64
// heads x 2048 keys), and for decode-sized launches with more heads: one run
// of fewer tokens than CUs whose 64-head groups fill the CUs.  There the two
// workgroups of a token each gather all of its rows (the second gather is
// mostly served by L2), which measured faster than one workgroup per token
// with the keys split into runs and merged afterwards.
//
// Running max.  Each wave keeps an integer running max m (log2 domain) for
// its heads and updates it lazily (only when a tile exceeds it by more than
// 2^8).  At the P exchange every head block moves to the larger of its
// pair's two maxima, so every rescale factor is a power of two: the two P
// quarters of a head block are brought to the common max through the E8M0
// block scales of the P.V MFMA (k-block 0 = the keys of the pair's wave 0,
// whose scale a lane of half 0 supplies, k-block 1 = those of wave 1, half
// 1), and O and the row sum by an exact exponent shift.
#include "smla_device.h"
#include "smla_fp8_ops.h"
#include "smla_gather.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr int kNS = 3;            // KV stages
constexpr int kGD = 2;            // gather distance (tiles in flight)
constexpr int kCT = 32;           // tiles per translated chunk (two chunk tables)
constexpr int kNoMax = -(1 << 20);  // running max before any key
constexpr int kLazy = 8;          // log2 headroom before O is rescaled

__device__ __forceinline__ int e8m0(int e) { return e < 0 ? 0 : (e > 254 ? 254 : e); }

// x * 2^d for a value held in an accumulation register, d <= 0 an integer
__device__ __forceinline__ float shift_down(float x, int d) { return __builtin_amdgcn_ldexpf(x, d); }

template <bool ROWSCALE, bool SINGLE, bool WIDE>
__global__ __launch_bounds__(256, 1) void smla_fp8pair_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t kvs[kNS][kTileBytes];
  __shared__ u32 rowid[2][kCT * kBK];        // pool rows of two translated chunks
  __shared__ u32 vmask[2][kCT * 2];          // validity masks of the same
  __shared__ __attribute__((aligned(16))) float rsc[ROWSCALE ? kNS : 1][kBK];
  __shared__ __attribute__((aligned(16))) float lrs[ROWSCALE ? kNS : 1][kBK];  // log2 of rsc
  __shared__ __attribute__((aligned(16))) int pex[4][2][64][4];  // P quarters: [wave][hi/lo][lane]
  __shared__ int sex[4][32][2];              // [wave][head]: running max, P exponent
  __shared__ float lex[4][32];               // row sums for the epilogue

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave >> 1, mm = wave & 1;  // pair = 32-head group, mm = key half of a tile
  const int HG = (p.H + 63) / 64;
  const int u0 = xcd_token(blockIdx.x, p.T * p.splits * HG);
  const int ur = u0 / HG, hg = u0 - ur * HG;
  const int t = ur / p.splits;
  const int sp = ur - t * p.splits;

  // ---- Prologue.  Every load that needs only the token number goes out
  // before anything waits, oldest first (as in smla_fp8x2): the sequence
  // boundaries, the index words of the first chunk of slots (read up to the
  // run's end in the row; the effective length masks them later), then q.
  // The index -> page chain then runs under the q load.
  int cu_next = 0x7fffffff;  // lane i: cu_seqlens[1 + i] (sequences 0..63)
  if (p.B <= 64 && 1 + lane <= p.B) cu_next = p.cu_seqlens[1 + lane];
  constexpr int kPer = kCT / 4;  // first-chunk tiles per wave
  u32 ix0[kPer];
  {
    const u32 cap = (u32)p.split_tiles * (u32)kBK;
    const u32 s0 = (u32)sp * cap;
    const u32 run = (u32)p.K > s0 ? ((u32)p.K - s0 < cap ? (u32)p.K - s0 : cap) : 0u;
    const u32* row = p.indices + (size_t)t * p.K + s0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const u32 j = (u32)(wave + 4 * r) * (u32)kBK + (u32)lane;
      ix0[r] = j < run ? row[j] : 0u;
    }
  }
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
  const v4i kv_rsrc = make_rsrc(p.kv, p.kv_bytes);
  const v4i sc_rsrc = make_rsrc(ROWSCALE ? (const void*)p.scales : (const void*)p.kv, ROWSCALE ? p.scale_bytes : 0u);

  const int hl = lane & 31, g = lane >> 5;
  const int head0 = hg * 64 + pair * 32;           // first head of the pair
  const int pair_heads = p.H - head0 < 32 ? (p.H - head0 > 0 ? p.H - head0 : 0) : 32;  // uniform
  const bool active = pair_heads > 0;  // wave-uniform

  // ---- Q, step 1: the pair's 32 head rows, loaded 1 KiB per instruction by
  // both waves of the pair (each takes half)
  v4i qv[18];
  {
    const uint8_t* qw = (const uint8_t*)(p.q + ((size_t)t * p.H + (size_t)head0) * kQK);
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      const u32 piece = 64u * (u32)(2 * kk + mm) + (u32)lane;
      qv[kk] = piece / 72u < (u32)pair_heads ? load_stream(qw + 16u * piece) : v4i{0, 0, 0, 0};
    }
  }

  // ---- the token's sequence and effective slot count, then the pages of
  // the first chunk (the same translation as translate_chunk)
  int b;
  if (p.B <= 64) {
    const int c0 = p.cu_seqlens[0];
    const int cnt = __popcll(__ballot(cu_next <= t));
    b = t < c0 ? p.B : cnt;
  } else {
    b = token_sequence(p.cu_seqlens, p.B, t);
  }
  TokenSlots ts;
  token_run(p, t, sp, b, ts);
  const int ntiles = (int)((ts.L + kBK - 1) / kBK);
  {
    const int n0 = ntiles < kCT ? ntiles : kCT;
    int pg0[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = wave + 4 * r;
      pg0[r] = i < n0 ? slot_page(ts, ga, i, lane, ix0[r]) : -1;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = wave + 4 * r;
      if (i < n0) {
        const u32 j = (u32)i * (u32)kBK + (u32)lane;
        publish_slots(ga, j < ts.L ? ix0[r] : 0u, pg0[r], rowid[0] + kBK * i, vmask[0] + 2 * i, lane);
      }
    }
  }

  // ---- Q, step 2: through LDS into the MFMA operand layout (read r of lane L
  // at 1024 r + 16 (L ^ (r % 16)), see smla_fp8x2).  Pair p stages its rows in
  // KV stage 1 + p, so tile 0 (stage 0) is gathered before q is split.
  {
    uint8_t* const qst = &kvs[1 + pair][0];
    static_assert(kNS >= 3, "q staging room");
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      const u32 piece = 64u * (u32)(2 * kk + mm) + (u32)lane;
      const u32 h = piece / 72u, pc = piece - 72u * h;
      const u32 r = 4u * (pc >> 3) + (pc & 3u), L = h + 32u * ((pc >> 2) & 1u);
      *(SMLA_LDS v4i*)((SMLA_LDS uint8_t*)qst + 1024u * r + 16u * (L ^ (r & 15u))) = qv[kk];
    }
  }
  __syncthreads();  // q rows and chunk 0 are in LDS

  // ---- gather tile 0 (in flight while q is split)
  if (ntiles > 0) {
    gather_tile<4, WIDE>(kv_rsrc, ga, rowid[0], kvs[0], wave, lane);
    if (ROWSCALE && wave == 0) {
      const u32 row = rowid[0][lane];
      const u32 soff = row < p.num_rows ? row * 4u : p.scale_bytes;
      load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&rsc[0][0], soff);
    }
  }

  v8i qhi[9], qlo[9];
  int sq_hi, sq_lo;
  {
    const uint8_t* const qst = &kvs[1 + pair][0];
    v4i raw[9][4];
#pragma unroll
    for (int ks = 0; ks < 9; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32 r = 4u * (u32)ks + (u32)c;
        raw[ks][c] = lds_read_b128((const SMLA_LDS uint8_t*)qst + 1024u * r + 16u * ((u32)lane ^ (r & 15u)));
      }
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int ks = 0; ks < 9; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) m2 = bf16x2_absmax(m2, (u32)raw[ks][c][w]);
    float amax = __uint_as_float((u32)(m2[0] > m2[1] ? m2[0] : m2[1]) << 16);
    amax = fmaxf(amax, shfl_xor32(amax));
    int e = fit_exponent(amax);
    e = e < -127 ? -127 : (e > 122 ? 122 : e);
    sq_hi = 127 - e;
    sq_lo = 123 - e;
    // codes: hi = fp8(x 2^e), lo = fp8(16 (x 2^e - hi)), the powers of two
    // applied by the conversions themselves.  Both waves of a pair hold the
    // same q registers, so each converts every other contraction step (wave
    // mm: ks = mm, mm + 2, ...) and the halves are swapped below.
    const float sdn = __builtin_amdgcn_ldexpf(1.0f, -e), sdn_lo = __builtin_amdgcn_ldexpf(1.0f, -e - 4);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      if ((ks & 1) != mm) continue;  // wave-uniform
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const u32 d0 = (u32)raw[ks][c][2 * w2], d1 = (u32)raw[ks][c][2 * w2 + 1];
          const float x0 = __uint_as_float(d0 << 16), x1 = __uint_as_float(d0 & 0xffff0000u);
          const float x2 = __uint_as_float(d1 << 16), x3 = __uint_as_float(d1 & 0xffff0000u);
          int h = cvt_fp8x2_div<false>(x0, x1, sdn, 0);
          h = cvt_fp8x2_div<true>(x2, x3, sdn, h);
          qhi[ks][2 * c + w2] = h;
          if (SINGLE) {
            qlo[ks][2 * c + w2] = 0;
            continue;
          }
          const v2f h01 = fp8x2_to_f32_mul<false>(h, sdn), h23 = fp8x2_to_f32_mul<true>(h, sdn);
          int lo = cvt_fp8x2_div<false>(x0 - h01[0], x1 - h01[1], sdn_lo, 0);
          lo = cvt_fp8x2_div<true>(x2 - h23[0], x3 - h23[1], sdn_lo, lo);
          qlo[ks][2 * c + w2] = lo;
        }
    }
  }
  __syncthreads();  // every wave has read its raw q rows
  {
    // the pair's staging area as [ks][hi, lo][lane] x 32 bytes (one stage)
    SMLA_LDS uint8_t* const qx = (SMLA_LDS uint8_t*)&kvs[1 + pair][0];
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      if ((ks & 1) != mm) continue;
      *(SMLA_LDS v8i*)(qx + 32u * ((u32)(128 * ks) + (u32)lane)) = qhi[ks];
      if (!SINGLE) *(SMLA_LDS v8i*)(qx + 32u * ((u32)(128 * ks + 64) + (u32)lane)) = qlo[ks];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      if ((ks & 1) == mm) continue;
      qhi[ks] = *(const SMLA_LDS v8i*)(qx + 32u * ((u32)(128 * ks) + (u32)lane));
      qlo[ks] = SINGLE ? v8i{} : *(const SMLA_LDS v8i*)(qx + 32u * ((u32)(128 * ks + 64) + (u32)lane));
    }
  }
  __syncthreads();  // every wave holds its q: the staging area is free

  // ---- gather tiles 1 .. kGD - 1
  const u32 kvs_lds = lds_addr_of(kvs);
  for (int tt = 1; tt < kGD && tt < ntiles; ++tt) {
    gather_tile<4, WIDE>(kv_rsrc, ga, rowid[0] + kBK * tt, kvs[tt], wave, lane);
    if (ROWSCALE && wave == 0) {
      const u32 row = rowid[0][kBK * tt + lane];
      const u32 soff = row < p.num_rows ? row * 4u : p.scale_bytes;
      load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&rsc[tt][0], soff);
    }
  }

  // ---- softmax state: integer running max (log2 domain) of the wave's
  // heads, its own row sum; O^T of both head blocks over the wave's 128
  // output columns, each block in units of its own running max m_o
  int m_run = kNoMax;
  float l_own = 0.f;
  const int gh = p.H - hg * 64 < 64 ? p.H - hg * 64 : 64;  // heads of the group (uniform)
  const bool blk1 = gh > 32;                              // head block 1 has heads
  int m_o[2] = {kNoMax, kNoMax};
  v16f o[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[b][c][i] = 0.f;
  const float c2 = p.scale_log2;
  const u32 kb0 = k_base(lane, 0), kb1 = k_base(lane, 1);

  // QK^T of this wave's 32 keys of the tile in stage st (hi and lo terms)
  auto qk = [&](int st) {
    const SMLA_LDS uint8_t* tb = (const SMLA_LDS uint8_t*)kvs[st];
    v16f s;
    v8i ka = read_k(tb, kb0, kb1, 0, mm);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      v8i kn;
      if (ks < 8) kn = read_k(tb, kb0, kb1, ks + 1, mm);
      s = ks == 0 ? mfma_fp8(ka, qhi[0], v16f{}, 127, sq_hi) : mfma_fp8(ka, qhi[ks], s, 127, sq_hi);
      if (!SINGLE) s = mfma_fp8(ka, qlo[ks], s, 127, sq_lo);
      if (ks < 8) ka = kn;
    }
    return s;
  };

  wait_vmem_all();  // tile 0 landed
  __syncthreads();
  // log2 of a tile's row scales, by the wave that loaded them, one iteration
  // before the softmax that reads them (the barrier at the top of that
  // iteration publishes them)
  if (ROWSCALE && wave == 0 && ntiles > 0) lrs[0][lane] = __builtin_amdgcn_logf(rsc[0][lane]);
  v16f s_cur;
  if (active && ntiles > 0) s_cur = qk(0);

  for (int tile = 0; tile < ntiles; ++tile) {
    const int st = tile % kNS;
    const int ch = tile / kCT, ct = tile - ch * kCT;
    const u32 mk = __builtin_amdgcn_readfirstlane(vmask[ch & 1][2 * ct + mm]);  // this wave's 32 keys

    // (1) tile + 1 has landed (issued one iteration ago) and every wave is
    // done with stage (tile - 1) % kNS, which the gather of tile + 2 refills
    wait_vmem_all();
    __syncthreads();
    if (ROWSCALE && wave == 0 && tile + 1 < ntiles)
      lrs[(tile + 1) % kNS][lane] = __builtin_amdgcn_logf(rsc[(tile + 1) % kNS][lane]);
    const int tg = tile + kGD;
    if (tg < ntiles && tg % kCT == 0) {  // tile tg opens a new chunk: translate it
      const int c0 = tg;
      translate_chunk<4, kCT>(ts, ga, c0, ntiles - c0 < kCT ? ntiles - c0 : kCT, rowid[(tg / kCT) & 1],
                              vmask[(tg / kCT) & 1], wave, lane);
      wait_vmem_all();
      __syncthreads();
    }
    const u32 gdst = kvs_lds + (u32)(tg % kNS) * (u32)kTileBytes;
    RowSrc<WIDE> gro = gather_no_src<WIDE>();  // past the last tile: zeros into a stage no tile reads any more
    if (tg < ntiles) {
      const u32* rid = rowid[(tg / kCT) & 1] + kBK * (tg % kCT);
      gro = gather_lane_src<WIDE>(ga, rid, wave, (int)opaque((u32)lane));
      if (ROWSCALE && wave == 0) {
        const u32 row = rid[lane];
        const u32 soff = row < p.num_rows ? row * 4u : p.scale_bytes;
        load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&rsc[tg % kNS][0], soff);
      }
    }

    // (2) this tile's softmax, cut into nine slices; with a next tile, slice
    // ks is issued between the two MFMAs of contraction step ks of that
    // tile's QK^T (measured: within one wave only a few VALU instructions per
    // MFMA run under the matrix pipe, the rest adds to its time; placing the
    // slices after every MFMA or in two accumulator chains measured slower).
    // Lane (hl, g), register i holds key 32 mm + 8 (i / 4) + 4 g + i % 4.
    v16f s_next;
    float x[16];
    float tmax = -__builtin_huge_valf(), tm_o = 0.f, pm = 0.f, pm_o = 0.f, bias = 0.f, lsum = 0.f;
    int m_cand = m_run, kp_own = 0;
    v4i phi_own = {0, 0, 0, 0}, plo_own = {0, 0, 0, 0};
    auto slice = [&](int k) {
      if (k == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v4f sc4;
          if (ROWSCALE) sc4 = *(const v4f*)&rsc[st][32 * mm + 8 * j + 4 * g];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) x[4 * j + ii] = ROWSCALE ? s_cur[4 * j + ii] * sc4[ii] : s_cur[4 * j + ii];
        }
      } else if (k == 1) {
        // slots not read get -inf (after the row scale, which is 0 for them);
        // the branch is wave-uniform and taken only by ragged tiles
        if (mk != 0xFFFFFFFFu) {
          const u32 m0 = mk >> (4 * g);
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = ((m0 >> (8 * (i >> 2) + (i & 3))) & 1u) ? x[i] : -__builtin_huge_valf();
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, x[i]);
      } else if (k == 2) {
        tm_o = shfl_xor32(tmax);
      } else if (k == 3) {
        tmax = fmaxf(tmax, tm_o) * c2;  // log2 domain, this wave's keys
        m_cand = tmax > (float)(m_run + kLazy) ? (int)__builtin_ceilf(tmax) : m_run;
        const float msub = (float)m_cand;
        if (!ROWSCALE) {
          pm = __builtin_amdgcn_exp2f(tmax - msub);
        } else {
          // largest p * row scale of the wave's keys, in the log2 domain:
          // max(x c2 + log2 scale) - m, one exp2 instead of sixteen
          float lm = -__builtin_huge_valf();
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v4f ls4 = *(const v4f*)&lrs[st][32 * mm + 8 * j + 4 * g];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) lm = fmaxf(lm, fmaf(x[4 * j + ii], c2, ls4[ii]));
          }
          pm = __builtin_amdgcn_exp2f(lm - msub);
          pm_o = shfl_xor32(pm);
        }
      } else if (k == 4) {
        if (ROWSCALE) pm = fmaxf(pm, pm_o);
        kp_own = fit_exponent(pm);
        kp_own = kp_own < -127 ? -127 : (kp_own > 122 ? 122 : kp_own);
        bias = (float)kp_own - (float)m_cand;
      } else {
        const int d = k - 5;  // keys of register group d
        float y[4];
        v4f sc4;
        if (ROWSCALE) sc4 = *(const v4f*)&rsc[st][32 * mm + 8 * d + 4 * g];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          y[bb] = __builtin_amdgcn_exp2f(fmaf(x[4 * d + bb], c2, bias));
          if (!(SINGLE && !ROWSCALE)) lsum += y[bb];
          if (ROWSCALE) y[bb] *= sc4[bb];
        }
        int h = cvt_fp8x2<false>(y[0], y[1], 0);
        h = cvt_fp8x2<true>(y[2], y[3], h);
        phi_own[d] = h;
        if (SINGLE && !ROWSCALE) {
          // one FP8 term: normalise by the weights as rounded, so that a
          // single key returns its row exactly
          const v2f r01 = fp8x2_to_f32<false>(h), r23 = fp8x2_to_f32<true>(h);
          lsum += (r01[0] + r01[1]) + (r23[0] + r23[1]);
        }
        if (!SINGLE) {
          const v2f h01 = fp8x2_to_f32<false>(h), h23 = fp8x2_to_f32<true>(h);
          int lo;
          if (ROWSCALE) {
            lo = cvt_fp8x2_x16<false>(y[0] - h01[0], y[1] - h01[1], 0);
            lo = cvt_fp8x2_x16<true>(y[2] - h23[0], y[3] - h23[1], lo);
          } else {
            lo = cvt_fp8x2<false>(y[0] - h01[0], y[1] - h01[1], 0);
            lo = cvt_fp8x2<true>(y[2] - h23[0], y[3] - h23[1], lo);
          }
          plo_own[d] = lo;
        }
      }
    };

    if (active && tile + 1 < ntiles) {
      const SMLA_LDS uint8_t* tn = (const SMLA_LDS uint8_t*)kvs[(tile + 1) % kNS];
      v8i ka = read_k(tn, kb0, kb1, 0, mm);
#pragma unroll
      for (int ks = 0; ks < 9; ++ks) {
        v8i kn;
        if (ks < 8) kn = read_k(tn, kb0, kb1, ks + 1, mm);
        // q hi and lo stay in AGPRs for the whole token; an empty asm that
        // reads and writes them in place at their use makes the MFMAs read
        // those registers directly (without it the allocator copied both
        // operands every step: 80 moves and 97 reads per tile)
        asm volatile("" : "+a"(qhi[ks]));
        s_next = ks == 0 ? mfma_fp8(ka, qhi[0], v16f{}, 127, sq_hi) : mfma_fp8(ka, qhi[ks], s_next, 127, sq_hi);
        __builtin_amdgcn_sched_barrier(0);
        slice(ks);
        __builtin_amdgcn_sched_barrier(0);
        if (!SINGLE) asm volatile("" : "+a"(qlo[ks]));
        if (!SINGLE) s_next = mfma_fp8(ka, qlo[ks], s_next, 127, sq_lo);
        gather_chunk_at<WIDE>(kv_rsrc, gdst, wave, gro, ks);
        __builtin_amdgcn_sched_barrier(0);
        if (ks < 8) ka = kn;
      }
    } else {
#pragma unroll
      for (int c = 0; c < kRowGranules / 4; ++c) gather_chunk_at<WIDE>(kv_rsrc, gdst, wave, gro, c);
      if (active) {
#pragma unroll
        for (int k = 0; k < 9; ++k) slice(k);
      }
    }

    if (active) {
      // the own row sum moves to the wave's new running max (O follows after
      // the exchange, together with the partner's max)
      l_own = shift_down(l_own, m_run - m_cand);
      m_run = m_cand;
      l_own += lsum * __builtin_amdgcn_ldexpf(1.0f, -kp_own);
      // (3) publish this wave's P quarter (its heads x its keys) and exponents
      *(SMLA_LDS v4i*)&pex[wave][0][lane][0] = phi_own;
      if (!SINGLE) *(SMLA_LDS v4i*)&pex[wave][1][lane][0] = plo_own;
      if (g == 0) {
        sex[wave][hl][0] = m_run;
        sex[wave][hl][1] = kp_own;
      }
    }
    __syncthreads();

    // (4) O^T[128 columns x 64 heads] += V^T . P^T over all 64 keys: every
    // wave takes output columns 128 wave .. 128 wave + 127 of both head
    // blocks, so each V^T fragment read feeds four MFMAs.  Head block b's
    // P^T: k-block 0 = the keys of wave 2 b, k-block 1 = those of wave 2 b + 1;
    // the scale of k-block g comes from this lane's half g.
    {
      // a group of at most 32 heads runs block 1 on zero P (no branch in the
      // MFMA sequence); its output is never stored
      int sp_hi[2] = {127, 127}, sp_lo[2] = {127, 127};
      v8i ph[2] = {}, pl[2] = {};
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (b == 1 && !blk1) continue;
        const int m0 = sex[2 * b][hl][0], k0 = sex[2 * b][hl][1];
        const int m1 = sex[2 * b + 1][hl][0], k1 = sex[2 * b + 1][hl][1];
        const int m_new = m0 > m1 ? m0 : m1;
        const int e = 127 - (g ? k1 : k0) + ((g ? m1 : m0) - m_new);
        sp_hi[b] = e8m0(e);
        sp_lo[b] = e8m0(e - (ROWSCALE ? 4 : 0));
        const v4i h0 = *(const SMLA_LDS v4i*)&pex[2 * b][0][lane][0];
        const v4i h1 = *(const SMLA_LDS v4i*)&pex[2 * b + 1][0][lane][0];
        ph[b] = v8i{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        if (!SINGLE) {
          const v4i l0 = *(const SMLA_LDS v4i*)&pex[2 * b][1][lane][0];
          const v4i l1 = *(const SMLA_LDS v4i*)&pex[2 * b + 1][1][lane][0];
          pl[b] = v8i{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        }
        // move block b to the pair's common max (an exact power-of-two shift)
        const int d = m_o[b] - m_new;  // <= 0
        if (__any(d < 0)) {
          asm volatile("" ::: "memory");  // a real branch: the rescale is rare and long
#pragma unroll
          for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[b][c][i] = shift_down(o[b][c][i], d);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        m_o[b] = m_new;
      }
      if (active) {
        l_own = shift_down(l_own, m_run - m_o[pair]);
        m_run = m_o[pair];
      }

      const SMLA_LDS uint8_t* tb = (const SMLA_LDS uint8_t*)kvs[st];
      const u32 vb = v_base(lane, 0);
      v8i va = read_vt(tb, vb, 4 * wave);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int gnb = 4 * wave + c;  // global output block
        v8i vn;
        if (c < 3) vn = read_vt(tb, (gnb + 1) & 1 ? (vb ^ 32u) : vb, gnb + 1);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          o[b][c] = mfma_fp8(va, ph[b], o[b][c], 127, sp_hi[b]);
          if (!SINGLE) o[b][c] = mfma_fp8(va, pl[b], o[b][c], 127, sp_lo[b]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (c < 3) va = vn;
      }
      if (active && tile + 1 < ntiles) s_cur = s_next;
    }
  }

  // ---- epilogue: row sums of each head block (both waves of its pair),
  // then normalise (sink in the denominator only) and store bf16, or hand the
  // run result to the combine
  wait_vmem_all();
  l_own += shfl_xor32(l_own);  // a lane summed half of its wave's keys
  if (active && g == 0) lex[wave][hl] = l_own;
  __syncthreads();
  float l_tot[2] = {0.f, 0.f}, inv[2] = {0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b == 1 && !blk1) continue;
    const int hb = hg * 64 + 32 * b + hl;  // this lane's head of block b
    const bool ok = 32 * b + hl < gh;
    const bool any_key = m_o[b] != kNoMax;
    l_tot[b] = lex[2 * b][hl] + lex[2 * b + 1][hl];
    if (p.splits == 1 && p.sink != nullptr && ok && any_key)
      l_tot[b] += __builtin_amdgcn_exp2f(p.sink[hb] * kLog2e - (float)m_o[b]);
    inv[b] = (any_key && l_tot[b] > 0.f) ? 1.0f / l_tot[b] : 0.f;
  }
  if (p.splits > 1) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if ((b == 1 && !blk1) || 32 * b + hl >= gh) continue;
      const size_t row = (size_t)ur * p.H + (size_t)(hg * 64 + 32 * b + hl);
      float* po = p.part_o + row * kV + 128 * wave;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(v4f*)(po + 32 * c + 8 * j + 4 * g) =
              v4f{o[b][c][4 * j], o[b][c][4 * j + 1], o[b][c][4 * j + 2], o[b][c][4 * j + 3]};
      if (wave == 0 && g == 0) {
        const bool any_key = m_o[b] != kNoMax;
        *(float2*)(p.part_ml + 2 * row) =
            float2{any_key ? (float)m_o[b] : -__builtin_huge_valf(), any_key ? l_tot[b] : 0.f};
      }
    }
    return;
  }
  // stage the group's bf16 rows (1 KiB per head) in LDS, 1040 bytes apart,
  // then write each row with one coalesced 16-byte-per-lane store
  constexpr u32 kPitch = 1040;
  static_assert(kNS * kTileBytes >= 64 * kPitch, "staging room");
  uint8_t* const stage = &kvs[0][0];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b == 1 && !blk1) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32 n = 128u * (u32)wave + 32u * (u32)c + 8u * (u32)j + 4u * (u32)g;
        const v2i w = {(int)pack_bf16x2(o[b][c][4 * j] * inv[b], o[b][c][4 * j + 1] * inv[b]),
                       (int)pack_bf16x2(o[b][c][4 * j + 2] * inv[b], o[b][c][4 * j + 3] * inv[b])};
        *(SMLA_LDS v2i*)((SMLA_LDS uint8_t*)stage + (u32)(32 * b + hl) * kPitch + 2u * n) = w;
      }
  }
  __syncthreads();
  uint16_t* const obase = p.out + ((size_t)t * p.H + (size_t)(hg * 64)) * kV + 8 * lane;
  for (int r = 16 * wave; r < 16 * wave + 16 && r < gh; ++r) {
    const v4i v = *(const SMLA_LDS v4i*)((const SMLA_LDS uint8_t*)stage + (u32)r * kPitch + 16u * (u32)lane);
    store_stream(obase + (size_t)r * kV, v);
  }
}

}  // namespace

hipError_t launch_fp8pair(const AttnParams& p, hipStream_t stream) {
  const int HG = (p.H + 63) / 64;
  dim3 grid((unsigned)(p.T * p.splits * HG)), block(256);
  const int v = (p.sbs != 0 ? 1 : 0) | (p.single_pass ? 2 : 0) | (p.wide_pool ? 4 : 0);
  switch (v) {
    case 0: hipLaunchKernelGGL((smla_fp8pair_kernel<false, false, false>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((smla_fp8pair_kernel<true, false, false>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((smla_fp8pair_kernel<false, true, false>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((smla_fp8pair_kernel<true, true, false>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((smla_fp8pair_kernel<false, false, true>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((smla_fp8pair_kernel<true, false, true>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((smla_fp8pair_kernel<false, true, true>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((smla_fp8pair_kernel<true, true, true>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace smla

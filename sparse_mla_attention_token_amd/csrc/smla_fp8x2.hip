// Sparse MLA prefill attention on gfx950 FP8 MFMA (unit scale and one scale
// per KV row).
//
// What is computed (page "mla_sm100_prefill_sparse_fp8", function
// description, Parameters and Args; page "mla_prefill_sparse_qkv_fp8" for the
// shared K/V latent): for token t and head h,
//   out[t,h,:] = sum_j softmax_j(scale * q[t,h,:] . k_j) v_j
// over the token's listed rows, k_j the 576-wide dequantised latent row and
// v_j its first 512 columns, with an optional per-head sink logit in the
// softmax denominator.
//
// Work decomposition: one workgroup per query token holds every head of that
// token (NW waves x 32 heads), so each gathered 64-row tile is read from L2 /
// HBM once and reused by all heads.  Per tile:
//   * the 64 rows are copied global->LDS (16 bytes per lane, no registers)
//     into a two-stage ring, one tile ahead of the compute; the index ->
//     page -> row translation of up to 2048 slots is done up front by the
//     whole workgroup into an LDS table;
//   * S^T[64 keys x 32 heads] = K . Q^T on v_mfma_scale_f32_32x32x64_f8f6f4
//     with keys on M (the score page "sparse_index_fp8_sm100" also puts keys
//     on the MMA M side), so a head's scores sit in one lane pair and the row
//     max needs a single cross-lane step;
//   * online softmax in the exp2 domain with a lazy rescale: the running max
//     only moves when a tile's max exceeds it by more than 2^8, and only then
//     is O rescaled (the "correction" step of the page "SM100MLA");
//   * O^T[512 x 32 heads] += V^T . P^T, V^T read from the same LDS bytes with
//     ds_read_b64_tr_b8 (the pages read V "mn-major" from the K buffer).
//
// Numerics.  K and V are used as stored (exact FP8).  q (bf16) and P (f32)
// are each split into two FP8 terms, x = hi + lo/16 with hi = fp8(x 2^e) and
// lo = fp8(16 (x 2^e - hi)); the power-of-two factors ride on the MFMA's E8M0
// operand scales, per head.  A bf16 q has 8 significant bits, so hi + lo
// holds it exactly (barring FP8 underflow below 2^-13 of the head's largest
// |q|); P keeps about 8 bits.  At unit scale the low term of P is taken
// without the factor 16 (one scale for both terms): its absolute error floor
// is then 2^-10 against a tile maximum in [128, 256), i.e. below 2^-17 of the
// row sum per key.  With row scales the factor stays: there the dominant
// p x scale of a row can sit many binades under the tile's largest value, and
// the factor keeps its residual out of FP8's subnormal range.  A single FP8
// pass for q or P does not meet the output tolerance.  The single-pass variant
// (SINGLE) keeps only the hi terms, i.e. q and P each as one FP8 operand as on
// the page "mla_prefill_sparse_qkv_fp8" (module description); it halves the
// MFMA work and is offered as an opt-in whose error is measured, not as the
// default.  In the one-scale-per-row mode the row scale multiplies the score
// column after QK^T and the P column before P.V.
#include "smla_device.h"
#include "smla_fp8_ops.h"
#include "smla_gather.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyRescale = 8.0f;  // log2 headroom before O is rescaled
constexpr int kChunkTiles = 32;       // 2048 slots translated at a time

// q_lo operand (B side of QK^T): row hl of the wave's 32-row block, granules
// 4 ks + 2 g + u, column stride 512 bytes.
__device__ __forceinline__ u32 q_base(int lane, int u) {
  const u32 hl = (u32)lane & 31u, g = (u32)lane >> 5;
  return (2u * g + (u32)u) * 512u + 16u * (hl ^ (4u * (((hl >> 3) & 1u) ^ (u32)u)));
}

__device__ __forceinline__ v8i read_qlo(const SMLA_LDS uint8_t* qb, u32 qb0, u32 qb1, int ks) {
  const u32 o = 2048u * (u32)ks;
  v4i a0 = lds_read_b128(qb + qb0 + o), a1 = lds_read_b128(qb + qb1 + o);
  return v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
}

// q_lo staging slot of head row hl in granule column gl (32 rows per column)
__device__ __forceinline__ u32 qlo_slot(u32 gl, u32 hl) { return hl ^ (4u * (((hl >> 3) ^ gl) & 1u)); }

template <int NW, int NS, bool ROWSCALE, bool SINGLE, bool WIDE>
__global__ __launch_bounds__(NW * 64, 1) void smla_fp8x2_kernel(AttnParams p) {
  constexpr int GD = NS - 1;       // gather distance (tiles in flight)
  constexpr int CT = kChunkTiles;  // tiles translated per chunk
  __shared__ __attribute__((aligned(1024))) uint8_t kvs[NS][kTileBytes];
  __shared__ u32 rowid[CT * kBK];  // pool rows of the current chunk
  __shared__ u32 vmask[CT * 2];     // 64-bit validity mask per tile
  __shared__ __attribute__((aligned(16))) float rsc[ROWSCALE ? NS : 1][kBK];
  // low FP8 term of q: per wave 32 head-rows x 36 granules, granule-major like
  // a KV tile (column stride 512 bytes), read exactly like the K operand
  __shared__ __attribute__((aligned(1024))) uint8_t qlo_lds[NW][32 * kQK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int u = xcd_token(blockIdx.x, p.T * p.splits);  // (token, run of slots)
  const int t = u / p.splits;
  const int sp = u - t * p.splits;

  // ---- Prologue.  Every load that needs only the token number goes out
  // before anything waits, oldest first: the sequence boundaries, the index
  // words of the first chunk of slots (read up to the run's end in the row;
  // the effective length masks them later), then q.  The waits that follow
  // then cover only the loads they need (the vector memory counter retires
  // in order), so the index -> page chain runs under the q load.
  int cu_next = 0x7fffffff;  // lane i: cu_seqlens[1 + i] (sequences 0..63)
  if (p.B <= 64 && 1 + lane <= p.B) cu_next = p.cu_seqlens[1 + lane];
  constexpr int kPer = CT / NW;  // first-chunk tiles per wave
  u32 ix0[kPer];
  {
    const u32 cap = (u32)p.split_tiles * (u32)kBK;
    const u32 s0 = (u32)sp * cap;
    const u32 run = (u32)p.K > s0 ? ((u32)p.K - s0 < cap ? (u32)p.K - s0 : cap) : 0u;
    const u32* row = p.indices + (size_t)t * p.K + s0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const u32 j = (u32)(wave + NW * r) * (u32)kBK + (u32)lane;
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

  const int hl = lane & 31;  // head within the wave (MFMA N column)
  const int g = lane >> 5;   // contraction half held by this lane
  const int head = wave * 32 + hl;
  const bool head_ok = head < p.H;

  // ---- Q, step 1: the wave's 32 head rows (32 x 1152 contiguous bytes) are
  // loaded 1 KiB per instruction (lane l of load k: bytes 1024 k + 16 l), so
  // every load covers 8 whole cache lines
  const int wave_heads = p.H - wave * 32 < 32 ? (p.H - wave * 32 > 0 ? p.H - wave * 32 : 0) : 32;  // uniform
  v4i ld[36];
  {
    const uint8_t* qw = (const uint8_t*)(p.q + ((size_t)t * p.H + (size_t)wave * 32) * kQK);
    if (wave_heads == 32) {
#pragma unroll
      for (int k = 0; k < 36; ++k) ld[k] = load_stream(qw + 16u * (64u * (u32)k + (u32)lane));
    } else {
#pragma unroll
      for (int k = 0; k < 36; ++k) {
        const u32 piece = 64u * (u32)k + (u32)lane;  // 16-byte piece of the wave's rows
        ld[k] = piece / 72u < (u32)wave_heads ? load_stream(qw + 16u * piece) : v4i{0, 0, 0, 0};
      }
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
    const int n0 = ntiles < CT ? ntiles : CT;
    int pg0[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = wave + NW * r;
      pg0[r] = i < n0 ? slot_page(ts, ga, i, lane, ix0[r]) : -1;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = wave + NW * r;
      if (i < n0) {
        const u32 j = (u32)i * (u32)kBK + (u32)lane;
        publish_slots(ga, j < ts.L ? ix0[r] : 0u, pg0[r], rowid + kBK * i, vmask + 2 * i, lane);
      }
    }
  }

  // ---- Q, step 2: through LDS into the MFMA operand layout.  Piece p of head
  // row h (p = 8 ks + 4 g + c: bf16 columns 64 ks + 32 g + 8 c .. +7) is what
  // lane h + 32 g reads with read 4 ks + c.  Read r occupies 1 KiB at
  // 1024 r, lane L at 16 (L ^ (r % 16)): each read is a lane permutation of
  // one 1 KiB line, and the 64 pieces one load writes fall on all 16 bank
  // positions.  The tile and q_lo buffers are free until the first gather.
  uint8_t* const qst = wave < 2 ? &kvs[0][0] + (u32)wave * 36864u : &qlo_lds[0][0] + (u32)(wave - 2) * 36864u;
  static_assert(NW == 4 && NS * kTileBytes >= 2 * 36864 && NW * 32 * kQK >= 2 * 36864, "q staging room");
#pragma unroll
  for (int k = 0; k < 36; ++k) {
    const u32 piece = 64u * (u32)k + (u32)lane;
    const u32 h = piece / 72u, pc = piece - 72u * h;
    const u32 r = 4u * (pc >> 3) + (pc & 3u), L = h + 32u * ((pc >> 2) & 1u);
    *(SMLA_LDS v4i*)((SMLA_LDS uint8_t*)qst + 1024u * r + 16u * (L ^ (r & 15u))) = ld[k];
  }
  v4i raw[9][4];
#pragma unroll
  for (int ks = 0; ks < 9; ++ks)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32 r = 4u * (u32)ks + (u32)c;
      raw[ks][c] = lds_read_b128((const SMLA_LDS uint8_t*)qst + 1024u * r + 16u * ((u32)lane ^ (r & 15u)));
    }
  __syncthreads();  // every wave is done with the staging area

  // ---- gather tiles 0..GD-1 (in flight while q is split)
  for (int tt = 0; tt < GD && tt < ntiles; ++tt) {
    gather_tile<NW, WIDE>(kv_rsrc, ga, rowid + kBK * (tt % CT), kvs[tt % NS], wave, lane);
    if (ROWSCALE && wave == 0) {
      const u32 row = rowid[kBK * (tt % CT) + lane];
      const u32 soff = row < p.num_rows ? row * 4u : p.scale_bytes;
      load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&rsc[tt % NS][0], soff);
    }
  }

  // ---- Q, step 3: split into FP8 hi/lo with a per-head power-of-two scale
  v8i qhi[9];
  int sq_hi, sq_lo;
  uint8_t* const qlo_w = qlo_lds[wave];
  {
    // largest |q| of the head from the raw bf16 magnitude bits (ordered like
    // the values for finite inputs), so no widened copy is kept live
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
    const float up = __builtin_amdgcn_ldexpf(1.0f, e);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const u32 d0 = (u32)raw[ks][c][2 * w2], d1 = (u32)raw[ks][c][2 * w2 + 1];
          const float x0 = __uint_as_float(d0 << 16) * up, x1 = __uint_as_float(d0 & 0xffff0000u) * up;
          const float x2 = __uint_as_float(d1 << 16) * up, x3 = __uint_as_float(d1 & 0xffff0000u) * up;
          int h = cvt_fp8x2<false>(x0, x1, 0);
          h = cvt_fp8x2<true>(x2, x3, h);
          const v2f h01 = fp8x2_to_f32<false>(h), h23 = fp8x2_to_f32<true>(h);
          int lo = cvt_fp8x2_x16<false>(x0 - h01[0], x1 - h01[1], 0);
          lo = cvt_fp8x2_x16<true>(x2 - h23[0], x3 - h23[1], lo);
          qhi[ks][2 * c + w2] = h;
          if (SINGLE) continue;
          // bytes 8c + 4 w2 .. +3 of this lane's slice = granule 4 ks + 2 g + c / 2
          const u32 gl = (u32)(4 * ks + 2 * g + (c >> 1));
          *(int*)(qlo_w + gl * 512u + 16u * qlo_slot(gl, (u32)hl) + 8u * (c & 1) + 4u * w2) = lo;
        }
  }

  // ---- softmax state (per lane: one head, half of each tile's keys)
  float m_run = kNegInf;  // running max, log2 domain
  float l_part = 0.f;     // partial row sum of exp2(s - m_run) over this lane's keys
  v16f o[16];
#pragma unroll
  for (int nb = 0; nb < 16; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[nb][i] = 0.f;

  wait_vmem_all();  // the first tiles landed
  __syncthreads();

  const float c2 = p.scale_log2;
  const u32 kvs_lds = lds_addr_of(kvs);

  const bool wave_active = wave * 32 < p.H;  // wave-uniform

  for (int tile = 0; tile < ntiles; ++tile) {
    const int st = tile % NS;
    // validity of this tile's 64 slots (read before a new chunk may reuse the table)
    const u32 mk0 = __builtin_amdgcn_readfirstlane(vmask[2 * (tile % CT)]);
    const u32 mk1 = __builtin_amdgcn_readfirstlane(vmask[2 * (tile % CT) + 1]);
    // (1) a new chunk of slots: translate it (the previous chunk's row
    // offsets were last read by the gather issued one iteration ago)
    if (tile + GD < ntiles && (tile + GD) % CT == 0) {
      __syncthreads();
      const int c0 = tile + GD;
      translate_chunk<NW, CT>(ts, ga, c0, ntiles - c0 < CT ? ntiles - c0 : CT, rowid, vmask, wave, lane);
      wait_vmem_all();
      __syncthreads();
    }
    // (2) gather tile + GD: the wave's 9 copies go out one per contraction
    // step below, so the texture path drains while the MFMAs run.  Past the
    // last tile they carry an out-of-range offset (zeros into the stage no
    // tile reads any more), which keeps that loop free of branches.
    const int tg = tile + GD;
    const u32 gdst = kvs_lds + (u32)(tg % NS) * (u32)kTileBytes;
    RowSrc<WIDE> gro = gather_no_src<WIDE>();  // past the last tile: zeros into a stage no tile reads
    if (tg < ntiles) {
      gro = gather_lane_src<WIDE>(ga, rowid + kBK * (tg % CT), wave, (int)opaque((u32)lane));
      if (ROWSCALE && wave == 0) {
        const u32 row = rowid[kBK * (tg % CT) + lane];
        const u32 soff = row < p.num_rows ? row * 4u : p.scale_bytes;
        load_to_lds<4>(sc_rsrc, (SMLA_LDS void*)&rsc[tg % NS][0], soff);
      }
    }

    if (!wave_active) {
      if (tg < ntiles)
        for (int ch = 0; ch < kRowGranules / 4; ++ch) gather_chunk_at<WIDE>(kv_rsrc, gdst, wave, gro, ch);
    } else {

    // (3) S^T = K . Q^T for the 64 keys of this tile.  Operand reads run one
    // contraction step ahead of the MFMAs; the scheduling fences keep the
    // compiler from hoisting all of them (and their registers) to the top.
    const SMLA_LDS uint8_t* tb = (const SMLA_LDS uint8_t*)kvs[st];
    const u32 kb0 = k_base((int)opaque((u32)lane), 0), kb1 = k_base((int)opaque((u32)lane), 1);
    v16f s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
    // q_lo: same lane pattern as K with a 512-byte granule column (rows = heads)
    const SMLA_LDS uint8_t* qb = (const SMLA_LDS uint8_t*)qlo_w;
    const u32 qb0 = q_base((int)opaque((u32)lane), 0), qb1 = q_base((int)opaque((u32)lane), 1);
    v8i ka0 = read_k(tb, kb0, kb1, 0, 0);
    v8i ka1 = read_k(tb, kb0, kb1, 0, 1);
    v8i ql;
    if (!SINGLE) ql = read_qlo(qb, qb0, qb1, 0);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      v8i kn0, kn1, qn;
      if (ks < 8) {
        kn0 = read_k(tb, kb0, kb1, ks + 1, 0);
        kn1 = read_k(tb, kb0, kb1, ks + 1, 1);
        if (!SINGLE) qn = read_qlo(qb, qb0, qb1, ks + 1);
      }
      // q_hi stays in AGPRs for the whole token.  Passing it through an empty
      // asm that reads and writes it in place, right at its use, makes the
      // MFMAs read those registers directly; without it the allocator split
      // the long live ranges and copied every step's 8 registers into a
      // scratch tuple first (72 copies per tile, and 6 spilled registers)
      asm volatile("" : "+a"(qhi[ks]));
      s0 = mfma_fp8(ka0, qhi[ks], s0, 127, sq_hi);
      s1 = mfma_fp8(ka1, qhi[ks], s1, 127, sq_hi);
      if (!SINGLE) {
        s0 = mfma_fp8(ka0, ql, s0, 127, sq_lo);
        s1 = mfma_fp8(ka1, ql, s1, 127, sq_lo);
      }
      gather_chunk_at<WIDE>(kv_rsrc, gdst, wave, gro, ks);
      __builtin_amdgcn_sched_barrier(0);
      if (ks < 8) {
        ka0 = kn0;
        ka1 = kn1;
        if (!SINGLE) ql = qn;
      }
    }

    // (4) online softmax.  Lane (head hl, half g) holds, in register i of
    // M-block mb, the score of key 32 mb + 8 (i / 4) + 4 g + i % 4.  Scores
    // are raw dot products here; the softmax scale (> 0) and, in the row-scale
    // mode, the row scale multiply them on the way into exp2.
    float x[2][16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v4f sc4;
        if (ROWSCALE) sc4 = *(const v4f*)&rsc[st][32 * mb + 8 * j + 4 * g];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 4 * j + ii;
          float sv = mb ? s1[i] : s0[i];
          if (ROWSCALE) sv *= sc4[ii];
          x[mb][i] = sv;
        }
      }
    }
    // slots that are not read get -inf (after the row scale, which is 0 for
    // them); the branch is wave-uniform and taken only by ragged tiles
    if ((mk0 & mk1) != 0xFFFFFFFFu) {
      const u32 m0 = mk0 >> (4 * g), m1 = mk1 >> (4 * g);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + (i & 3);  // key index minus 4 g
        x[0][i] = ((m0 >> key) & 1u) ? x[0][i] : kNegInf;
        x[1][i] = ((m1 >> key) & 1u) ? x[1][i] : kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, x[mb][i]);
    tmax = fmaxf(tmax, shfl_xor32(tmax)) * c2;  // log2 domain
    const bool upd = tmax > m_run + kLazyRescale;
    if (__any(upd)) {
      const float m_new = upd ? tmax : m_run;
      const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[nb][i] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float msub = (m_run == kNegInf) ? 0.f : m_run;
    // P is formed pre-multiplied by 2^kp so that its largest value sits in
    // [128, 256): y = exp2(s c2 + kp - m) (x row scale).  Without row scales
    // the tile's largest p is exp2(tmax - m) in closed form.
    int kp;
    if (!ROWSCALE) {
      kp = fit_exponent(__builtin_amdgcn_exp2f(tmax - msub));
    } else {
      // largest p * row_scale of the tile, key by key
      float pm = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f sc4 = *(const v4f*)&rsc[st][32 * mb + 8 * j + 4 * g];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float e = __builtin_amdgcn_exp2f(fmaf(x[mb][4 * j + ii], c2, -msub));
            pm = fmaxf(pm, e * sc4[ii]);
          }
        }
      pm = fmaxf(pm, shfl_xor32(pm));
      kp = fit_exponent(pm);
    }
    kp = kp < -127 ? -127 : (kp > 122 ? 122 : kp);
    const int sp_hi = 127 - kp, sp_lo = (ROWSCALE ? 123 : 127) - kp;
    const float bias = (float)kp - msub;
    // P^T operand bytes: byte 4d + b = key of (mb = d / 4, i = 4 (d % 4) + b)
    v8i phi, plo;
    float lsum = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int mb = d >> 2, i0 = 4 * (d & 3);
      float y[4];
      v4f sc4;
      if (ROWSCALE) sc4 = *(const v4f*)&rsc[st][32 * mb + 8 * (d & 3) + 4 * g];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        y[b] = __builtin_amdgcn_exp2f(fmaf(x[mb][i0 + b], c2, bias));
        lsum += y[b];
        if (ROWSCALE) y[b] *= sc4[b];
      }
      int h = cvt_fp8x2<false>(y[0], y[1], 0);
      h = cvt_fp8x2<true>(y[2], y[3], h);
      phi[d] = h;
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
        plo[d] = lo;
      }
    }
    l_part += lsum * __builtin_amdgcn_ldexpf(1.0f, -kp);

    // (5) O^T += V^T . P^T, V^T operands read one output block ahead.  The
    // empty asm makes the read base depend on P, so the compiler cannot
    // hoist the 64 transposed reads above the softmax and hold 128 registers.
    // odd output blocks flip granule bit 1: their base is vb ^ 32
    u32 vb = v_base(lane, 0);
    if (SINGLE) asm volatile("" : "+v"(vb) : "v"(phi));
    else asm volatile("" : "+v"(vb) : "v"(phi), "v"(plo));
    v8i va = read_vt(tb, vb, 0);
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      v8i vn;
      if (nb < 15) vn = read_vt(tb, (nb + 1) & 1 ? (vb ^ 32u) : vb, nb + 1);
      o[nb] = mfma_fp8(va, phi, o[nb], 127, sp_hi);
      if (!SINGLE) o[nb] = mfma_fp8(va, plo, o[nb], 127, sp_lo);
      __builtin_amdgcn_sched_barrier(0);
      if (nb < 15) va = vn;
    }

    }  // wave_active

    // (6) the gather of tile + GD landed
    wait_vmem_all();
    __syncthreads();
  }

  // ---- epilogue: normalise (sink in the denominator only) and store bf16,
  // or hand the unnormalised run result to the combine step
  float l_tot = l_part + shfl_xor32(l_part);
  if (p.splits > 1) {
    if (head_ok) {
      const size_t row = (size_t)u * p.H + head;
      float* po = p.part_o + row * kV;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(v4f*)(po + 32 * nb + 8 * j + 4 * g) = v4f{o[nb][4 * j], o[nb][4 * j + 1], o[nb][4 * j + 2], o[nb][4 * j + 3]};
      if (g == 0) *(float2*)(p.part_ml + 2 * row) = float2{m_run, l_tot};
    }
    return;
  }
  if (p.sink != nullptr && head_ok && m_run != kNegInf) l_tot += __builtin_amdgcn_exp2f(p.sink[head] * kLog2e - m_run);
  const float inv = (m_run != kNegInf && l_tot > 0.f) ? 1.0f / l_tot : 0.f;
  // The bf16 rows go through LDS (the tile and q_lo buffers are free once the
  // last tile is done): a lane holds 4-column pieces of one head's row, so
  // direct stores would touch 32 rows per instruction; from LDS every store
  // instruction writes one head's whole 1 KiB row.  Rows are 1040 bytes apart
  // in LDS (4 banks of skew) so that the 32 rows written at once do not
  // collide on one bank.
  constexpr u32 kPitch = 1040;
  static_assert(NW == 4 && NS * kTileBytes >= 2 * 32 * kPitch && NW * 32 * kQK >= 2 * 32 * kPitch, "staging room");
  uint8_t* const stage = wave < 2 ? &kvs[0][0] + (u32)wave * 32u * kPitch : &qlo_lds[0][0] + (u32)(wave - 2) * 32u * kPitch;
  if (wave_active) {
#pragma unroll
    for (int nb = 0; nb < 16; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32 n = 32u * (u32)nb + 8u * (u32)j + 4u * (u32)g;
        const v2i w = {(int)pack_bf16x2(o[nb][4 * j] * inv, o[nb][4 * j + 1] * inv),
                       (int)pack_bf16x2(o[nb][4 * j + 2] * inv, o[nb][4 * j + 3] * inv)};
        *(SMLA_LDS v2i*)((SMLA_LDS uint8_t*)stage + (u32)hl * kPitch + 2u * n) = w;
      }
  }
  __syncthreads();
  if (wave_active) {
    const int rows = p.H - wave * 32 < 32 ? p.H - wave * 32 : 32;  // wave-uniform
    uint16_t* const obase = p.out + ((size_t)t * p.H + (size_t)wave * 32) * kV + 8 * lane;
    for (int r = 0; r < rows; ++r) {
      const v4i v = lds_read_b128((const SMLA_LDS uint8_t*)stage + (u32)r * kPitch + 16u * (u32)lane);
      store_stream(obase + (size_t)r * kV, v);
    }
  }
}

template <int NS>
hipError_t launch_ns(const AttnParams& p, hipStream_t stream) {
  // Four waves (128 head slots) for every head count: with its LDS footprint
  // a workgroup holds a whole CU, so waves without heads cost no MFMA time;
  // they still help with the gather.
  constexpr int NW = 4;
  dim3 grid(p.T * p.splits), block(NW * 64);
  const int v = (p.sbs != 0 ? 1 : 0) | (p.single_pass ? 2 : 0) | (p.wide_pool ? 4 : 0);
  switch (v) {
    case 0: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, false, false, false>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, true, false, false>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, false, true, false>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, true, true, false>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, false, false, true>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, true, false, true>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, false, true, true>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((smla_fp8x2_kernel<NW, NS, true, true, true>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8x2(const AttnParams& p, hipStream_t stream) { return launch_ns<2>(p, stream); }

}  // namespace smla

// FP8 lightning indexer on gfx950: per-(query token, key) scores and the
// top-k selection that turns them into the attention's index lists.
//
// Scores (page "sparse_index_fp8_sm100", module description):
//   score[t, j] = k_scale[row_j] * sum_h relu(q[t, h, :] . k[row_j, :]) * q_scale[t, h]
// with q [T, H, 128] and the paged keys [keys, 128] in FP8 e4m3.  As on that
// page the depth-128 products run on the matrix cores with keys on one side
// and (token, head) on the other, and the head reduction happens in the
// epilogue: here D[32 heads x 32 keys] = Q . K^T on
// v_mfma_scale_f32_32x32x64_f8f6f4, so a lane holds 16 heads of one key and
// the head sum is 16 in-lane multiply-adds plus one cross-half add.  Each
// wave owns one query token (its Q fragments stay in registers); the four
// waves of a workgroup take four consecutive tokens and share every 64-key
// tile of K, staged global->LDS one tile ahead of the MFMAs.  Readings: the
// keys of a token are the causal prefix of its sequence (queries are the last
// positions of the sequence), score rows hold -inf past that prefix, and a
// page id outside the pool masks its key with -inf.
//
// Top-k: one workgroup per score row (held in registers when it fits), a
// four-pass radix select on an order-preserving 32-bit key of the f32 scores
// (the K-th largest value and how many of its ties to take), then one pass in
// key order that writes the chosen keys ascending, ties going to the lower
// key index.  NaN orders below -inf, -0 equals +0.
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

constexpr int kIdxDepth = 128;
constexpr int kKeyTile = 64;
constexpr u32 kKeyTileBytes = kKeyTile * kIdxDepth;  // 8 KiB

struct SeqInfo {
  int b;  // sequence (B when the token does not exist)
  int n;  // keys the token sees (causal prefix, clamped to the row stride)
};

__device__ __forceinline__ SeqInfo token_info(const IndexParams& p, int t) {
  SeqInfo s{p.B, 0};
  if (t >= p.T) return s;
  // the last sequence b with cu[b] <= t (binary search; t is wave-uniform)
  if (p.B <= 0 || p.cu_seqlens[0] > t || p.cu_seqlens[p.B] <= t) return s;
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu_seqlens[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  s.b = b;
  const int q0 = p.cu_seqlens[b], q_len = p.cu_seqlens[b + 1] - q0;
  const int pos = p.seq_lens_k[b] - q_len + (t - q0);
  int n = pos + 1;
  n = n < 0 ? 0 : n;
  s.n = n < p.stride ? n : p.stride;
  return s;
}

// Byte offset of logical key j of sequence b inside the key pool, or
// p.k_bytes when its page id is out of range.
__device__ __forceinline__ u32 key_offset(const IndexParams& p, int b, u32 j, bool* ok) {
  const u32 lp = j / (u32)p.P;
  int page = lp < (u32)p.max_pages ? p.page_table[(size_t)b * p.max_pages + lp] : -1;
  *ok = page >= 0 && page < p.num_pages;
  return *ok ? ((u32)page * (u32)p.P + j % (u32)p.P) * (u32)kIdxDepth : p.k_bytes;
}

// LDS position of granule G (16 bytes) of key row n in a staged tile: rows
// of 128 bytes, granules XOR-swizzled by n & 7 so that the B-operand reads
// (32 rows x one granule per half wave) spread over all 16 bank slots.
__device__ __forceinline__ u32 tile_pos(u32 n, u32 G) { return 128u * n + 16u * (G ^ (n & 7u)); }

template <int HB>
__global__ __launch_bounds__(256) void smla_index_score_kernel(IndexParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t ktile[2][kKeyTileBytes];
  __shared__ __attribute__((aligned(16))) float kscale[2][kKeyTile];
  __shared__ u32 kvalid[2][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = 4 * blockIdx.x;
  const int t = t0 + wave;
  const SeqInfo me = token_info(p, t);
  const int last = t0 + 3 < p.T ? t0 + 3 : p.T - 1;
  const int b_first = token_info(p, t0).b, b_last = token_info(p, last).b;

  const v4i k_rsrc = make_rsrc(p.k, p.k_bytes);
  const v4i s_rsrc = make_rsrc(p.k_scale, p.ks_bytes);
  const u32 tile_lds = lds_addr_of(ktile);
  const int m = lane & 31, g = lane >> 5;

  // Q fragments (A operand: row = head, bytes 0-15 = depth 16 g + j and
  // bytes 16-31 = depth 32 + 16 g + j of each 64-deep step) and head weights
  // (D rows 8 (i / 4) + 4 g + i % 4 of each 32-head block)
  v8i qa[HB][2];
  v4f qs[HB][4];
  if (me.b < p.B) {
    const uint8_t* qt = p.q + (size_t)t * p.H * kIdxDepth;
#pragma unroll
    for (int mb = 0; mb < HB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint8_t* src = qt + (size_t)(32 * mb + m) * kIdxDepth + 64 * ks + 16 * g;
        const v4i lo = *(const v4i*)src, hi = *(const v4i*)(src + 32);
        qa[mb][ks] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    const float* qst = p.q_scale + (size_t)t * p.H;
#pragma unroll
    for (int mb = 0; mb < HB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) qs[mb][j] = *(const v4f*)(qst + 32 * mb + 8 * j + 4 * g);
  } else {
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) {
      qa[mb][0] = qa[mb][1] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) qs[mb][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
  float* const srow = p.scores + (size_t)t * p.stride;

  // one pass per sequence among the workgroup's tokens
  for (int b = b_first; b <= b_last && b < p.B; ++b) {
    int seg_n = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const SeqInfo o = token_info(p, t0 + w);
      if (o.b == b && o.n > seg_n) seg_n = o.n;
    }
    const int ntiles = (seg_n + kKeyTile - 1) / kKeyTile;
    const bool active = me.b == b;

    // staging of tile kt into stage kt & 1: wave w copies rows 16 w .. 16 w + 15
    // (two 1 KiB copies), wave 0 also the 64 key scales and the validity mask
    auto stage_tile = [&](int kt) {
      const int st = kt & 1;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32 blk = 2u * (u32)wave + (u32)c;        // 1 KiB block = rows 8 blk .. 8 blk + 7
        const u32 n = 8u * blk + ((u32)lane >> 3);      // row in the tile
        const u32 G = ((u32)lane & 7u) ^ (n & 7u);      // granule landing at slot lane & 7
        const u32 j = (u32)kt * kKeyTile + n;
        bool ok;
        u32 off = key_offset(p, b, j, &ok);
        off = (j < (u32)seg_n && ok) ? off + 16u * G : p.k_bytes;
        load_to_lds_at<16>(k_rsrc, tile_lds + (u32)st * kKeyTileBytes + 1024u * blk, off);
      }
      if (wave == 0) {
        const u32 j = (u32)kt * kKeyTile + (u32)lane;
        bool ok;
        const u32 off = key_offset(p, b, j, &ok);
        const bool v = ok && j < (u32)seg_n;
        load_to_lds<4>(s_rsrc, (SMLA_LDS void*)&kscale[st][0], v ? (off / (u32)kIdxDepth) * 4u : p.ks_bytes);
        const unsigned long long mask = __ballot(v);
        if (lane == 0) {
          kvalid[st][0] = (u32)mask;
          kvalid[st][1] = (u32)(mask >> 32);
        }
      }
    };

    if (ntiles > 0) stage_tile(0);
    for (int kt = 0; kt < ntiles; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < ntiles) {
        stage_tile(kt + 1);
        if (wave == 0) wait_vmem_le<3>();
        else wait_vmem_le<2>();
      } else {
        wait_vmem_all();
      }
      __syncthreads();  // tile kt, its scales and mask are in LDS

      if (active) {
        const SMLA_LDS uint8_t* tb = (const SMLA_LDS uint8_t*)ktile[st];
        v16f d[2][HB];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32 n = 32u * (u32)nb + (u32)m;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const v4i lo = lds_read_b128(tb + tile_pos(n, 4u * (u32)ks + (u32)g));
            const v4i hi = lds_read_b128(tb + tile_pos(n, 4u * (u32)ks + 2u + (u32)g));
            const v8i kb = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int mb = 0; mb < HB; ++mb) {
              if (ks == 0) d[nb][mb] = mfma_fp8(qa[mb][0], kb, v16f{}, 127, 127);
              else d[nb][mb] = mfma_fp8(qa[mb][1], kb, d[nb][mb], 127, 127);
            }
          }
        }
        float tot[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          float acc = 0.f;
#pragma unroll
          for (int mb = 0; mb < HB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc = fmaf(fmaxf(d[nb][mb][i], 0.f), qs[mb][i >> 2][i & 3], acc);
          tot[nb] = acc + shfl_xor32(acc);
        }
        // lane l writes key 64 kt + l (its half g picks the 32-key block)
        const u32 key_local = (u32)lane;
        const u32 j = (u32)kt * kKeyTile + key_local;
        const u32 vm = kvalid[st][g];
        const bool valid = (vm >> m) & 1u;
        const float v = valid ? (g ? tot[1] : tot[0]) * kscale[st][key_local] : -__builtin_huge_valf();
        if (j < (u32)me.n) srow[j] = v;
      }
      __syncthreads();  // everyone is done with stage st before it is refilled
    }
  }

  // the rest of the row: keys past the causal prefix
  if (t < p.T) {
    for (int j = me.n + lane; j < p.stride; j += 64) srow[j] = -__builtin_huge_valf();
  }
}

// ---------------------------------------------------------------- top-k

constexpr int kTopkThreads = 512;

// order-preserving key of an f32 score: larger score -> larger key; NaN -> 0
// (below -inf), -0 -> +0
__device__ __forceinline__ u32 order_key(float f) {
  u32 u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix of a per-thread 0/1 flag over the workgroup, in thread
// order; also returns the total.  Uses `wsum` (one slot per wave).
__device__ __forceinline__ u32 block_scan_flag(bool flag, u32* wsum, u32* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const u32 below = (u32)__popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = (u32)__popcll(bal);
  __syncthreads();
  u32 before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const u32 c = wsum[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  __syncthreads();  // wsum may be reused right after
  *total = all;
  return before + below;
}

// R > 0: the row (at most R * kTopkThreads keys) is loaded once into
// registers, thread i holding keys i + kTopkThreads k; R = 0: every pass
// re-reads the row from memory.
template <int R>
__global__ __launch_bounds__(kTopkThreads) void smla_index_topk_kernel(IndexParams p) {
  // 16 copies of the 256-bin histogram, copy = lane % 16: the scores of a row
  // crowd into a few bins, and lanes of one wave adding to the same counter
  // serialise; with copies at most 4 lanes of a wave share one
  constexpr int kCopies = 16;
  __shared__ u32 hist[kCopies][256];
  __shared__ u32 total[4];
  __shared__ u32 wsum[kTopkThreads / 64];
  __shared__ u32 pick[3];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const SeqInfo me = token_info(p, t);
  const int n = me.n;
  const int K = p.K;
  uint32_t* const out = p.indices + (size_t)t * K;

  if (n <= K || K == 0) {
    for (int j = tid; j < K; j += kTopkThreads) out[j] = j < n ? (u32)j : 0xFFFFFFFFu;
    if (tid == 0) p.lengths[t] = (u32)(n < K ? n : K);
    return;
  }
  const float* row = p.scores + (size_t)t * p.stride;
  u32 keys[R > 0 ? R : 1];
  if constexpr (R > 0) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int e = tid + kTopkThreads * k;
      keys[k] = e < n ? order_key(row[e]) : 0u;
    }
  }

  // radix select of the K-th largest key, 8 bits per pass from the top
  u32 prefix = 0, mask = 0, remaining = (u32)K;
  const int copy = tid & (kCopies - 1);
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kCopies * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    if constexpr (R > 0) {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const u32 kk = keys[k];
        if (tid + kTopkThreads * k < n && (kk & mask) == prefix) atomicAdd(&hist[copy][(kk >> shift) & 255u], 1u);
      }
    } else {
      for (int e = tid; e < n; e += kTopkThreads) {
        const u32 kk = order_key(row[e]);
        if ((kk & mask) == prefix) atomicAdd(&hist[copy][(kk >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    // the bin holding the remaining-th largest key: threads 0..255 take bins
    // 255..0; an inclusive prefix over them counts the keys in that bin and
    // above, and exactly one thread sees the count cross `remaining`
    u32 c = 0, incl = 0;
    if (tid < 256) {
      const int lane = tid & 63;
#pragma unroll
      for (int cp = 0; cp < kCopies; ++cp) c += hist[cp][255 - tid];
      incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const u32 up = (u32)__shfl_up((int)incl, d);
        if (lane >= d) incl += up;
      }
      if (lane == 63) total[tid >> 6] = incl;  // per-wave sums
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < (tid >> 6); ++w) incl += total[w];
      if (incl >= remaining && incl - c < remaining) {
        pick[0] = (u32)(255 - tid);
        pick[1] = remaining - (incl - c);  // keys of this bin still to take
        pick[2] = c;                       // keys in this bin
      }
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    mask |= 255u << shift;
    remaining = pick[1];
    const bool whole_bin = pick[1] == pick[2];
    __syncthreads();  // pick is rewritten by the next pass
    if (whole_bin) break;  // every key of the bin is taken: no finer split needed
  }
  // The K-th largest key lies in the bucket of keys whose masked top bits
  // equal `prefix` (one exact key after four passes); `ties` keys of that
  // bucket are taken, lowest index first (all of them after an early exit).
  const u32 thr = prefix;
  const u32 ties = remaining;

  // emit in key order: blocks of kTopkThreads consecutive keys
  u32 written = 0, eq_seen = 0;
  auto emit_block = [&](int base, u32 k) {
    const int e = base + tid;
    const bool in = e < n;
    const u32 km = k & mask;
    const bool eq = in && km == thr;
    u32 eq_total;
    const u32 eq_rank = block_scan_flag(eq, wsum, &eq_total) + eq_seen;
    const bool take = in && (km > thr || (eq && eq_rank < ties));
    u32 take_total;
    const u32 pos = block_scan_flag(take, wsum, &take_total) + written;
    if (take && pos < (u32)K) out[pos] = (u32)e;
    written += take_total;
    eq_seen += eq_total;
  };
  if constexpr (R > 0) {
#pragma unroll
    for (int k = 0; k < R; ++k)
      if (kTopkThreads * k < n) emit_block(kTopkThreads * k, keys[k]);  // uniform guard
  } else {
    for (int base = 0; base < n; base += kTopkThreads) {
      const int e = base + tid;
      emit_block(base, e < n ? order_key(row[e]) : 0u);
    }
  }
  if (tid == 0) p.lengths[t] = (u32)K;
}

template <int HB>
hipError_t launch_scores_hb(const IndexParams& p, hipStream_t stream) {
  dim3 grid((unsigned)((p.T + 3) / 4)), block(256);
  hipLaunchKernelGGL((smla_index_score_kernel<HB>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores(const IndexParams& p, hipStream_t stream) {
  switch (p.H / 32) {
    case 1: return launch_scores_hb<1>(p, stream);
    case 2: return launch_scores_hb<2>(p, stream);
    case 3: return launch_scores_hb<3>(p, stream);
    case 4: return launch_scores_hb<4>(p, stream);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_index_topk(const IndexParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.T), block(kTopkThreads);
  // rows are at most `stride` keys long: hold them in registers when they fit
  if (p.stride <= 4 * kTopkThreads) hipLaunchKernelGGL(smla_index_topk_kernel<4>, grid, block, 0, stream, p);
  else if (p.stride <= 16 * kTopkThreads) hipLaunchKernelGGL(smla_index_topk_kernel<16>, grid, block, 0, stream, p);
  else if (p.stride <= 32 * kTopkThreads) hipLaunchKernelGGL(smla_index_topk_kernel<32>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(smla_index_topk_kernel<0>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla

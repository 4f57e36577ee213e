// Measurement probes for MI355X (gfx950): the matrix-core peak of the MFMA
// shapes the attention kernels use, and the rate of the attention's row
// gather (64 listed 576-byte latent rows per tile, copied global->LDS with
// the same swizzled copies) from HBM and from L2.  They give measured
// ceilings next to the published ones; they are not part of the attention.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/smla_probe.h"
#include "../csrc/smla_device.h"
#include "../csrc/smla_gather.h"

namespace {

using namespace smla;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Four independent accumulators per wave, back-to-back MFMAs with operands in
// registers; the sum of the accumulators leaves the kernel so nothing is
// optimised away.  KIND 0: v_mfma_scale_f32_32x32x64_f8f6f4 (FP8 e4m3, unit
// E8M0 scales), 1: v_mfma_f32_32x32x16_f16, 2: v_mfma_f32_32x32x16_bf16,
// 3: v_mfma_f32_16x16x32_f16, 4: v_mfma_f32_16x16x32_bf16.
template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma16_kernel(float* out, int64_t iters) {
  const int lane = threadIdx.x & 63;
  typedef typename std::conditional<KIND == 3, f16x8, bf16x8>::type T8;
  typedef typename std::conditional<KIND == 3, _Float16, __bf16>::type T;
  v4f acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = v4f{0.f, 0.f, 0.f, 0.f};
  T8 x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (T)(0.001f * (float)(lane + i));
    y[i] = (T)(0.002f * (float)(lane - i));
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if constexpr (KIND == 3) acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, acc[a], 0, 0, 0);
      else acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[a], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a) s += acc[a][0] + acc[a][1] + acc[a][2] + acc[a][3];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* out, int64_t iters) {
  const int lane = threadIdx.x & 63;
  v16f acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[a][i] = 0.f;
  if constexpr (KIND == 0) {
    v8i x, y;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = 0x38383838 ^ (lane * 7 + i);  // small e4m3 values
      y[i] = 0x30303030 ^ (lane * 3 + i);
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a] = mfma_fp8(x, y, acc[a], 127, 127);
    }
  } else {
    typedef typename std::conditional<KIND == 1, f16x8, bf16x8>::type T8;
    typedef typename std::conditional<KIND == 1, _Float16, __bf16>::type T;
    T8 x, y;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = (T)(0.001f * (float)(lane + i));
      y[i] = (T)(0.002f * (float)(lane - i));
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if constexpr (KIND == 1) acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, acc[a], 0, 0, 0);
        else acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[a], 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[a][i];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// One workgroup of four waves per block of tiles: each tile's 64 rows come
// from `rows` (row ids of the pool), the rows are copied into a
// two-stage LDS ring exactly as the attention stages them (one row group per
// wave, nine 1 KiB copies per wave), one tile in flight while the previous
// one is checked in.  out[block] gets one byte of every tile so the copies
// are consumed.
__global__ __launch_bounds__(256, 1) void probe_gather_kernel(const uint8_t* pool, uint32_t pool_rows,
                                                              const uint32_t* rows, int tiles_per_block,
                                                              uint32_t* out) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2][kTileBytes];
  __shared__ u32 ro[2][kBK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  GatherArgs ga{};
  ga.kv = pool;
  ga.num_rows = pool_rows;
  const uint32_t* my = rows + (size_t)blockIdx.x * tiles_per_block * kBK;
  u32 acc = 0;
  if (wave == 0) ro[0][lane] = my[lane];
  __syncthreads();
  gather_tile<4, true>(v4i{}, ga, ro[0], ring[0], wave, lane);
  for (int t = 0; t < tiles_per_block; ++t) {
    const int st = t & 1;
    if (t + 1 < tiles_per_block) {
      if (wave == 0) ro[st ^ 1][lane] = my[(size_t)(t + 1) * kBK + lane];
      __syncthreads();
      gather_tile<4, true>(v4i{}, ga, ro[st ^ 1], ring[st ^ 1], wave, lane);
      wait_vmem_le<9>();  // this wave's copies of tile t have landed
    } else {
      wait_vmem_all();
    }
    __syncthreads();
    acc += ring[st][threadIdx.x * 16];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

// Issue behaviour of a SIMD: does VALU work run while the matrix pipe is
// busy?  One workgroup per CU, cycles (s_memtime, shader clock) per
// iteration of each wave.  MODE 0: one wave per SIMD, one dependent FP8
// 32x32x64 MFMA chain with N independent FMAs after every MFMA.  MODE 1: one
// wave per SIMD, two independent chains alternating, N FMAs after every
// MFMA.  MODE 2: two waves per SIMD, waves 0-3 run the MFMA chain alone and
// waves 4-7 run N FMAs per iteration alone.
template <int MODE, int N>
__global__ __launch_bounds__(512, 1) void probe_coexec_kernel(int iters, unsigned long long* cycles, float* out) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + lane;
    b[i] = 0x30303030 + i;
  }
  v16f acc0 = {}, acc1 = {};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 1.0f + 0.001f * (float)(lane + i);
  const float c = 0.999f, d = 0.0001f;
  auto fmas = [&]() {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[i]) : "v"(c), "v"(d));
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mfma = [&](v16f& acc) {
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
    __builtin_amdgcn_sched_barrier(0);
  };
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  if (MODE == 0 && wave < 4) {
    for (int it = 0; it < iters; ++it) {
      mfma(acc0);
      fmas();
    }
  } else if (MODE == 1 && wave < 4) {
    for (int it = 0; it < iters; ++it) {
      mfma(acc0);
      fmas();
      mfma(acc1);
      fmas();
    }
  } else if (MODE == 2 && wave < 4) {
    for (int it = 0; it < iters; ++it) mfma(acc0);
  } else if (MODE == 2) {
    for (int it = 0; it < iters; ++it) fmas();
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += acc0[i] + acc1[i] + x[i];
  const int w = blockIdx.x * 8 + wave;
  if (lane == 0) {
    out[w] = sum;
    cycles[w] = t1 - t0;
  }
}

}  // namespace

extern "C" {

int smla_probe_mfma(int kind, int64_t iters, int blocks, float* out, void* stream) {
  if (kind < 0 || kind > 4 || iters < 1 || blocks < 1 || !out) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (kind == 0) hipLaunchKernelGGL(probe_mfma_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters);
  else if (kind == 1) hipLaunchKernelGGL(probe_mfma_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters);
  else if (kind == 2) hipLaunchKernelGGL(probe_mfma_kernel<2>, dim3(blocks), dim3(256), 0, s, out, iters);
  else if (kind == 3) hipLaunchKernelGGL(probe_mfma16_kernel<3>, dim3(blocks), dim3(256), 0, s, out, iters);
  else hipLaunchKernelGGL(probe_mfma16_kernel<4>, dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int64_t smla_probe_mfma_flop(int kind, int64_t iters, int blocks) {
  const int64_t per = kind == 0 ? 2ll * 32 * 32 * 64 : (kind <= 2 ? 2ll * 32 * 32 * 16 : 2ll * 16 * 16 * 32);
  return (int64_t)blocks * 4 * iters * 4 * per;
}

int smla_probe_gather(const void* pool, uint64_t pool_bytes, const uint32_t* rows, int tiles_per_block, int blocks,
                      uint32_t* out, void* stream) {
  if (!pool || !rows || !out || tiles_per_block < 1 || blocks < 1) return 1;
  if (pool_bytes / kQK > 0xFFFFFFFFull) return 3;
  if ((reinterpret_cast<uintptr_t>(pool) & 15) != 0) return 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(probe_gather_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint8_t*>(pool),
                     (uint32_t)(pool_bytes / kQK), rows, tiles_per_block, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int smla_probe_coexec(int mode, int valu, int64_t iters, int blocks, unsigned long long* cycles, float* out,
                      void* stream) {
  if (mode < 0 || mode > 2 || iters < 1 || iters > 0x7FFFFFFF || blocks < 1 || !cycles || !out) return 1;
  if (valu != 0 && valu != 4 && valu != 8 && valu != 16) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 g((unsigned)blocks), t(512);
#define SMLA_COEXEC(M, V) hipLaunchKernelGGL((probe_coexec_kernel<M, V>), g, t, 0, s, (int)iters, cycles, out)
#define SMLA_COEXEC_V(M)                \
  if (valu == 0) SMLA_COEXEC(M, 0);     \
  else if (valu == 4) SMLA_COEXEC(M, 4); \
  else if (valu == 8) SMLA_COEXEC(M, 8); \
  else SMLA_COEXEC(M, 16);
  if (mode == 0) { SMLA_COEXEC_V(0) }
  else if (mode == 1) { SMLA_COEXEC_V(1) }
  else { SMLA_COEXEC_V(2) }
#undef SMLA_COEXEC_V
#undef SMLA_COEXEC
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"

// Combine step of the split top-k launch.
//
// With few query tokens (decode and multi-token prediction) one workgroup per
// token leaves most CUs idle (the indexer page "sparse_index_fp8_sm100",
// Grid, likewise cuts work into extra slices when its grid underfills the
// machine), so the token's listed slots are cut into runs and each run gets
// its own workgroup, which leaves the run's unnormalised result: numerator
// O_s (in units of 2^-m_s), running max m_s (log2 domain) and row sum l_s.
// The softmax over the whole list is then the log-sum-exp merge the online
// softmax already does tile by tile (the correction step of page "SM100MLA"):
//   m = max_s m_s,  w_s = 2^(m_s - m),
//   out = sum_s w_s O_s / (sum_s w_s l_s [+ 2^(sink log2 e - m)]).
// Runs without a valid slot (l_s = 0) carry no weight; a token without any
// valid slot gets zeros, with or without a sink.
#include "smla_device.h"
#include "smla_kernels.h"

namespace smla {

namespace {

// One 128-thread half of a block per (token, head), four columns per thread.
__global__ __launch_bounds__(256) void smla_combine_kernel(AttnParams p) {
  const int idx = blockIdx.x * 2 + (int)(threadIdx.x >> 7);
  if (idx >= p.T * p.H) return;
  const int t = idx / p.H;
  const int h = idx - t * p.H;
  const int c = 4 * (int)(threadIdx.x & 127u);
  const int S = p.splits;
  const float2* ml = (const float2*)p.part_ml;

  float m = -__builtin_huge_valf();
  for (int s = 0; s < S; ++s) {
    const float2 v = ml[(size_t)(t * S + s) * p.H + h];
    if (v.y > 0.f) m = fmaxf(m, v.x);
  }
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  const bool any = m != -__builtin_huge_valf();
  if (any) {
    for (int s = 0; s < S; ++s) {
      const size_t row = (size_t)(t * S + s) * p.H + h;
      const float2 v = ml[row];
      if (v.y > 0.f) {
        const float w = __builtin_amdgcn_exp2f(v.x - m);
        l += w * v.y;
        acc += w * *(const v4f*)(p.part_o + row * kV + c);
      }
    }
    if (p.sink != nullptr) l += __builtin_amdgcn_exp2f(p.sink[h] * kLog2e - m);
  }
  const float inv = (any && l > 0.f) ? 1.0f / l : 0.f;
  uint2 w;
  w.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(uint2*)(p.out + ((size_t)t * p.H + h) * kV + c) = w;
}

}  // namespace

hipError_t launch_combine(const AttnParams& p, hipStream_t stream) {
  const long long rows = (long long)p.T * p.H;
  dim3 grid((unsigned)((rows + 1) / 2)), block(256);
  hipLaunchKernelGGL(smla_combine_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace smla

/*
 * smla_probe.h -- measurement probes of libsmla_probe.so (not part of the
 * attention).  They measure, on the GPU they run on, the ceilings the
 * attention kernels are compared with: the matrix-core rate of the MFMA
 * shapes they use, and the rate of their row gather.
 *
 * Device pointers are owned by the caller; calls enqueue on `stream` (a
 * hipStream_t, NULL = default stream) and never synchronise.  Return 0 on
 * success, 1 for a bad argument, 3 for a pool of 4 GiB or more, 4 for a
 * misaligned pool, 5 when the launch fails.
 */
#ifndef SMLA_PROBE_H
#define SMLA_PROBE_H

#include <stdint.h>

#if defined(__GNUC__)
#define SMLA_PROBE_API __attribute__((visibility("default")))
#else
#define SMLA_PROBE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Back-to-back MFMAs, four independent accumulators per wave, `blocks`
 * workgroups of four waves, `iters` steps: kind 0 = FP8 e4m3 32x32x64 with
 * E8M0 scales (the attention's QK^T and P.V), 1 = FP16 32x32x16 (blockwise
 * scales), 2 = BF16 32x32x16, 3 = FP16 16x16x32, 4 = BF16 16x16x32.
 * out: f32 [blocks * 4], written. */
SMLA_PROBE_API int smla_probe_mfma(int kind, int64_t iters, int blocks, float* out, void* stream);

/* Dense FLOP one smla_probe_mfma call performs. */
SMLA_PROBE_API int64_t smla_probe_mfma_flop(int kind, int64_t iters, int blocks);

/* The attention's row gather alone: `blocks` workgroups, each copying
 * tiles_per_block tiles of 64 rows of 576 bytes global->LDS (two-stage ring,
 * the attention's swizzled copies).  rows: uint32 [blocks * tiles_per_block *
 * 64] row ids inside the pool (rows of 576 bytes; an id at or past
 * pool_bytes / 576 stages zeros; 16-byte aligned pool).  out: uint32 [blocks],
 * written. */
SMLA_PROBE_API int smla_probe_gather(const void* pool, uint64_t pool_bytes, const uint32_t* rows, int tiles_per_block,
                                     int blocks, uint32_t* out, void* stream);

/* Issue behaviour of a SIMD, one workgroup of eight waves per block (waves
 * w and w + 4 share a SIMD; in modes 0 and 1 waves 4-7 only time an empty
 * loop): mode 0 = one dependent FP8 32x32x64 MFMA chain per wave with `valu`
 * independent FMAs after every MFMA; mode 1 = two independent chains
 * alternating, `valu` FMAs after every MFMA; mode 2 = waves 0-3 run the MFMA
 * chain alone while waves 4-7 run `valu` FMAs per iteration alone.  valu is
 * 0, 4, 8 or 16.  cycles: uint64 [blocks * 8], each wave's s_memtime count
 * (shader clocks) over the loop; out: f32 [blocks * 8]; both written. */
SMLA_PROBE_API int smla_probe_coexec(int mode, int valu, int64_t iters, int blocks, unsigned long long* cycles,
                                     float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_PROBE_H */

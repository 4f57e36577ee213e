// Device building blocks for the gfx950 sparse MLA kernels.
//
// Data layout of one staged KV tile in LDS: 64 gathered latent rows of 576
// FP8 bytes (the shared K/V buffer of the page "mla_prefill_sparse_qkv_fp8":
// K reads all 576 columns, V the first 512 of the same bytes), in 36 blocks
// of 1 KiB.  Block 4 ch + rg holds rows 16 rg .. 16 rg + 15 (row group rg)
// and granules 4 ch .. 4 ch + 3 (16-byte granules, chunk ch of 64 bytes):
//   offset(r, G) = 1024 (4 (G >> 2) + (r >> 4)) + 16 (4 (r & 15) + ((G & 3) ^ h(r & 15))),
//   h(q)         = ((q >> 1) & 3) ^ (3 ((q >> 3) & 1)).
// One wave-wide 16-byte-per-lane global->LDS copy fills one block, each
// group of four lanes fetching one 64-byte line of one row (lane order within
// the line permuted by h), which the texture path serves about twice as fast
// as 64 lanes on 64 different rows.  h keeps the row-wise K operand reads
// (16 consecutive rows of one granule) and the transposed V operand reads
// (8 rows x 2 granules per 32 lanes) free of LDS bank conflicts for both 32
// and 64 banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef uint32_t u32;

constexpr int kQK = 576;           // latent width (512 nope + 64 rope)
constexpr int kV = 512;            // value width
constexpr int kBK = 64;            // keys per tile
constexpr int kRowGranules = 36;   // 576 / 16
constexpr int kTileBytes = kBK * kQK;  // 36864
constexpr float kLog2e = 1.4426950408889634f;

#define SMLA_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- layout
// granule position swizzle of row q (0..15) of a row group
__device__ __forceinline__ u32 tile_h(u32 q) { return ((q >> 1) & 3u) ^ (3u * ((q >> 3) & 1u)); }

// byte offset of (row, 16-byte granule G) inside a staged tile
__device__ __forceinline__ u32 tile_off(u32 row, u32 G) {
  const u32 q = row & 15u;
  return 1024u * (4u * (G >> 2) + (row >> 4)) + 16u * (4u * q + ((G & 3u) ^ tile_h(q)));
}

// ---------------------------------------------------------------- buffers
// Raw buffer descriptor (gfx9 family: dword3 = 0x00020000).  Accesses at or
// beyond `nbytes` return zero; loads into LDS then write zeros.
__device__ __forceinline__ v4i make_rsrc(const void* base, u32 nbytes) {
  uint64_t p = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = (int)(u32)(p & 0xffffffffu);
  r[1] = (int)(u32)(p >> 32);
  r[2] = (int)nbytes;
  r[3] = 0x00020000;
  return r;
}

// One wave-wide global->LDS copy: lane i fetches `size` bytes at byte offset
// voff[i] of the buffer and writes them to lds_base + i * size (offsets past
// the buffer's size read as zero).  lds_base must be wave-uniform.
//
// Issued as inline assembly on purpose: the compiler then does not model the
// copy as an LDS store, so it adds no vmcnt(0) before later LDS reads of other
// buffers.  The caller owns the ordering: wait_vmem_all() then a workgroup
// barrier before anything reads the destination, and a barrier after the last
// read of the destination before the copy is issued.  Outstanding untracked
// copies can only make the compiler's own vmcnt waits stricter (vector memory
// loads complete in issue order), never looser.
// m0 is a reserved register to the compiler; nothing it generates here reads
// m0 (no other LDS-DMA, GWS or message instructions), so the clobber is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int SIZE>
__device__ __forceinline__ void load_to_lds(v4i rsrc, SMLA_LDS void* lds_base, u32 voff) {
  static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4 copies only");
  const u32 base = __builtin_amdgcn_readfirstlane((u32)(uintptr_t)lds_base);
  if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(base), "v"(voff), "s"(rsrc) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(base), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// The same copy with the LDS destination given as a wave-uniform LDS byte
// address (no pointer cast or lane read per copy).
template <int SIZE>
__device__ __forceinline__ void load_to_lds_at(v4i rsrc, u32 lds_addr, u32 voff) {
  static_assert(SIZE == 16, "dwordx4 copies only");
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// 16-byte global->LDS copy from a 64-bit address per lane (lane i writes
// lds_addr + 16 i): the latent pool is addressed this way, so its size is not
// bound by a buffer descriptor's 32-bit offsets.  Every address must be
// valid; same ordering rules as load_to_lds.
__device__ __forceinline__ void load_global_to_lds_at(u32 lds_addr, uint64_t addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_addr), "v"(addr) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wave-uniform LDS byte address of a __shared__ object.
__device__ __forceinline__ u32 lds_addr_of(const void* shared_obj) {
  return __builtin_amdgcn_readfirstlane((u32)(uintptr_t)(const SMLA_LDS void*)shared_obj);
}

// s_waitcnt vmcnt(0): every vector memory op of this wave (including the
// global->LDS copies) has completed.  expcnt/lgkmcnt fields left at 'no wait'.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): at most the N most recent vector memory ops of this
// wave are still in flight (N < 16).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// ---------------------------------------------------------------- streams
// Read-once / write-once global accesses (q rows, output rows) whose every
// instruction covers whole cache lines: non-temporal, so streaming them
// through L2 does not evict the gathered latent rows that the other query
// tokens of the same XCD read again (on the DSv3.2 prefill the L2 misses fell
// from 1.15 to 0.84 GB per call).  Loads that read a line over several
// instructions stay ordinary: a streamed line may be gone before the next.
__device__ __forceinline__ v4i load_stream(const void* p) { return __builtin_nontemporal_load((const v4i*)p); }
__device__ __forceinline__ void store_stream(void* p, v4i v) { __builtin_nontemporal_store(v, (v4i*)p); }
__device__ __forceinline__ void store_stream(void* p, v2i v) { __builtin_nontemporal_store(v, (v2i*)p); }

// ---------------------------------------------------------------- LDS reads
__device__ __forceinline__ v4i lds_read_b128(const SMLA_LDS uint8_t* p) { return *(const SMLA_LDS v4i*)p; }

// Transposed 8-bit read.  Within each 16-lane group, lane 2k+c supplies the
// address of 8 bytes (row k of an 8 x 16 byte block, column half c); lane j
// of the group receives column j of that block: byte k comes from row k.
__device__ __forceinline__ v2i lds_read_tr8(const SMLA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((SMLA_LDS v2i*)p);
}

// ---------------------------------------------------------------- MFMA
// D[32x32] += A[32x64] * B[64x32] on FP8 e4m3 operands with E8M0 block
// scales (127 = 1.0).  Lane l holds row (A) / column (B) l % 32 and half of
// the contraction; D lane l holds column l % 32, rows 8*(i/4) + 4*(l/32) + i%4.
__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// Opaque copy: the compiler cannot see through it, so values derived from the
// result are recomputed where they are used instead of being hoisted and kept
// live across a loop.
__device__ __forceinline__ u32 opaque(u32 x) {
  asm volatile("" : "+v"(x));
  return x;
}

// ---------------------------------------------------------------- numbers
// f32 pair -> two e4m3fn bytes (round to nearest even; values must already be
// within +-448, larger magnitudes become NaN) into the low or high half word.
template <bool HI>
__device__ __forceinline__ int cvt_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// The same for 16 a and 16 b (v_cvt_scalef32_pk_fp8_f32 divides by the
// scale's power of two): the low term of a two-term split without a multiply.
template <bool HI>
__device__ __forceinline__ int cvt_fp8x2_x16(float a, float b, int old) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, old), a, b, 0.0625f, HI);
  return __builtin_bit_cast(int, r);
}

// the two e4m3fn bytes in the low (HI = false) or high half word -> f32 pair
template <bool HI>
__device__ __forceinline__ v2f fp8x2_to_f32(int w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI); }

// a / s and b / s -> two e4m3fn bytes (round to nearest even) into the low or
// high half word, for s a power of two: the division only moves the exponent,
// so this is cvt_fp8x2(a / s, b / s, old) without the two multiplies
template <bool HI>
__device__ __forceinline__ int cvt_fp8x2_div(float a, float b, float s, int old) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, old), a, b, s, HI);
  return __builtin_bit_cast(int, r);
}

// the two e4m3fn bytes times s (a power of two, exact) -> f32 pair
template <bool HI>
__device__ __forceinline__ v2f fp8x2_to_f32_mul(int w, float s) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, s, HI);
}

// largest |x| of the two bf16 values in each dword, as a bf16 bit pattern
// (non-negative bf16 values order like their bit patterns): one mask and one
// packed 16-bit max per dword
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 bf16x2_absmax(u16x2 m, u32 two) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, two & 0x7FFF7FFFu));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((u32)b) << 16); }

// f32 pair -> packed bf16 pair (lo in the low half), round to nearest even
// (v_cvt_pk_bf16_f32)
__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(u32, __builtin_convertvector(v2f{lo, hi}, v2bf16));
}

// power-of-two exponent e with |x| * 2^e in [128, 256) (x != 0)
__device__ __forceinline__ int fit_exponent(float amax) {
  int e = 8 - __builtin_amdgcn_frexp_expf(amax);
  return amax > 0.f ? e : 0;
}

// x of lane i ^ 32 (every lane of the wave must be active).  With both
// operands x, v_permlane32_swap leaves x[i] and x[i ^ 32] in its two results
// (the low half holds the partner in the second, the high half in the first):
// a VALU exchange, no LDS round trip.
__device__ __forceinline__ float shfl_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32u) ? r[0] : r[1]);
}

// x of lane i ^ 16 (every lane of the wave must be active): v_permlane16_swap,
// the partner in the second result for even 16-lane rows, the first for odd.
__device__ __forceinline__ float shfl_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16u) ? r[0] : r[1]);
}

// ---------------------------------------------------------------- tokens
// Sequence of token t from cu_seqlens [B+1]: the number of offsets cu[1..B]
// that are <= t.  Returns B when t is not covered (caller treats it as empty).
__device__ __forceinline__ int token_sequence(const int32_t* cu, int B, int t) {
  int lane = threadIdx.x & 63;
  int count = 0;
  for (int base = 0; base < B; base += 64) {
    int i = base + 1 + lane;
    int v = (i <= B) ? cu[i] : 0x7fffffff;
    unsigned long long m = __ballot(v <= t);
    count += __popcll(m);
  }
  int c0 = cu[0];
  return (t < c0) ? B : count;
}

// XCD-aware block -> token map: blocks are dispatched round-robin over the 8
// XCDs, so give each XCD a contiguous range of tokens (tokens of a sequence
// share KV rows and therefore L2 lines).  Bijective on [0, T).
__device__ __forceinline__ int xcd_token(int i, int T) {
  int q = T >> 3, r = T & 7;
  int x = i & 7, s = i >> 3;
  return x * q + (x < r ? x : r) + s;
}

}  // namespace smla

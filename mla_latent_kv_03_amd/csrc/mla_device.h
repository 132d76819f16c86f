// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA wrappers,
// LDS transpose reads, direct global->LDS copies, wavefront reductions and the
// OCP E4M3 conversions used by the MLA decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// C[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) + j], B[8*(l/16) + j][l%16] (j = 0..7) and
// C[4*(l/16) + i][l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed 8-byte LDS read: in each 16-lane block, lanes 4r..4r+3 give the
// addresses of row r (4 x 4 consecutive 16-bit values = 16 columns); lane i of the
// block receives column i of the 4 rows.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Cache-policy bit "nt" (non-temporal) of gfx950 vector memory instructions.  For
// data streamed once it roughly doubles the HBM read rate of direct-to-LDS copies
// (measured on MI355X: about 3.9 -> 6.9 TB/s).
constexpr int kCachePolicyNT = 2;

// Cache-policy bits "sc0 sc1" (system scope) of a store: the data is written through the
// L2 instead of staying there dirty until the write-back at the end of the launch.  For
// output that a later launch reads, written at the end of a kernel, this moves the
// write-back off the launch's tail.
constexpr int kCachePolicyWriteThrough = 17;

// 16-byte store through a buffer resource: lane l writes base + voffset_l.
template <int kPolicy>
__device__ __forceinline__ void buffer_store16(u32x4 v, __amdgpu_buffer_rsrc_t rsrc, uint32_t voffset) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)voffset, 0, kPolicy);
}

// 16-byte global -> LDS copy without a register round trip: lane l's 16 bytes land
// at lds_wave_base + 16 * l (lds_wave_base must be wave-uniform).  Streaming policy.
__device__ __forceinline__ void global_to_lds16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (MLA_LDS void*)(lds_wave_base), 16, 0, kCachePolicyNT);
}

// The same copy through a buffer resource: lane l reads base + soffset + voffset_l.
// `base` and `soffset` must be wave-uniform.  The compiler tracks these (MUBUF) copies
// as ordinary vector-memory operations, whereas a global_load_lds in a loop makes it
// wait for every outstanding LDS read (lgkmcnt(0)) before the next LDS use, which
// defeats software prefetching of LDS operands.  `num_records` bounds voffset
// (bytes); a load past it reads nothing from memory and returns zeros, so a resource
// with num_records = 0 turns a copy into a no-op of the same instruction count.
constexpr int kBufferWord3 = 0x00020000;   // gfx9-family raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int num_records = 0x7fffffff) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, num_records, kBufferWord3);
}

__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t soffset,
                                                void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(lds_wave_base), 16, voffset, soffset, 0,
                                           kCachePolicyNT);
}

// A load through the scalar cache (the address must be wave-uniform, and the memory must
// not be written while the kernel runs): its wait is counted apart from the vector-memory
// operations, so it never waits for copies in flight.
__device__ __forceinline__ int32_t load_scalar(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)ptr;
}

// The same copy, 4 bytes per lane: lane l's 4 bytes land at lds_wave_base + 4 * l.
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t soffset,
                                               void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(lds_wave_base), 4, voffset, soffset, 0,
                                           kCachePolicyNT);
}

// Transposed 8-byte LDS read of 8-bit values: in each 16-lane block, lane 2r + q gives
// the address of bytes 8q .. 8q+7 of row r (8 rows of 16 bytes); lane i of the block
// receives byte i of rows 0..7, row r in byte r (lane layout measured on MI355X).
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ bf16x8 concat4(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x2 pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
}

// Four floats to bf16, round to nearest even.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  const bf16x2 a = pack_bf16(v[0], v[1]), b = pack_bf16(v[2], v[3]);
  return bf16x4{a[0], a[1], b[0], b[1]};
}

// Four bf16 to float (exact).
__device__ __forceinline__ f32x4 from_bf16x4(bf16x4 v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reductions across the four 16-lane rows of a wave with gfx950's row-swapping
// permutes (no LDS round trip).  permlane16_swap(v, v) yields rows (0,0,2,2) and
// (1,1,3,3); permlane32_swap(v, v) yields halves (lo,lo) and (hi,hi).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Two OCP E4M3 codes (bytes 0/1 or 2/3 of `packed`, selected by HI) -> two bf16,
// exactly (every E4M3 value is representable in bf16).
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(unsigned packed) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, HI);
}

// float -> OCP E4M3 code, round to nearest even, saturating to +-448, NaN -> 0x7F.
// Written from the format: 4 exponent bits (bias 7), 3 mantissa bits, subnormal
// quantum 2^-9, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7Fu;  // NaN
  float a = __uint_as_float(u & 0x7FFFFFFFu);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                                   // below 2^-6: quantum 2^-9
    uint32_t k = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling, RNE; k = 8 is 2^-6
    return sign | k;
  }
  int e = (int)((u >> 23) & 0xFFu) - 127;                // a in [2^e, 2^(e+1)), e in [-6, 8]
  uint32_t k = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8..16
  if (k == 16u) { e += 1; k = 8u; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | (k - 8u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

}  // namespace mla

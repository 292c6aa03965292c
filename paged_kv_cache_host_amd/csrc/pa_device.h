// Device-side helpers shared by the libpa kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 16;  // tokens per block of the staged and fused paths; decode, prefill
                             // and the cache write also take 8- and 32-token blocks (templated)
constexpr float kLog2e = 1.4426950408889634f;

// Storage tags: the element type of a buffer as the kernels see it.
struct F32 {
  using raw = float;
};
struct BF16 {
  using raw = uint16_t;
};
struct FP8 {
  using raw = uint8_t;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Two e4m3fn codes (bytes 0,1 or, with HI, 2,3 of `packed`) -> two exact floats.
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t packed, float& a, float& b) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(packed), HI);
  a = v[0];
  b = v[1];
}

__device__ __forceinline__ float fp8_to_f32(uint8_t c) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(c), 0);
}

// Eight e4m3fn codes (two dwords) -> eight bf16 (every e4m3fn value is
// exactly representable in bf16, so this is exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 w) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  bf16x8 r;
  r[0] = p0[0];
  r[1] = p0[1];
  r[2] = p1[0];
  r[3] = p1[1];
  r[4] = p2[0];
  r[5] = p2[1];
  r[6] = p3[0];
  r[7] = p3[1];
  return r;
}

// Eight e4m3fn codes -> eight fp16 (exact: every e4m3fn value is an fp16
// value).
__device__ __forceinline__ f16x8 fp8x8_to_f16x8(u32x2 w) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true);
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two bf16 (one dword) -> two fp16, rounding toward zero.  Exact for
// magnitudes in [2^-14, 65504]; smaller ones keep an absolute error below
// 2^-24 and larger finite ones saturate at 65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                 __uint_as_float(w & 0xFFFF0000u)));
}

// float -> e4m3fn code: nearest value, ties to even mantissa, |x| > 448
// saturates to 448, NaN stays NaN (0x7F with the sign).  Written from the
// format definition: 4 exponent bits of bias 7, 3 mantissa bits, subnormal
// quantum 2^-9, smallest normal 2^-6.
__device__ __forceinline__ uint8_t f32_to_e4m3_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return static_cast<uint8_t>(sign | 0x7Fu);
  if (a >= 448.0f) return static_cast<uint8_t>(sign | 0x7Eu);
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9, exact scaling by 2^9
    const float q = __builtin_rintf(a * 512.0f);  // round half to even
    return static_cast<uint8_t>(sign | static_cast<uint32_t>(q));
  }
  const uint32_t ua = __float_as_uint(a);
  // keep 3 of the 23 mantissa bits, round half to even on the 20 dropped
  const uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20;
  return static_cast<uint8_t>(sign | (r - (120u << 3)));  // rebias 127 -> 7
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Clamp a block-table entry into the pool: out-of-range entries read block 0
// so that no access leaves the cache buffers.
__device__ __forceinline__ int32_t safe_block(int32_t b, int32_t num_blocks) {
  return static_cast<uint32_t>(b) < static_cast<uint32_t>(num_blocks) ? b : 0;
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

}  // namespace pa

// Device helpers shared by the libdmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmoe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// ---------------------------------------------------------------------------
// bfloat16: the upper half of an IEEE binary32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round a float to bfloat16, nearest with ties to even, with v_cvt_pk_bf16_f32
// (identical to the integer RNE rule on every non-NaN binary32 pattern,
// denormals included; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats to a packed BF16 pair (lo in bits 0-15), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------------------
// OCP E4M3FN encode: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
// largest finite 448 (0x7E), smallest subnormal 2^-9; no infinities.
// Rounds |v| to the nearest representable magnitude with ties to the even
// code, saturates magnitudes >= 448 to 0x7E and copies the sign bit of v.
// Written from the format definition with integer operations on the binary32
// fields, so the result is identical on every device. Input must be finite.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t u = bits & 0x7fffffffu;
  uint32_t mag;
  if (u >= 0x43e00000u) {  // |v| >= 448
    mag = 0x7eu;
  } else {
    const int ef = (int)(u >> 23);       // binary32 exponent field
    const uint32_t mf = u & 0x7fffffu;   // binary32 mantissa field
    if (ef >= 127 - 6) {
      // E4M3 normal range: exponent >= -6. Keep 3 mantissa bits, round the 20 dropped.
      const uint32_t base = ((uint32_t)(ef - 127 + 7) << 3) | (mf >> 20);
      const uint32_t rem = mf & 0xfffffu;
      const uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (base & 1u));
      mag = base + up;  // a carry moves into the next binade, which is the right value
      if (mag > 0x7eu) mag = 0x7eu;
    } else if (ef == 0) {
      mag = 0;  // binary32 zero or subnormal: far below 2^-10
    } else {
      // E4M3 subnormal range: value = sig * 2^(ef-150); in units of 2^-9 that is sig >> (141 - ef).
      const uint32_t sig = mf | 0x800000u;
      const int shift = 141 - ef;  // >= 21 here
      if (shift >= 25) {
        mag = 0;  // below half of 2^-9... (sig < 2^24 <= 2^(shift-1))
      } else {
        const uint32_t q = sig >> shift;
        const uint32_t rem = sig & ((1u << shift) - 1u);
        const uint32_t half = 1u << (shift - 1);
        mag = q + ((rem > half) || (rem == half && (q & 1u)));
      }
    }
  }
  return sign | mag;
}

// E4M3FN code -> float (finite codes; 0x7F/0xFF decode as NaN).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  float mag;
  if (e == 0xfu && m == 7u) mag = __uint_as_float(0x7fc00000u);
  else if (e == 0) mag = (float)m * 0.001953125f;  // m * 2^-9
  else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// Wave-level helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_width(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, width));
  return v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)v, off);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src);
  const uint32_t hi = __shfl((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int off) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return __longlong_as_double((long long)shfl_xor_u64(b, off));
}

}  // namespace dmoe

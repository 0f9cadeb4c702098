// Device helpers for the gfx950 kernels: vector types, conversions, MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16. Operand lane layout (lane l, g = l / 16):
//   A (16 x 32): row l % 16, k = 8g + j for element j of the bf16x8;
//   B (32 x 16): column l % 16, k = 8g + j;
//   C/D (16 x 16, fp32): column l % 16, rows 4g + i for element i.
// The k order inside an operand is free as long as A and B agree; the kernels use that
// to feed MFMA outputs straight back in as operands without any transposition.
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float from_bf16(__bf16 x) { return (float)x; }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Split x into hi + lo, both bf16, with hi + lo = x to ~16 significant bits.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - from_bf16(hi));
}

__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  bf16x8 r;
  r[0] = to_bf16(a[0]); r[1] = to_bf16(a[1]); r[2] = to_bf16(a[2]); r[3] = to_bf16(a[3]);
  r[4] = to_bf16(b[0]); r[5] = to_bf16(b[1]); r[6] = to_bf16(b[2]); r[7] = to_bf16(b[3]);
  return r;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Logistic function with the fast exponential; -inf -> 0, +inf -> 1.
__device__ __forceinline__ float sigmoidf_fast(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace kda

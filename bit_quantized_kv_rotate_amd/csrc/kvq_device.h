// Device helpers shared by libkvq's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return as_f32((uint32_t)b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = as_u32(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16x2 (element 0 in the low half), round to nearest
// even; gfx950 has a single instruction for this.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// UE8M0 scale byte -> the fp32 whose exponent field the gfx950 scaled
// conversions read (value 2^(byte - 127)).
__device__ __forceinline__ float scale_operand(uint32_t byte) { return as_f32(byte << 23); }

// In-place orthonormal Walsh-Hadamard transform of `rows` rows of length d
// held in LDS (row stride d floats), fp32, radix-2 stages h = 1, 2, ..., d/2
// (x[j] + x[j+h], x[j] - x[j+h], one rounding each), then one multiply by c.
// All threads of the block take part; ends with a barrier.
__device__ __forceinline__ void fwht_rows_lds(float* x, int rows, int d, float c, int tid,
                                              int nthreads) {
  const int half = d >> 1;
  const int pairs = rows * half;
#pragma unroll 1
  for (int h = 1; h < d; h <<= 1) {
    for (int p = tid; p < pairs; p += nthreads) {
      const int r = p / half;
      const int q = p - r * half;
      const int i = (q / h) * (2 * h) + (q % h);
      float* row = x + r * d;
      const float a = row[i];
      const float b = row[i + h];
      row[i] = a + b;
      row[i + h] = a - b;
    }
    __syncthreads();
  }
  for (int p = tid; p < rows * d; p += nthreads) x[p] = x[p] * c;
  __syncthreads();
}

}  // namespace kvq

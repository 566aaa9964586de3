// Test harness (not part of libkvq): runs the append's own group encoders,
// encode_fp4_group and encode_fp8_group from kvq_append_dev.h, over arbitrary
// fp32 inputs at a given scale byte, so that a GPU test can compare every
// code with the CPU oracle's encoders.  Built by the package's build step
// into tests/libconvert_harness.so.
//
// Each thread encodes one group of 32 consecutive values.  The values come
// either from an array (harness_encode) or are generated as the fp32 bit
// patterns u0, u0 + 1, ... with an optional sign (harness_encode_bits).
// Output: FP4, 16 bytes per group (channel 2i in the low nibble of byte i);
// FP8, 32 bytes per group.  n must be a multiple of 32; the grid covers
// exactly n / 32 groups.
#include <hip/hip_runtime.h>

#include "kvq_append_dev.h"

namespace {

using namespace kvq;

__device__ __forceinline__ void encode_one(int fp4, float (&x)[32], int byte, uint8_t* out, long long grp) {
  const float scale = as_f32((uint32_t)byte << 23);
  if (fp4) {
    *reinterpret_cast<u32x4_t*>(out + grp * 16) = encode_fp4_group(x, scale);
  } else {
    u32x4_t w[2];
    encode_fp8_group(x, byte - 127, scale, w);
    *reinterpret_cast<u32x4_t*>(out + grp * 32) = w[0];
    *reinterpret_cast<u32x4_t*>(out + grp * 32 + 16) = w[1];
  }
}

__global__ __launch_bounds__(256) void encode_array_kernel(int fp4, const float* __restrict__ in, long long groups,
                                                           int byte, uint8_t* out) {
  const long long grp = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (grp >= groups) return;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = in[grp * 32 + i];
  encode_one(fp4, x, byte, out, grp);
}

__global__ __launch_bounds__(256) void encode_bits_kernel(int fp4, uint32_t u0, long long groups, uint32_t sign,
                                                          int byte, uint8_t* out) {
  const long long grp = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (grp >= groups) return;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = as_f32((u0 + (uint32_t)(grp * 32 + i)) | sign);
  encode_one(fp4, x, byte, out, grp);
}

int launch_grid(long long groups, dim3* grid) {
  if (groups <= 0 || groups > (1LL << 31) * 256 - 1) return -1;
  *grid = dim3((unsigned)((groups + 255) / 256));
  return 0;
}

}  // namespace

// fmt: 1 = FP4 (E2M1), 2 = FP8 (E4M3).  Returns 0 or a HIP error code (-1 for
// bad sizes).
extern "C" int harness_encode(int fmt, const float* in, long long n, int byte, uint8_t* out, void* stream) {
  dim3 grid;
  if (!in || !out || n % 32 || byte < 0 || byte > 254 || launch_grid(n / 32, &grid)) return -1;
  hipLaunchKernelGGL(encode_array_kernel, grid, dim3(256), 0, (hipStream_t)stream, fmt == 1 ? 1 : 0, in, n / 32,
                     byte, out);
  return (int)hipGetLastError();
}

extern "C" int harness_encode_bits(int fmt, uint32_t u0, long long n, int negative, int byte, uint8_t* out,
                                   void* stream) {
  dim3 grid;
  if (!out || n % 32 || byte < 0 || byte > 254 || launch_grid(n / 32, &grid)) return -1;
  if ((unsigned long long)u0 + (unsigned long long)n > 0x80000000ull) return -1;  // stay in one sign's patterns
  hipLaunchKernelGGL(encode_bits_kernel, grid, dim3(256), 0, (hipStream_t)stream, fmt == 1 ? 1 : 0, u0, n / 32,
                     negative ? 0x80000000u : 0u, byte, out);
  return (int)hipGetLastError();
}

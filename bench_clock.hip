// Shader-clock sampler for bench.py's --clock-trace option (measurement only,
// not part of libkvq).  One wave, launched on a side stream next to the timed
// decode steps, records n pairs (wall clock, shader clock) at fixed
// wall-clock intervals; the ratio of the two counters over a window is the
// shader clock the compute units ran at.  The wave needs a handful of
// registers and no LDS, so it fits beside the decode waves on a SIMD without
// taking one of their slots.
//
// Every wait ends: the loop waits for the wall clock to pass a fixed target,
// and the wall clock always advances.
#include <hip/hip_runtime.h>

#include <cstdint>

__global__ __launch_bounds__(64) void bench_clock_sample(unsigned long long* out, int n,
                                                          unsigned long long interval) {
  const unsigned long long w0 = wall_clock64();
  for (int i = 0; i < n; ++i) {
    const unsigned long long target = w0 + (unsigned long long)(i + 1) * interval;
    while (wall_clock64() < target) __builtin_amdgcn_s_sleep(2);
    const unsigned long long w = wall_clock64();
    const unsigned long long c = clock64();
    if (threadIdx.x == 0) {
      out[2 * i] = w;
      out[2 * i + 1] = c;
    }
  }
}

// out: device buffer of 2 n uint64; interval in wall-clock ticks.
extern "C" int bench_clock_launch(void* out, int n, unsigned long long interval, void* stream) {
  if (!out || n <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(bench_clock_sample, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (unsigned long long*)out, n, interval);
  return (int)hipGetLastError();
}

// Wall-clock counter rate of the current device, kHz.
extern "C" int bench_clock_wall_khz(int* khz) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return (int)e;
}

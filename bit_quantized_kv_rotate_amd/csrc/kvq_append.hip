// Write path of the rotated 4-bit KV cache: Walsh-Hadamard rotation, shared
// power-of-two (UE8M0) scale per 32 channels, E2M1 codes (or the E4M3
// comparator), stored into the paged layout; and the dequantiser used by
// tests.  Method: ROCm blog "UltraQuant on AMD Instinct", section "What is
// UltraQuant?" (rotation before the FP4 grid, one power-of-two scale per 32
// channels, 17 bytes per group).
//
// Built with -ffp-contract=off: every fp32 add, subtract and multiply of the
// rotation rounds once, in the documented order, so the stored codes are
// reproducible bit for bit.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMaxD = 1024;

// E2M1 code (bit 3 = sign) of y in a group with scale exponent e_s: round
// |y| * 2^-e_s to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, a tie going to
// the even code, saturating at 6.  The thresholds are the midpoints; ">="
// where the upper neighbour has the even code, ">" where the lower one does.
__device__ __forceinline__ uint32_t e2m1_code(float y, int e_s) {
  const float a = fabsf(ldexpf(y, -e_s));
  const uint32_t k = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return k | ((as_u32(y) >> 31) << 3);
}

// E4M3FN code of y with scale exponent e_s: round to nearest even onto
// subnormals m * 2^-9 or normals with 3 mantissa bits, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(float y, int e_s) {
  const float a = fabsf(ldexpf(y, -e_s));
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);  // 0..8; 8 is the smallest normal
  } else {
    uint32_t u = as_u32(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    const int e = (int)(u >> 23) - 127;
    const uint32_t m = (u >> 20) & 7u;
    code = (e > 8 || (e == 8 && m == 7)) ? 0x7Eu : (((uint32_t)(e + 7) << 3) | m);
  }
  return code | ((as_u32(y) >> 31) << 7);
}

struct AppendParams {
  CacheGeom c;
  uint8_t* kc;
  uint8_t* ks;
  uint8_t* vc;
  uint8_t* vs;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* slots;
  float norm;
};

// One wave per (token, KV head, tensor).
__global__ __launch_bounds__(64) void append_kernel(const AppendParams p) {
  __shared__ float x[kMaxD];
  __shared__ int gexp[kMaxD / 32];
  const int tid = threadIdx.x;
  const int tok = blockIdx.x;
  const int h = blockIdx.y;
  const int tensor = blockIdx.z;
  const int slot = p.slots[tok];
  if (slot < 0) return;
  const CacheGeom& c = p.c;
  const int d = c.d;
  const uint16_t* src = (tensor == 0 ? p.k_new : p.v_new) + ((size_t)tok * c.hkv + h) * d;
  for (int i = tid; i < d; i += 64) x[i] = bf16_to_f32(src[i]);
  __syncthreads();
  if (c.rotate) fwht_rows_lds(x, 1, d, p.norm, tid, 64);

  const int page = slot / c.p;
  const int off = slot - page * c.p;
  uint8_t* codes = (tensor == 0 ? p.kc : p.vc) + (int64_t)page * c.c_page + (int64_t)h * c.c_head;
  uint8_t* scales = (tensor == 0 ? p.ks : p.vs) + (int64_t)page * c.s_page + (int64_t)h * c.s_head;
  const int emax = (c.fmt == KVQ_FMT_FP4_E2M1) ? 2 : 8;

  // Scale exponent per group: floor(log2 amax) is the exponent field of amax
  // (a subnormal or zero amax has field 0); byte = max(field - emax, 0).
  for (int g = tid; g < c.g; g += 64) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[32 * g + i]));
    const int field = (int)((as_u32(amax) >> 23) & 0xFFu);
    const int byte = max(field - emax, 0);
    gexp[g] = byte - 127;
    scales[(int64_t)g * c.p + off] = (uint8_t)byte;
  }
  __syncthreads();

  if (c.fmt == KVQ_FMT_FP4_E2M1) {
    for (int b = tid; b < d / 2; b += 64) {
      const int g = b >> 4;
      const int i = b & 15;
      const int e_s = gexp[g];
      const uint32_t lo = e2m1_code(x[32 * g + 2 * i], e_s);
      const uint32_t hi = e2m1_code(x[32 * g + 2 * i + 1], e_s);
      codes[((int64_t)g * c.p + off) * 16 + i] = (uint8_t)(lo | (hi << 4));
    }
  } else {
    for (int ch = tid; ch < d; ch += 64) {
      const int g = ch >> 5;
      codes[((int64_t)g * c.p + off) * 32 + (ch & 31)] = (uint8_t)e4m3_code(x[ch], gexp[g]);
    }
  }
}

struct DequantParams {
  CacheGeom c;
  const int32_t* slots;
  float* k_out;
  float* v_out;
};

__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t k = code & 7u;
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6
  float v = (k < 4) ? 0.5f * (float)k : (float)(2u << ((k - 4) >> 1)) * ((k & 1) ? 1.5f : 1.0f);
  return (code & 8u) ? -v : v;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u;
  const uint32_t m = code & 7u;
  float v;
  if (e == 15u && m == 7u)
    v = __builtin_nanf("");
  else if (e == 0u)
    v = ldexpf((float)m, -9);
  else
    v = ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  return (code & 0x80u) ? -v : v;
}

__global__ __launch_bounds__(64) void dequant_kernel(const DequantParams p) {
  const int tid = threadIdx.x;
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int tensor = blockIdx.z;
  const CacheGeom& c = p.c;
  const int slot = p.slots[n];
  const int page = slot / c.p;
  const int off = slot - page * c.p;
  const uint8_t* codes = (tensor == 0 ? c.kc : c.vc) + (int64_t)page * c.c_page + (int64_t)h * c.c_head;
  const uint8_t* scales = (tensor == 0 ? c.ks : c.vs) + (int64_t)page * c.s_page + (int64_t)h * c.s_head;
  float* out = (tensor == 0 ? p.k_out : p.v_out) + ((size_t)n * c.hkv + h) * c.d;
  for (int ch = tid; ch < c.d; ch += 64) {
    const int g = ch >> 5;
    const int byte = scales[(int64_t)g * c.p + off];
    float v;
    if (c.fmt == KVQ_FMT_FP4_E2M1) {
      const uint32_t pair = codes[((int64_t)g * c.p + off) * 16 + ((ch & 31) >> 1)];
      v = e2m1_value((ch & 1) ? (pair >> 4) : (pair & 15u));
    } else {
      v = e4m3_value(codes[((int64_t)g * c.p + off) * 32 + (ch & 31)]);
    }
    out[ch] = ldexpf(v, byte - 127);
  }
}

}  // namespace

hipError_t launch_append(const CacheGeom& c, uint8_t* kc, uint8_t* ks, uint8_t* vc, uint8_t* vs,
                         const uint16_t* k_new, const uint16_t* v_new, const int32_t* slots,
                         int n_tokens, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  AppendParams p;
  p.c = c;
  p.kc = kc;
  p.ks = ks;
  p.vc = vc;
  p.vs = vs;
  p.k_new = k_new;
  p.v_new = v_new;
  p.slots = slots;
  p.norm = fwht_norm(c.d);
  dim3 grid((unsigned)n_tokens, (unsigned)c.hkv, c.kv_shared ? 1u : 2u);
  hipLaunchKernelGGL(append_kernel, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dequant(const CacheGeom& c, const int32_t* slots, int n, float* k_out,
                          float* v_out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  DequantParams p;
  p.c = c;
  p.slots = slots;
  p.k_out = k_out;
  p.v_out = v_out;
  dim3 grid((unsigned)n, (unsigned)c.hkv, c.kv_shared ? 1u : 2u);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq

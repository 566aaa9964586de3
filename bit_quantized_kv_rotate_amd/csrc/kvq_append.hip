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
  int n_tokens;
  float norm;
};

// One wave covers 64 / G tokens of one (KV head, tensor) for vectors of
// G = D / 32 channel groups: lane l holds the 32 channels of group l % G of
// token l / G.  Stages h = 1 .. 16 of the transform run inside the lane;
// stage h >= 32 pairs lane l with lane l ^ (h / 32).  Every stage is the fp32
// a + b / a - b of the radix-2 definition, in stage order, followed by one
// multiply by fp32(1/sqrt(D)): the operations and their order are those of
// the definition, so the codes are reproducible bit for bit.  The group's
// amax, scale byte and codes are then all lane-local: 16 code bytes (FP4)
// or 32 (FP8) leave in 16-byte stores, and the tokens of a wave that share a
// page fill whole 16-token runs of each group.
template <int G>
__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  constexpr int TW = 64 / G;  // tokens per wave
  constexpr int D = 32 * G;
  const CacheGeom& c = p.c;
  const int lane = threadIdx.x & 63;
  const int g = lane & (G - 1);
  const int tok = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TW + lane / G;
  const int h = blockIdx.y;
  const int tensor = blockIdx.z;
  const bool valid = tok < p.n_tokens;
  const int slot = valid ? p.slots[tok] : -1;

  float x[32];
  const uint16_t* base = tensor == 0 ? p.k_new : p.v_new;
  if (valid) {
    const uint16_t* src = base + ((size_t)tok * c.hkv + h) * D + 32 * g;
    if (((uintptr_t)base & 15) == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src + 8 * k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * k + 2 * e] = as_f32(w[e] << 16);
          x[8 * k + 2 * e + 1] = as_f32(w[e] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = bf16_to_f32(src[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.0f;
  }

  if (c.rotate) {
#pragma unroll
    for (int hh = 1; hh < 32; hh <<= 1) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (!(j & hh)) {
          const float a = x[j];
          const float b = x[j + hh];
          x[j] = a + b;
          x[j + hh] = a - b;
        }
      }
    }
#pragma unroll
    for (int s = 1; s < G; s <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float y = __shfl_xor(x[i], s, 64);
        x[i] = (g & s) ? (y - x[i]) : (x[i] + y);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = x[i] * p.norm;
  }
  if (slot < 0) return;  // no shuffles below

  // Scale exponent: floor(log2 amax) is the exponent field of amax (a
  // subnormal or zero amax has field 0); byte = max(field - emax, 0).
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(x[i]));
  const bool fp4 = c.fmt == KVQ_FMT_FP4_E2M1;
  const int field = (int)((as_u32(am) >> 23) & 0xFFu);
  const int byte = max(field - (fp4 ? 2 : 8), 0);
  const int e_s = byte - 127;

  const int page = slot / c.p;
  const int off = slot - page * c.p;
  const int64_t unit = (int64_t)g * c.p + off;  // (group, offset) inside the (page, head) block
  uint8_t* codes = (tensor == 0 ? p.kc : p.vc) + (int64_t)page * c.c_page + (int64_t)h * c.c_head + unit * c.cb;
  uint8_t* scales = (tensor == 0 ? p.ks : p.vs) + (int64_t)page * c.s_page + (int64_t)h * c.s_head;
  scales[unit] = (uint8_t)byte;
  if (fp4) {
    u32x4_t w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t d = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 8 * k + 2 * e;
        d |= (e2m1_code(x[i], e_s) | (e2m1_code(x[i + 1], e_s) << 4)) << (8 * e);
      }
      w[k] = d;
    }
    *reinterpret_cast<u32x4_t*>(codes) = w;
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4_t w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t d = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) d |= e4m3_code(x[16 * half + 4 * k + e], e_s) << (8 * e);
        w[k] = d;
      }
      *reinterpret_cast<u32x4_t*>(codes + 16 * half) = w;
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
  p.n_tokens = n_tokens;
  p.norm = fwht_norm(c.d);
  const int G = c.d / 32;
  const long long chunks = ((long long)n_tokens * G + 63) / 64;  // waves per (head, tensor)
  const dim3 grid((unsigned)((chunks + 3) / 4), (unsigned)c.hkv, c.kv_shared ? 1u : 2u);
  switch (G) {
    case 1: hipLaunchKernelGGL((append_kernel<1>), grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((append_kernel<2>), grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((append_kernel<4>), grid, dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((append_kernel<8>), grid, dim3(256), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((append_kernel<16>), grid, dim3(256), 0, stream, p); break;
    case 32: hipLaunchKernelGGL((append_kernel<32>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
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

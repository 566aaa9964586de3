// Device side of the append (rotate, scale, E2M1 / E4M3 codes, store into
// the paged layout), shared by the append kernel and the decode prologue
// that appends a step's new tokens before it prepares the queries.  Method:
// ROCm blog "UltraQuant on AMD Instinct", section "What is UltraQuant?"
// (rotation before the FP4 grid, one power-of-two scale per 32 channels, 17
// bytes per group).
//
// Every fp32 add, subtract and multiply of the rotation rounds once, in the
// documented order (contraction is off inside append_wave whatever the
// including file's flags), so the stored codes are reproducible bit for bit.
#pragma once

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
// Wave `wave` of (KV head h, tensor): the append kernel runs one per 64
// threads; the decode prologue runs them beside the query rows of a call
// that appends and then attends.
template <int G>
__device__ __forceinline__ void append_wave(const AppendParams& p, int wave, int h, int tensor, int lane) {
#pragma clang fp contract(off)
  constexpr int TW = 64 / G;  // tokens per wave
  constexpr int D = 32 * G;
  const CacheGeom& c = p.c;
  const int g = lane & (G - 1);
  const int tok = wave * TW + lane / G;
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
  if (slot < 0) return;  // no shuffles below (the caller's wave ends here)

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

inline AppendParams make_append_params(const CacheGeom& c, const AppendArgs& a) {
  AppendParams p;
  p.c = c;
  p.kc = a.kc;
  p.ks = a.ks;
  p.vc = a.vc;
  p.vs = a.vs;
  p.k_new = a.k_new;
  p.v_new = a.v_new;
  p.slots = a.slots;
  p.n_tokens = a.n_tokens;
  p.norm = fwht_norm(c.d);
  return p;
}

// waves of the append per (KV head, tensor), and its blocks of 4 waves
inline long long append_waves(const CacheGeom& c, int n_tokens) {
  return ((long long)n_tokens * (c.d / 32) + 63) / 64;
}

}  // namespace
}  // namespace kvq

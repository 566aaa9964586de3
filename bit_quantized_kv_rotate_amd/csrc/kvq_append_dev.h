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

// Codes come from the hardware conversions (v_cvt_scalef32_pk_fp4_f32 and
// v_cvt_scalef32_pk_fp8_f32) with the group's scale 2^e_s as the scale
// operand: they divide by it and round to nearest even onto the format's
// grid, the sign copied (negative values that round to zero give the code of
// -0).  E2M1 saturates at 6 by itself; E4M3FN does not, so values are first
// clamped to +-448 * 2^e_s, which leaves every other code unchanged.  The
// GPU test test_gpu_convert_sweep.py compares encode_fp4_group and
// encode_fp8_group below with the test suite's independent CPU encoders:
// every finite fp32 input with |x| < 8 at scale 2^0 (E2M1), the grid values,
// the ties between them and their neighbours at the extreme and middle scale
// bytes, and random inputs over each format's whole range.

// The 16 code bytes of one 32-value group at scale 2^e_s (scale: the fp32
// whose exponent field is the group's scale byte): channel 2i in the low
// nibble of byte i.
__device__ __forceinline__ u32x4_t encode_fp4_group(const float (&x)[32], float scale) {
  u32x4_t w;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * k + 0], x[8 * k + 1], scale, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * k + 2], x[8 * k + 3], scale, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * k + 4], x[8 * k + 5], scale, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * k + 6], x[8 * k + 7], scale, 3);
    w[k] = d;
  }
  return w;
}

// The 32 E4M3 bytes of one group at scale 2^e_s, after the clamp to
// +-448 * 2^e_s (x is clamped in place); w[0] holds channels 0..15.
__device__ __forceinline__ void encode_fp8_group(float (&x)[32], int e_s, float scale, u32x4_t (&w)[2]) {
  typedef __attribute__((ext_vector_type(2))) short s16x2_t;
  const float lim = ldexpf(448.0f, e_s);
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fminf(fmaxf(x[i], -lim), lim);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 16 * half + 4 * k;
      s16x2_t d = {0, 0};
      d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, x[i + 0], x[i + 1], scale, false);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(d, x[i + 2], x[i + 3], scale, true);
      w[half][k] = __builtin_bit_cast(uint32_t, d);
    }
  }
}

// The value x holds in lane l ^ s (s a power of two below 64): a DPP quad
// permutation for s = 1 and 2 (every source lane is in range, so the zero
// fill of bound_ctrl never applies; it lets the move fold into the add that
// uses it), the LDS permute network above.
__device__ __forceinline__ float xor_lane(float x, int s) {
  if (s == 1) return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  if (s == 2) return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return __shfl_xor(x, s, 64);
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
    // y - x is y + (-x) and x + y is y + x, exactly: one add with the
    // lane's sign on x
#pragma unroll
    for (int s = 1; s < G; s <<= 1) {
      float sx[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) sx[i] = (g & s) ? -x[i] : x[i];
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = xor_lane(x[i], s) + sx[i];
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

  // (the page size is 16, 32 or 64 and the slot is not negative here)
  const int page = slot >> __builtin_ctz((unsigned)c.p);
  const int off = slot & (c.p - 1);
  const int64_t unit = (int64_t)g * c.p + off;  // (group, offset) inside the (page, head) block
  uint8_t* codes = (tensor == 0 ? p.kc : p.vc) + (int64_t)page * c.c_page + (int64_t)h * c.c_head + unit * c.cb;
  uint8_t* scales = (tensor == 0 ? p.ks : p.vs) + (int64_t)page * c.s_page + (int64_t)h * c.s_head;
  scales[unit] = (uint8_t)byte;
  const float scale = as_f32((uint32_t)byte << 23);  // 2^e_s (field 0: 2^-127)
  if (fp4) {
    *reinterpret_cast<u32x4_t*>(codes) = encode_fp4_group(x, scale);
  } else {
    u32x4_t w[2];
    encode_fp8_group(x, e_s, scale, w);
    *reinterpret_cast<u32x4_t*>(codes) = w[0];
    *reinterpret_cast<u32x4_t*>(codes + 16) = w[1];
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

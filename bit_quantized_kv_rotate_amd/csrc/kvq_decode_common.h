// Pieces shared by the decode kernels (head_dim 128 in kvq_decode.hip, 512
// in kvq_decode512.hip): kernel parameters, code conversions, lane
// reductions, the FP6 query split, buffer resources, the wave-level
// Walsh-Hadamard transform and the split merge.  Everything sits in an
// anonymous namespace: each translation unit gets its own copy.
#pragma once

#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct DecodeParams {
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int64_t c_head, c_page, s_head, s_page;
  int64_t c_total, s_total;  // bytes of one code / scale array
  // 1: both arrays below 4 GiB, so a page's offset fits the 32-bit scalar
  // offset of one buffer resource per array (flat addressing); 0: one
  // resource per (page, head) block
  int flat;
  int P;
  int p_shift;  // log2(P)
  int hkv;
  int batch;     // sequences (set by the kernels that derive units from it)
  int rows_pad;  // padded rows per (sequence, KV head) of the many-row kernel
  const uint16_t* q;
  int hq, n_q, group, rows;
  const int32_t* block_tables;
  int max_pages;
  const int32_t* context_lens;
  float qscale;
  float norm;
  int rotate_q, rotate_out;
  int splits, tiles_per_split;
  float* out;
  float* ws_o;       // [B][hkv][splits][8*NT][kD]
  float* ws_ml;      // [B][hkv][splits][8*NT][2]
  uint32_t* qops;    // [B][hkv][NT][QOpsLayout::kSlots][64 lanes][kDwords]
  // Shared-prefix decode (null / zero in a plain call).  Suffix level: each
  // sequence's scan starts at token tok_start[b] (a multiple of 16).  Prefix
  // level (head_dim 128 many-row kernel): units are prefix groups, group g's
  // member sequences are grp_seq[grp_ptr[g] .. grp_ptr[g + 1]), its pages are
  // block_tables[g], member s sees its tokens 0 .. shared_lens[s] - 1, and
  // the partials are stored per member sequence, rows_seq rows each.
  const int32_t* tok_start;
  const int32_t* grp_ptr;
  const int32_t* grp_seq;
  const int32_t* shared_lens;
  int rows_seq;
  int keep_partials;  // always leave split partials (a later merge combines them)
  // Selected-position decode (latent kernel): the scan runs over the list
  // sel[b * sel_stride + j], j < context_lens[b], of token positions instead
  // of over the positions themselves.
  const int32_t* sel;
  int sel_stride;
};

// Kernel format: the cache format, or kFmtFP4Conv, an FP4 cache whose score
// product converts the K codes with their scales to bf16 for bf16 MFMAs
// against a bf16 hi + lo query (the alternative to the native scaled MFMA,
// kept for comparison: KVQ_QK_CONVERT).
constexpr int kFmtFP4Conv = 3;

template <int FMT>
struct Fmt {
  static constexpr bool kFP4 = FMT == KVQ_FMT_FP4_E2M1 || FMT == kFmtFP4Conv;  // FP4 codes in the cache
  static constexpr bool kNativeQK = FMT == KVQ_FMT_FP4_E2M1;  // codes straight into the scaled MFMA
  static constexpr int kWords = kFP4 ? 4 : 8;      // uint32 of codes per (token, group)
};

// Dequantise one (token, 32-channel group) into 16 packed bf16x2 words
// (channel order 0..31), applying the group's power-of-two scale.
template <int FMT>
__device__ __forceinline__ void dequant_group(const uint32_t (&w)[Fmt<FMT>::kWords], float scale,
                                              uint32_t (&o)[16]) {
  if constexpr (Fmt<FMT>::kFP4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 0));
      o[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 1));
      o[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 2));
      o[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 3));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[2 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], scale, false));
      o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], scale, true));
    }
  }
}

__device__ __forceinline__ float dpp_ror8(float x) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(x), 0x128, 0xF, 0xF, false));
}

// max over lanes l, l^16, l^32, l^48 (VALU lane swaps, no LDS traffic)
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = fmaxf(as_f32(a[0]), as_f32(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return fmaxf(as_f32(b[0]), as_f32(b[1]));
}

__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = as_f32(a[0]) + as_f32(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return as_f32(b[0]) + as_f32(b[1]);
}

// x + (the value in lane l ^ 32)
__device__ __forceinline__ float add_half_swap(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return as_f32(b[0]) + as_f32(b[1]);
}

// Round y * 2^-e onto FP6 E2M3 (1 sign, 2 exponent bits with bias 1, 3
// mantissa bits; largest 7.5), nearest even, saturating.  Returns the 6-bit
// code (bit 5 = sign) and, in `val`, the value it stands for (code * 2^e), so
// y - val is the exact residual.
__device__ __forceinline__ uint32_t e2m3_split(float y, int e, float& val) {
  const float a = fabsf(ldexpf(y, -e));
  float r;
  uint32_t code;
  if (a < 1.0f) {
    const float m = rintf(a * 8.0f);  // 0..8; 8 is the smallest normal
    code = (uint32_t)m;
    r = m * 0.125f;
  } else {
    uint32_t u = as_u32(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    u &= 0xFFF00000u;
    const int ex = (int)(u >> 23) - 127;
    const uint32_t mm = (u >> 20) & 7u;
    if (ex > 2) {
      code = 31u;
      r = 7.5f;
    } else {
      code = ((uint32_t)(ex + 1) << 3) | mm;
      r = as_f32(u);
    }
  }
  const uint32_t sign = as_u32(y) & 0x80000000u;
  val = as_f32(as_u32(ldexpf(r, e)) | sign);
  return code | (sign >> 26);
}

// Buffer resource over one (page, KV head) block: loads through it take a
// scalar base, a scalar in-page offset and the lane's constant offset, and
// reads past the block return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* base, int64_t off,
                                                             int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), 0, (int)bytes, 0x00020000);
}

// Largest cache array (bytes) the flat addressing serves: page offsets are
// 32-bit scalar offsets.
constexpr int64_t kFlatMaxBytes = 0xFFFFF000LL;
inline int flat_ok(int64_t c_total, int64_t s_total) {
  return c_total <= kFlatMaxBytes && s_total <= kFlatMaxBytes;
}

// DPP source x of every lane (all masks set; the listed patterns never leave
// the row, so the zero fill never applies)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppXor3 = 0x1B;        // quad_perm [3, 2, 1, 0]
constexpr int kDppMirror = 0x140;     // lane i of a row of 16 reads lane 15 - i (i ^ 15)
constexpr int kDppHalfMirror = 0x141; // lane i of a half row reads lane 7 - i (i ^ 7)

// The value lane l ^ s holds (s = 1, 2, 4, 8, 16, 32), with no LDS permute:
// DPP quad permutations and row mirrors below 16 (i ^ 4 = (i ^ 3) ^ 7 and
// i ^ 8 = (i ^ 7) ^ 15), a VALU lane swap of rows or halves above.
template <int S>
__device__ __forceinline__ float lane_xor(float x, int lane) {
  if constexpr (S == 1) return dpp_f32<kDppXor1>(x);
  if constexpr (S == 2) return dpp_f32<kDppXor2>(x);
  if constexpr (S == 4) return dpp_f32<kDppHalfMirror>(dpp_f32<kDppXor3>(x));
  if constexpr (S == 8) return dpp_f32<kDppMirror>(dpp_f32<kDppHalfMirror>(x));
  if constexpr (S == 16 || S == 32) {
    // the swap leaves (own, partner) in the lower lanes and (partner, own)
    // in the upper ones
    const auto a = S == 16 ? __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false)
                           : __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
    return as_f32((lane & S) ? a[0] : a[1]);
  }
  return __shfl_xor(x, S, 64);
}

// max and sum over the 64 lanes, by the butterfly of lane_xor (the sum adds
// in the order of the l ^ 1, l ^ 2, ... l ^ 32 butterfly)
__device__ __forceinline__ float wave_max(float x, int lane) {
  x = fmaxf(x, lane_xor<1>(x, lane));
  x = fmaxf(x, lane_xor<2>(x, lane));
  x = fmaxf(x, lane_xor<4>(x, lane));
  x = fmaxf(x, lane_xor<8>(x, lane));
  x = fmaxf(x, lane_xor<16>(x, lane));
  return fmaxf(x, lane_xor<32>(x, lane));
}
__device__ __forceinline__ float wave_sum(float x, int lane) {
  x += lane_xor<1>(x, lane);
  x += lane_xor<2>(x, lane);
  x += lane_xor<4>(x, lane);
  x += lane_xor<8>(x, lane);
  x += lane_xor<16>(x, lane);
  return x + lane_xor<32>(x, lane);
}

// max over the 16 lanes of a row (DPP only)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<0x124>(x));  // row_ror:4
  return fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8
}

// Walsh-Hadamard transform of one row of D = 64 C channels held by a wave,
// lane l holding channels C l .. C l + C - 1: stages h < C inside the lane,
// stage h >= C between lanes l and l ^ (h / C); fp32 a + b and a - b in the
// order of the radix-2 definition, then one multiply by c.
template <int C>
__device__ __forceinline__ void wave_fwht(float (&x)[C], int lane, float c) {
#pragma unroll
  for (int hh = 1; hh < C; hh <<= 1) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      if (!(j & hh)) {
        const float a = x[j];
        const float b = x[j + hh];
        x[j] = a + b;
        x[j + hh] = a - b;
      }
    }
  }
  // (y - x is y + (-x) and x + y is y + x, exactly)
  auto stage = [&](auto s_tag) {
    constexpr int S = decltype(s_tag)::value;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const float sx = (lane & S) ? -x[i] : x[i];
      x[i] = lane_xor<S>(x[i], lane) + sx;
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
  stage(std::integral_constant<int, 16>{});
  stage(std::integral_constant<int, 32>{});
#pragma unroll
  for (int i = 0; i < C; ++i) x[i] = x[i] * c;
}

constexpr int kMaxSplits = 64;
// The online softmax keeps a per-row reference maximum that may lag the
// running maximum by up to 2^kLazyLog2 (weights exp2(s - ref) <= 2^8): a
// rescale of the output is needed only when a row's maximum passes its
// reference by more than that.  The split partials carry the reference as m.
constexpr float kLazyLog2 = 8.0f;

// acc += w_s * O_s over the splits s < S (1 <= S <= 64) of one query row, in
// split order, skipping splits of weight zero (an empty split stores no O):
// src(s) points at this lane's C channels of split s, and weights() returns
// ws, whose lane s holds w_s.  The loads of a round are issued before any is
// used (a loop of one load and one wait per split pays a memory round trip
// per split).  The first eight splits are loaded before weights() runs, so
// that their loads share a round trip with the (m, l) loads it waits for; of
// the others only those of nonzero weight are loaded, K at a time (K = 32 for
// two channels per lane: up to 56 more splits in two rounds).  The sums are
// the same for every K: the same fused multiply-adds in split order.
template <int C, int K = 8, typename Src, typename Weights>
__device__ __forceinline__ void merge_splits(float (&acc)[C], int S, Src src, Weights weights) {
  static_assert(K >= 8 && K <= 32, "splits per round");
  constexpr int K0 = 8;  // the first round, beside the (m, l) loads
  f32x2_t o[K][C / 2];
  int idx[K];
  // the next N splits of the wave-uniform mask todo, in ascending order;
  // past its last split, idx = -1 and split idx[0] is loaded again
  auto load = [&](uint64_t& todo, auto n_tag) {
    constexpr int N = decltype(n_tag)::value;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      idx[k] = todo ? __builtin_ctzll(todo) : -1;
      todo &= todo - 1;
      const float* ptr = src(idx[k] >= 0 ? idx[k] : idx[0]);
#pragma unroll
      for (int i = 0; i < C; i += 2) o[k][i / 2] = *reinterpret_cast<const f32x2_t*>(ptr + i);
    }
  };
  auto add = [&](float ws, auto n_tag) {
    constexpr int N = decltype(n_tag)::value;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const float wl = as_f32((uint32_t)__builtin_amdgcn_readlane((int)as_u32(ws), idx[k] & 63));
      const float w = idx[k] >= 0 ? wl : 0.0f;
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const float f = __builtin_fmaf(w, o[k][i / 2][i & 1], acc[i]);
        acc[i] = (w != 0.0f) ? f : acc[i];
      }
    }
  };
  using First = std::integral_constant<int, K0>;
  using Later = std::integral_constant<int, K>;
  uint64_t todo = S >= K0 ? (1ull << K0) - 1 : (1ull << S) - 1;
  load(todo, First{});
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the waits in weights()
  const float ws = weights();
  add(ws, First{});
  todo = __ballot(ws != 0.0f) & ~((1ull << K0) - 1);
  while (todo) {
    load(todo, Later{});
    add(ws, Later{});
  }
}

// Combine the split partials of each query row: weights 2^(m_s - M),
// normalise by the combined sum, rotate back, store.  A split of weight zero
// (an empty one, which writes only its (m, l)) adds nothing.  One wave per row
// (four per block, ROWS padded rows per (sequence, KV head), or p.rows_pad
// when ROWS is 0); lane s < S
// holds split s's (m, l), lane l accumulates channels C l .. C l + C - 1 of
// the D = 64 C channels over the splits, loading up to K nonzero-weight
// splits per round after the first eight.
template <int ROWS_T, int C, int K = 8>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeParams p) {
  constexpr int D = 64 * C;
  const int ROWS = ROWS_T > 0 ? ROWS_T : p.rows_pad;  // 0: padded row count at run time
  const int lane = threadIdx.x & 63;
  const long long gr = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // grid covers exactly B * hkv * ROWS
  const int r = (int)(gr % ROWS);
  const int bh = (int)(gr / ROWS);
  if (r >= p.rows) return;  // padding row: the whole wave leaves (no barrier follows)
  const int kvh = bh % p.hkv;
  const int b = bh / p.hkv;
  const int S = p.splits;
  const size_t row0 = (size_t)bh * S * ROWS + r;  // split s: row0 + s * ROWS

  float ms = -INFINITY, ls = 0.0f;
  if (lane < S) {
    ms = p.ws_ml[(row0 + (size_t)lane * ROWS) * 2 + 0];
    ls = p.ws_ml[(row0 + (size_t)lane * ROWS) * 2 + 1];
  }
  float lsum = 0.0f;
  float acc[C];
#pragma unroll
  for (int i = 0; i < C; ++i) acc[i] = 0.0f;
  const float* po = p.ws_o + row0 * D + C * lane;
  merge_splits<C, K>(acc, S, [&](int sp) { return po + (size_t)sp * ROWS * D; }, [&] {
    float M = ms;
    M = wave_max(M, lane);
    const float ws = (M != -INFINITY) ? __builtin_amdgcn_exp2f(ms - M) : 0.0f;
    lsum = ws * ls;
    lsum = wave_sum(lsum, lane);
    return ws;
  });
  const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int i = 0; i < C; ++i) acc[i] *= inv;
  if (p.rotate_out) wave_fwht<C>(acc, lane, p.norm);
  const int j = r / p.group;
  const int hh = r - j * p.group;
  float* dst = p.out + (((size_t)b * p.n_q + j) * p.hq + (size_t)kvh * p.group + hh) * D + C * lane;
#pragma unroll
  for (int i = 0; i < C; ++i) dst[i] = acc[i];
}

}  // namespace
}  // namespace kvq

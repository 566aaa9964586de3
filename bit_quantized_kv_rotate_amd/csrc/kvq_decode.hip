// Decode attention over the paged FP4 (E2M1 + UE8M0 per 32 channels) cache,
// and over the FP8 (E4M3 + UE8M0 per 32) comparator cache.
//
// Method: ROCm blog "UltraQuant on AMD Instinct", section "Why UltraQuant
// beats 8-bit KV": a decode step re-reads the whole cache, so time follows
// the bytes moved; the codes and power-of-two scales go to the matrix cores
// without a lookup table.  Section "Throughput vs latency trade-off": an MTP
// verify step has several query positions per sequence; here they share one
// pass over the cache (the page names this fusion as future work).
//
// Design (gfx950, wave64, one wave per (sequence, KV head, context split)):
//  * The page scan streams 16-token tiles.  Lane l loads the 16 (FP4) or 32
//    (FP8) code bytes of token l%16, channel group l/16, plus that group's
//    scale byte: one contiguous 1 KB (FP4) block per tile and tensor.
//  * K codes become the A operand of v_mfma_f32_16x16x32_bf16 through the
//    gfx950 scaled converts (2 values and the UE8M0 scale per instruction; no
//    table).  E2M1 x 2^k is exact in bf16.  The channel order inside the
//    contraction is permuted so each lane feeds its own group: lane group j
//    covers channels 32j + 8s .. 32j + 8s + 7 in k-step s.
//  * Scores are computed transposed (S^T = K q^T: tokens x query rows), so
//    the accumulator layout is directly the A operand of the PV product.
//  * Precision: q and P are split into bf16 hi + lo parts (residual ~2^-17),
//    placed in the 16 MFMA columns as 8 hi rows + the same 8 rows lo; one
//    DPP row rotate adds the halves.  Accumulation is fp32.
//  * V codes are converted with their scale into a wave-private LDS tile and
//    read back transposed with ds_read_b64_tr_b16 as the B operand of PV.
//  * Online softmax in base 2 (q pre-scaled by sm_scale * log2 e), row max by
//    cross-lane shuffles, lazy O rescale only when a row max moves.
//  * Context split into `splits` ranges; partial (m, l, O) go to the
//    workspace and a merge kernel combines them, normalises, rotates back.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kD = 128;        // head_dim handled by this kernel
constexpr int kG = kD / 32;    // scale groups per vector
constexpr int kVRow = 2 * kD + 16;  // LDS bytes per token row of V (bf16, padded)

struct DecodeParams {
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int64_t c_head, c_page, s_head, s_page;
  int P;
  int hkv;
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
  float* ws_o;   // [B][hkv][splits][8*NT][kD]
  float* ws_ml;  // [B][hkv][splits][8*NT][2]
};

template <int FMT>
struct CodeWords {
  static constexpr int kWords = (FMT == KVQ_FMT_FP4_E2M1) ? 4 : 8;  // uint32 per (token, group)
  static constexpr int kBytes = kWords * 4;
};

// Dequantise one (token, 32-channel group) into 16 packed bf16x2 words
// (channel order 0..31), applying the group's power-of-two scale.
template <int FMT>
__device__ __forceinline__ void dequant_group(const uint32_t (&w)[CodeWords<FMT>::kWords],
                                              float scale, uint32_t (&o)[16]) {
  if constexpr (FMT == KVQ_FMT_FP4_E2M1) {
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

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m, 64)); }

template <int FMT>
struct RawTile {
  uint32_t k[CodeWords<FMT>::kWords];
  uint32_t v[CodeWords<FMT>::kWords];
  uint32_t ksc, vsc;
};

template <int FMT>
__device__ __forceinline__ void load_tile(const DecodeParams& p, int b, int kvh, int tile, int lane,
                                          RawTile<FMT>& t) {
  constexpr int W = CodeWords<FMT>::kWords;
  const int tok = tile * 16;
  const int page = p.block_tables[(size_t)b * p.max_pages + tok / p.P];
  const int off = tok % p.P + (lane & 15);
  const int grp = lane >> 4;
  const int64_t cidx = (int64_t)page * p.c_page + (int64_t)kvh * p.c_head +
                       ((int64_t)grp * p.P + off) * (4 * W);
  const int64_t sidx = (int64_t)page * p.s_page + (int64_t)kvh * p.s_head + (int64_t)grp * p.P + off;
  const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(p.kc + cidx);
  const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(p.vc + cidx);
#pragma unroll
  for (int i = 0; i < W / 4; ++i) {
    const u32x4_t a = __builtin_nontemporal_load(kp + i);
    const u32x4_t c = __builtin_nontemporal_load(vp + i);
    t.k[4 * i + 0] = a[0]; t.k[4 * i + 1] = a[1]; t.k[4 * i + 2] = a[2]; t.k[4 * i + 3] = a[3];
    t.v[4 * i + 0] = c[0]; t.v[4 * i + 1] = c[1]; t.v[4 * i + 2] = c[2]; t.v[4 * i + 3] = c[3];
  }
  t.ksc = p.ks[sidx];
  t.vsc = p.vs[sidx];
}

template <int FMT, int NT>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeParams p) {
  constexpr int ROWS = 8 * NT;
  __shared__ __attribute__((aligned(16))) float s_rows[ROWS * kD];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][16][kVRow];

  const int lane = threadIdx.x;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int L = p.context_lens[b];
  const int n_tiles = (L + 15) >> 4;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(n_tiles, t_begin + p.tiles_per_split);
  const int tok_limit = min(L, t_end * 16);
  const int col = lane & 15;       // MFMA column: query row (col & 7), hi if col < 8
  const int quad = lane >> 4;      // lane group
  const bool hi_col = col < 8;

  // ---- query prologue: load, rotate, pre-scale, split into bf16 hi/lo B operands
  for (int i = lane; i < ROWS * kD; i += 64) {
    const int r = i / kD;
    const int ch = i % kD;
    float v = 0.0f;
    if (r < p.rows) {
      const int j = r / p.group;
      const int hh = r - j * p.group;
      v = bf16_to_f32(p.q[(((size_t)b * p.n_q + j) * p.hq + (size_t)kvh * p.group + hh) * kD + ch]);
    }
    s_rows[i] = v;
  }
  __syncthreads();
  if (p.rotate_q) fwht_rows_lds(s_rows, ROWS, kD, p.norm, lane, 64);

  bf16x8_t qB[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* src = s_rows + (8 * t + (col & 7)) * kD + 32 * quad + 8 * s;
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = src[2 * e] * p.qscale;
        const float x1 = src[2 * e + 1] * p.qscale;
        uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
        if (!hi_col) {
          h0 = f32_to_bf16_rne(x0 - bf16_to_f32((uint16_t)h0));
          h1 = f32_to_bf16_rne(x1 - bf16_to_f32((uint16_t)h1));
        }
        w[e] = h0 | (h1 << 16);
      }
      qB[t][s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x4_t O[NT][8];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.0f;
#pragma unroll
    for (int n = 0; n < 8; ++n) O[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Causal limit of each row this lane's column stands for.
  int row_last[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = 8 * t + (col & 7);
    row_last[t] = (r < p.rows) ? (L - p.n_q + r / p.group) : -1;
  }

  RawTile<FMT> cur[2], nxt[2];
  if (t_begin < t_end) {
    load_tile<FMT>(p, b, kvh, t_begin, lane, cur[0]);
    load_tile<FMT>(p, b, kvh, min(t_begin + 1, t_end - 1), lane, cur[1]);
  }

#pragma unroll 1
  for (int tile = t_begin; tile < t_end; tile += 2) {
    // prefetch the next pair of tiles
    const bool more = tile + 2 < t_end;
    if (more) {
      load_tile<FMT>(p, b, kvh, tile + 2, lane, nxt[0]);
      load_tile<FMT>(p, b, kvh, min(tile + 3, t_end - 1), lane, nxt[1]);
    }

    // ---- scores S^T = K q^T for both tiles
    f32x4_t S[2][NT];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t kb[16];
      dequant_group<FMT>(cur[s].k, scale_operand(cur[s].ksc), kb);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4_t a = {kb[4 * ks], kb[4 * ks + 1], kb[4 * ks + 2], kb[4 * ks + 3]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qB[t][ks],
                                                        acc, 0, 0, 0);
        }
        S[s][t] = acc;
      }
    }

    // ---- V tiles -> LDS (bf16, token rows), invalid tokens zeroed
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t vb[16];
      dequant_group<FMT>(cur[s].v, scale_operand(cur[s].vsc), vb);
      const int tok = (tile + s) * 16 + col;
      if (tok >= tok_limit) {
#pragma unroll
        for (int i = 0; i < 16; ++i) vb[i] = 0u;
      }
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(&s_v[s][col][64 * quad]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{vb[4 * i], vb[4 * i + 1], vb[4 * i + 2], vb[4 * i + 3]};
    }

    // ---- softmax update and P (bf16 hi/lo) per row tile
    bf16x8_t A[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float sc[8];
      float mloc = -INFINITY;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = S[s][t][i];
          x = x + dpp_ror8(x);
          const int tok = (tile + s) * 16 + 4 * quad + i;
          const bool ok = (tok < tok_limit) && (tok <= row_last[t]);
          x = ok ? x : -INFINITY;
          sc[4 * s + i] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = xor_max(mloc, 16);
      mloc = xor_max(mloc, 32);
      const float m_new = fmaxf(m_run[t], mloc);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = (m_new == m_run[t]) ? 1.0f : __builtin_amdgcn_exp2f(m_run[t] - m_use);
      m_run[t] = m_new;
      float psum = 0.0f;
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(sc[2 * e] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(sc[2 * e + 1] - m_use);
        psum += p0 + p1;
        const uint32_t h = pack_bf16x2(p0, p1);
        if (hi_col) {
          pw[e] = h;
        } else {
          pw[e] = pack_bf16x2(p0 - as_f32(h << 16), p1 - as_f32(h & 0xFFFF0000u));
        }
      }
      l_run[t] = l_run[t] * alpha + psum;
      A[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]});
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * quad + i, 64);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) O[t][n][i] *= ar[i];
        }
      }
    }

    // ---- PV: B operand from LDS, transposed on read
    {
      const int r = (col >> 2);          // row inside the 4-token block
      const int c4 = (col & 3) * 4;      // 4 channels per lane address
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
        const lds_bf16x4* a0 = (const lds_bf16x4*)(
            (__attribute__((address_space(3))) uint8_t*)&s_v[0][4 * quad + r][2 * (16 * n + c4)]);
        const lds_bf16x4* a1 = (const lds_bf16x4*)(
            (__attribute__((address_space(3))) uint8_t*)&s_v[1][4 * quad + r][2 * (16 * n + c4)]);
        const u32x2_t w0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a0));
        const u32x2_t w1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a1));
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
        for (int t = 0; t < NT; ++t) O[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], B, O[t][n], 0, 0, 0);
      }
    }

    if (more) {
      cur[0] = nxt[0];
      cur[1] = nxt[1];
    }
  }

  // ---- epilogue: full row sums, hi + lo halves of O
  float lrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float l = l_run[t];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    lrow[t] = l;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) O[t][n][i] += __shfl_xor(O[t][n][i], 32, 64);
    }
  }

  // lanes 0..31 hold row 8t + 4*quad + i, channel 16n + col
  if (p.splits == 1) {
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float inv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float l = __shfl(lrow[t], (4 * quad + i) & 7, 64);
        inv[i] = (l > 0.0f) ? 1.0f / l : 0.0f;
      }
      if (lane < 32) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s_rows[(8 * t + 4 * quad + i) * kD + 16 * n + col] = O[t][n][i] * inv[i];
        }
      }
    }
    __syncthreads();
    if (p.rotate_out) fwht_rows_lds(s_rows, ROWS, kD, p.norm, lane, 64);
    for (int i = lane; i < p.rows * kD; i += 64) {
      const int r = i / kD;
      const int ch = i % kD;
      const int j = r / p.group;
      const int hh = r - j * p.group;
      p.out[(((size_t)b * p.n_q + j) * p.hq + (size_t)kvh * p.group + hh) * kD + ch] = s_rows[i];
    }
  } else {
    const size_t base = (((size_t)b * p.hkv + kvh) * p.splits + split) * ROWS;
    if (lane < 32) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) p.ws_o[(base + 8 * t + 4 * quad + i) * kD + 16 * n + col] = O[t][n][i];
        }
      }
    }
    if (lane < 8) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        p.ws_ml[(base + 8 * t + lane) * 2 + 0] = m_run[t];
        p.ws_ml[(base + 8 * t + lane) * 2 + 1] = lrow[t];
      }
    }
  }
}

// Combine the split partials of one (sequence, KV head): weights 2^(m_s - M),
// normalise by the combined sum, rotate back, store.
template <int NT>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeParams p) {
  constexpr int ROWS = 8 * NT;
  __shared__ float s_rows[ROWS * kD];
  __shared__ float s_w[ROWS][64];
  __shared__ float s_inv[ROWS];
  const int tid = threadIdx.x;
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const size_t base = ((size_t)b * p.hkv + kvh) * p.splits * ROWS;
  const int S = p.splits;
  // per-row weights (S <= 64 enforced by the planner)
  for (int r = tid; r < ROWS; r += blockDim.x) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, p.ws_ml[(base + (size_t)s * ROWS + r) * 2]);
    float lsum = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float m = p.ws_ml[(base + (size_t)s * ROWS + r) * 2];
      const float w = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      s_w[r][s] = w;
      lsum += w * p.ws_ml[(base + (size_t)s * ROWS + r) * 2 + 1];
    }
    s_inv[r] = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
  }
  __syncthreads();
  for (int i = tid; i < ROWS * kD; i += blockDim.x) {
    const int r = i / kD;
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) acc += s_w[r][s] * p.ws_o[(base + (size_t)s * ROWS) * kD + i];
    s_rows[i] = acc * s_inv[r];
  }
  __syncthreads();
  if (p.rotate_out) fwht_rows_lds(s_rows, ROWS, kD, p.norm, tid, blockDim.x);
  for (int i = tid; i < p.rows * kD; i += blockDim.x) {
    const int r = i / kD;
    const int ch = i % kD;
    const int j = r / p.group;
    const int hh = r - j * p.group;
    p.out[(((size_t)b * p.n_q + j) * p.hq + (size_t)kvh * p.group + hh) * kD + ch] = s_rows[i];
  }
}

template <int FMT, int NT>
hipError_t launch_nt(const DecodeParams& p, int batch, hipStream_t stream) {
  dim3 grid((unsigned)p.splits, (unsigned)p.hkv, (unsigned)batch);
  hipLaunchKernelGGL((decode_kernel<FMT, NT>), grid, dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL((merge_kernel<NT>), dim3((unsigned)p.hkv, (unsigned)batch), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const DecodeParams& p, int row_tiles, int batch, hipStream_t stream) {
  switch (row_tiles) {
    case 1: return launch_nt<FMT, 1>(p, batch, stream);
    case 2: return launch_nt<FMT, 2>(p, batch, stream);
    case 3: return launch_nt<FMT, 3>(p, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int plan_decode(const CacheGeom& c, int batch, int hq, int n_q, int max_context_len, uint32_t flags,
                DecodePlan* plan) {
  if (c.d != kD) return KVQ_ERR_UNSUPPORTED;
  const int group = hq / c.hkv;
  const int rows = group * n_q;
  const int row_tiles = (rows + 7) / 8;
  if (row_tiles > 3) return KVQ_ERR_UNSUPPORTED;
  const int n_tiles = (max_context_len + 15) / 16;
  int splits = (int)((flags & KVQ_SPLITS_MASK) >> KVQ_SPLITS_SHIFT);
  if (splits <= 0) {
    // Aim at ~4096 waves in total, each scanning at least 8 tiles (128 tokens).
    const long long units = (long long)batch * c.hkv;
    const long long want_tiles = ((long long)units * n_tiles + 4095) / 4096;
    long long per = want_tiles < 8 ? 8 : want_tiles;
    splits = (int)((n_tiles + per - 1) / per);
  }
  if (splits < 1) splits = 1;
  if (splits > 64) splits = 64;
  int per = (n_tiles + splits - 1) / splits;
  per = (per + 1) & ~1;  // tiles are processed in pairs
  if (per < 2) per = 2;
  splits = (n_tiles + per - 1) / per;
  if (splits < 1) splits = 1;
  plan->rows = rows;
  plan->row_tiles = row_tiles;
  plan->splits = splits;
  plan->tiles_per_split = per;
  plan->workspace = (splits > 1)
                        ? (size_t)batch * c.hkv * splits * (8 * row_tiles) * (kD + 2) * sizeof(float)
                        : 0;
  return KVQ_OK;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  DecodeParams p;
  p.kc = a.c.kc;
  p.ks = a.c.ks;
  p.vc = a.c.kv_shared ? a.c.kc : a.c.vc;
  p.vs = a.c.kv_shared ? a.c.ks : a.c.vs;
  p.c_head = a.c.c_head;
  p.c_page = a.c.c_page;
  p.s_head = a.c.s_head;
  p.s_page = a.c.s_page;
  p.P = a.c.p;
  p.hkv = a.c.hkv;
  p.q = a.q;
  p.hq = a.hq;
  p.n_q = a.n_q;
  p.group = a.group;
  p.rows = a.plan.rows;
  p.block_tables = a.block_tables;
  p.max_pages = a.max_pages;
  p.context_lens = a.context_lens;
  p.qscale = a.qscale;
  p.norm = fwht_norm(kD);
  p.rotate_q = a.rotate_q;
  p.rotate_out = a.rotate_out;
  p.splits = a.plan.splits;
  p.tiles_per_split = a.plan.tiles_per_split;
  p.out = a.out;
  const size_t n_o = (size_t)a.batch * a.c.hkv * a.plan.splits * (8 * a.plan.row_tiles) * kD;
  p.ws_o = a.workspace;
  p.ws_ml = a.workspace ? a.workspace + n_o : nullptr;
  if (a.c.fmt == KVQ_FMT_FP4_E2M1) return launch_fmt<KVQ_FMT_FP4_E2M1>(p, a.plan.row_tiles, a.batch, stream);
  return launch_fmt<KVQ_FMT_FP8_E4M3>(p, a.plan.row_tiles, a.batch, stream);
}

}  // namespace kvq

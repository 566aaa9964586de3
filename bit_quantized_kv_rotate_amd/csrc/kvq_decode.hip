// Decode attention over the paged FP4 (E2M1 + UE8M0 per 32 channels) cache,
// and over the FP8 (E4M3 + UE8M0 per 32) comparator cache.
//
// Method: ROCm blog "UltraQuant on AMD Instinct", section "What is
// UltraQuant?": CDNA4 matrix cores take FP4 operands directly and apply the
// power-of-two scale inside the scaled MFMA, with no separate dequantisation
// and no lookup table; section "Why UltraQuant beats 8-bit KV": a decode step
// re-reads the whole cache, so time follows the bytes moved.  Section
// "Throughput vs latency trade-off": an MTP verify step has several query
// positions per sequence; here they share one pass over the cache (the page
// names this fusion as future work).
//
// Design (gfx950, wave64, one wave per (sequence, KV head, context split)):
//  * The page scan streams 16-token tiles.  Lane l loads the code bytes of
//    token l%16, channel group l/16, plus that group's scale byte.
//  * QK^T runs on v_mfma_scale_f32_16x16x128_f8f6f4: the K codes (FP4, or
//    E4M3 for the comparator) and their UE8M0 scale bytes are the A operand
//    and A scale as loaded -- the FP4 operand layout of that instruction is
//    exactly one (token, 32-channel group) per lane.  The query (rotated and
//    pre-scaled by sm_scale * log2 e) is split into kQTerms E4M3 terms with
//    their own per-32 scales (each term carries the previous residual, ~4
//    more bits per term), two terms per MFMA in columns c and c + 8; one DPP
//    row rotate adds the halves.  Scores come out transposed (S^T: tokens x
//    query rows), which is directly the A operand layout of the PV product.
//  * V codes are converted with their scale (gfx950 scaled converts, 2
//    values per instruction) into a wave-private bf16 LDS tile and read back
//    transposed with ds_read_b64_tr_b16 as the B operand of PV; P is split
//    into bf16 hi + lo (8 rows each in the 16 MFMA rows).  fp32 accumulation.
//  * Online softmax in base 2 with lane-swap reductions; the O rescale runs
//    only when a row maximum moves.
//  * Codes are prefetched through a ring of kRing tile pairs held in
//    registers; refills are unconditional (clamped to the last tile) so the
//    memory wait counts stay exact.
//  * Context split into `splits` ranges; partial (m, l, O) go to the
//    workspace and a merge kernel combines them, normalises, rotates back.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kD = 128;              // head_dim handled by this kernel
constexpr int kQTerms = 6;           // FP6 (E2M3) terms of the pre-scaled query (FP4 cache)
constexpr int kQMfma = kQTerms / 2;  // scaled MFMAs per tile and row tile
constexpr int kVRow = 2 * kD + 32;   // LDS bytes per token row of V (bf16, padded)
constexpr int kRing = 2;             // tile pairs held in registers per wave

typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct DecodeParams {
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int64_t c_head, c_page, s_head, s_page;
  int P;
  int p_shift;  // log2(P)
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
struct Fmt {
  static constexpr bool kFP4 = FMT == KVQ_FMT_FP4_E2M1;
  static constexpr int kWords = kFP4 ? 4 : 8;      // uint32 of codes per (token, group)
};

// Query operands of the score product.
//  FP4 cache: kQTerms FP6 terms for the scaled MFMA (6 packed dwords + scale).
//  FP8 cache: bf16 hi + lo parts for the bf16 MFMA (4 k-steps of 32 channels).
template <int FMT, int NT>
struct QOps;
template <int NT>
struct QOps<KVQ_FMT_FP4_E2M1, NT> {
  i32x8_t b[NT][kQMfma];
  int sc[NT][kQMfma];
};
template <int NT>
struct QOps<KVQ_FMT_FP8_E4M3, NT> {
  bf16x8_t b[NT][4];
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

template <int FMT>
struct RawTile {
  uint32_t k[Fmt<FMT>::kWords];
  uint32_t v[Fmt<FMT>::kWords];
  uint32_t ksc, vsc;
};

template <int FMT>
__device__ __forceinline__ void load_tile(const DecodeParams& p, const int32_t* bt_row, int kvh,
                                          int tile, int lane, RawTile<FMT>& t) {
  const int tok = tile * 16;
  const int page = bt_row[tok >> p.p_shift];
  const int off = (tok & (p.P - 1)) + (lane & 15);
  const int grp = lane >> 4;
  const int64_t head = (int64_t)page * p.c_page + (int64_t)kvh * p.c_head;
  const int64_t sidx = (int64_t)page * p.s_page + (int64_t)kvh * p.s_head + (int64_t)grp * p.P + off;
  if constexpr (Fmt<FMT>::kFP4) {
    const int64_t cidx = head + ((int64_t)grp * p.P + off) * 16;
    const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.kc + cidx));
    const u32x4_t c = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.vc + cidx));
#pragma unroll
    for (int i = 0; i < 4; ++i) { t.k[i] = a[i]; t.v[i] = c[i]; }
  } else {
    const int64_t cidx = head + ((int64_t)grp * p.P + off) * 32;
    const u32x4_t a0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.kc + cidx));
    const u32x4_t a1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.kc + cidx + 16));
    const u32x4_t c0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.vc + cidx));
    const u32x4_t c1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.vc + cidx + 16));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t.k[i] = a0[i]; t.k[4 + i] = a1[i];
      t.v[i] = c0[i]; t.v[4 + i] = c1[i];
    }
  }
  t.ksc = p.ks[sidx];
  t.vsc = p.vs[sidx];
}

// Per-wave softmax / accumulator state.
template <int NT>
struct WaveState {
  f32x4_t O[NT][8];
  float m_run[NT];
  float l_run[NT];
};

template <int FMT>
__device__ __forceinline__ void issue_pair(const DecodeParams& p, const int32_t* bt_row, int kvh,
                                           int tile, int t_end, int lane, RawTile<FMT> (&r)[2]) {
  load_tile<FMT>(p, bt_row, kvh, min(tile, t_end - 1), lane, r[0]);
  load_tile<FMT>(p, bt_row, kvh, min(tile + 1, t_end - 1), lane, r[1]);
}

// One pair of 16-token tiles: scores, V staging, softmax update, PV.
// Once the codes of `r` are consumed, the loads of tile pair `refill` are
// issued into the same registers (clamped to the split's last tile).
template <int FMT, int NT>
__device__ __forceinline__ void compute_pair(const DecodeParams& p, const int32_t* bt_row, int kvh,
                                             int tile, int t_end, int refill, int tok_limit,
                                             int interior_limit, const int (&row_last)[NT],
                                             const QOps<FMT, NT>& q, RawTile<FMT> (&r)[2],
                                             uint8_t (*s_v)[16][kVRow], int lane,
                                             WaveState<NT>& st) {
  const int col = lane & 15;
  const int quad = lane >> 4;
  const bool hi_col = col < 8;

  // ---- scores S^T = K q^T
  f32x4_t S[2][NT];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if constexpr (Fmt<FMT>::kFP4) {
      // FP4 codes and UE8M0 scales straight into the scaled MFMA (A operand)
      const i32x8_t A = {(int)r[s].k[0], (int)r[s].k[1], (int)r[s].k[2], (int)r[s].k[3], 0, 0, 0, 0};
      const int ksc = (int)r[s].ksc;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < kQMfma; ++m)
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.b[t][m], acc, 4, 2, 0, ksc, 0,
                                                                 q.sc[t][m]);
        S[s][t] = acc;
      }
    } else {
      // E4M3 codes dequantised to bf16 (exact) as the A operand of bf16 MFMAs
      uint32_t kb[16];
      dequant_group<FMT>(r[s].k, scale_operand(r[s].ksc), kb);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4_t a = {kb[4 * ks], kb[4 * ks + 1], kb[4 * ks + 2], kb[4 * ks + 3]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), q.b[t][ks], acc,
                                                        0, 0, 0);
        }
        S[s][t] = acc;
      }
    }
  }

  // ---- V tiles -> LDS as bf16 token rows
  const bool interior = (tile * 16 + 32) <= interior_limit;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint32_t vb[16];
    dequant_group<FMT>(r[s].v, scale_operand(r[s].vsc), vb);
    if (!interior) {
      const int tok = (tile + s) * 16 + col;
      if (tok >= tok_limit) {
#pragma unroll
        for (int i = 0; i < 16; ++i) vb[i] = 0u;
      }
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&s_v[s][col][64 * quad]);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{vb[4 * i], vb[4 * i + 1], vb[4 * i + 2], vb[4 * i + 3]};
  }

  // the raw codes are consumed: start the next loads into the same registers
  issue_pair<FMT>(p, bt_row, kvh, refill, t_end, lane, r);

  // ---- B operands of PV (transposed LDS reads)
  bf16x8_t Bv[8];
  {
    const int rr = col >> 2;
    const int c4 = (col & 3) * 4;
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      lds_bf16x4* a0 = (lds_bf16x4*)((__attribute__((address_space(3))) uint8_t*)&s_v[0][4 * quad + rr][2 * (16 * n + c4)]);
      lds_bf16x4* a1 = (lds_bf16x4*)((__attribute__((address_space(3))) uint8_t*)&s_v[1][4 * quad + rr][2 * (16 * n + c4)]);
      const u32x2_t w0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a0));
      const u32x2_t w1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a1));
      Bv[n] = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
    }
  }

  // ---- softmax update and P (bf16 hi/lo) per row tile, then PV
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float sc[8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = S[s][t][i];
        sc[4 * s + i] = x + dpp_ror8(x);
      }
    }
    if (!interior) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = (tile + s) * 16 + 4 * quad + i;
          const bool ok = (tok < tok_limit) && (tok <= row_last[t]);
          sc[4 * s + i] = ok ? sc[4 * s + i] : -INFINITY;
        }
      }
    }
    float mloc = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                       fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mloc = quad_max(mloc);
    const float m_old = st.m_run[t];
    const float m_new = fmaxf(m_old, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    st.m_run[t] = m_new;
    float psum = 0.0f;
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(sc[2 * e] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(sc[2 * e + 1] - m_use);
      psum += p0 + p1;
      const uint32_t h = pack_bf16x2(p0, p1);
      const uint32_t l = pack_bf16x2(p0 - as_f32(h << 16), p1 - as_f32(h & 0xFFFF0000u));
      pw[e] = hi_col ? h : l;
    }
    if (__builtin_amdgcn_ballot_w64(m_new != m_old)) {
      // a row max moved in some lane: rescale (rare once the scan settles)
      const float alpha = __builtin_amdgcn_exp2f(m_old - m_use);
      st.l_run[t] *= alpha;
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * quad + i, 64);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st.O[t][n][i] *= ar[i];
      }
    }
    st.l_run[t] += psum;
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int n = 0; n < 8; ++n)
      st.O[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bv[n], st.O[t][n], 0, 0, 0);
  }
}

template <int FMT, int NT>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeParams p) {
  constexpr int ROWS = 8 * NT;
  // s_rows: query rows (prologue) and output rows (epilogue); s_work: packed
  // FP6 query terms (prologue, FP4 cache), then the V tiles of the page scan.
  constexpr int kQpBytes = kQTerms * ROWS * 4 * 24;
  constexpr int kVBytes = 2 * 16 * kVRow;
  constexpr int kWorkBytes = kQpBytes > kVBytes ? kQpBytes : kVBytes;
  __shared__ __attribute__((aligned(16))) float s_rows[ROWS * kD];
  __shared__ __attribute__((aligned(16))) uint8_t s_work[kWorkBytes];
  __shared__ uint8_t s_qsc[kQTerms][ROWS][4];
  uint8_t (*s_v)[16][kVRow] = reinterpret_cast<uint8_t (*)[16][kVRow]>(s_work);
  uint32_t* s_qp = reinterpret_cast<uint32_t*>(s_work);  // [kQTerms][ROWS][4 blocks][6 dwords]

  const int lane = threadIdx.x;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int L = p.context_lens[b];
  const int n_tiles = (L + 15) >> 4;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(n_tiles, t_begin + p.tiles_per_split);
  const int tok_limit = min(L, t_end * 16);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int32_t* bt_row = p.block_tables + (size_t)b * p.max_pages;
  const bool has_work = t_end > t_begin;
  const int n_pairs = has_work ? ((t_end - t_begin + 1) >> 1) : 0;
  const int n_iter = (n_pairs + kRing - 1) / kRing;

  // ---- start streaming the first tile pairs before the query prologue
  RawTile<FMT> ring[kRing][2];
  if (has_work) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) issue_pair<FMT>(p, bt_row, kvh, t_begin + 2 * u, t_end, lane, ring[u]);
  }

  // ---- query prologue: load, rotate, pre-scale
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

  QOps<FMT, NT> q;
  if constexpr (Fmt<FMT>::kFP4) {
    // ---- split each (row, 32-channel block) of the pre-scaled query into
    // kQTerms FP6 (E2M3) terms, each with its own UE8M0 scale and carrying
    // the previous residual.  Two lanes per (row, block), 16 channels each;
    // 16 six-bit codes are exactly 3 dwords of the operand bitstream.
    for (int pr = lane >> 1; pr < ROWS * 4; pr += 32) {
      const int row = pr >> 2;
      const int blk = pr & 3;
      const int half = lane & 1;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = s_rows[row * kD + 32 * blk + 16 * half + i] * p.qscale;
#pragma unroll 1
      for (int t = 0; t < kQTerms; ++t) {
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));
        const int byte = max((int)((as_u32(am) >> 23) & 0xFFu) - 2, 0);
        const int e = byte - 127;
        uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float val;
          const uint32_t c = e2m3_split(x[i], e, val);
          x[i] -= val;
          const int bit = 6 * i;
          w[bit >> 5] |= c << (bit & 31);
          if ((bit & 31) > 26) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
        }
        uint32_t* dst = s_qp + (((size_t)t * ROWS + row) * 4 + blk) * 6 + 3 * half;
        dst[0] = w[0];
        dst[1] = w[1];
        dst[2] = w[2];
        if (half == 0) s_qsc[t][row][blk] = (uint8_t)byte;
      }
    }
    __syncthreads();
    // B operands: lane (j = l/16, column n = l%16) holds the 32 codes of block
    // j for row 8t + (n & 7), term 2m + (n >= 8), with that block's scale.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int m = 0; m < kQMfma; ++m) {
        const int row = 8 * t + (col & 7);
        const int term = 2 * m + (col >> 3);
        const uint32_t* src = s_qp + (((size_t)term * ROWS + row) * 4 + quad) * 6;
        q.b[t][m] = i32x8_t{(int)src[0], (int)src[1], (int)src[2], (int)src[3], (int)src[4], (int)src[5], 0, 0};
        q.sc[t][m] = s_qsc[term][row][quad];
      }
    }
    __syncthreads();  // s_work becomes the V tile buffer
  } else {
    // ---- bf16 hi + lo parts of the pre-scaled query; lane group j covers
    // channels 32j + 8s .. 32j + 8s + 7 in k-step s (the K operand order)
    const bool hi_col = col < 8;
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
        q.b[t][s] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
  }

  WaveState<NT> st;
  int row_last[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st.m_run[t] = -INFINITY;
    st.l_run[t] = 0.0f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.O[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int r = 8 * t + (col & 7);
    row_last[t] = (r < p.rows) ? (L - p.n_q + r / p.group) : -1;
  }
  // Pairs entirely below this token need no mask for any valid row.  Padded
  // rows (r >= rows) have zero queries: exact zero scores, never stored.
  const int interior_limit = min(tok_limit, L - p.n_q + 1);

  // ---- page scan: ring of kRing tile pairs; the pair count is padded to a
  // multiple of kRing with fully masked pairs so every refill is unconditional
#pragma unroll 1
  for (int it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int pi = it * kRing + u;
      compute_pair<FMT, NT>(p, bt_row, kvh, t_begin + 2 * pi, t_end, t_begin + 2 * (pi + kRing),
                            tok_limit, interior_limit, row_last, q, ring[u], s_v, lane, st);
    }
  }

  // ---- epilogue: full row sums, hi + lo halves of O
  float lrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    lrow[t] = quad_sum(st.l_run[t]);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st.O[t][n][i] = add_half_swap(st.O[t][n][i]);
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
          for (int i = 0; i < 4; ++i) s_rows[(8 * t + 4 * quad + i) * kD + 16 * n + col] = st.O[t][n][i] * inv[i];
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
          for (int i = 0; i < 4; ++i) p.ws_o[(base + 8 * t + 4 * quad + i) * kD + 16 * n + col] = st.O[t][n][i];
        }
      }
    }
    if (lane < 8) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        p.ws_ml[(base + 8 * t + lane) * 2 + 0] = st.m_run[t];
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
  p.p_shift = __builtin_ctz((unsigned)a.c.p);
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

// Decode attention over a latent-width FP4 cache: head_dim 512, keys and
// values from the same rotated latent vectors (or separate ones), up to 64
// query rows per KV head (absorbed query heads x MTP positions).
//
// Method: ROCm blog "UltraQuant on AMD Instinct", section "What is
// UltraQuant?" (FP4 codes and their power-of-two scales straight into the
// scaled MFMA); the latent width and the absorbed query heads are the shape
// of the MLA-style models the blog's serving stack runs.
//
// At 64 rows x 512 channels the step is MFMA-bound, not HBM-bound: the query
// operands (four FP6 terms) and the output accumulators of 64 rows do not fit
// one wave, and the bf16 V operands must be shared.  One block of 8 waves
// per (sequence, KV head, context split):
//  * wave w is the score owner of rows 8w .. 8w + 7 (QK^T on the scaled
//    MFMA, online softmax, P split into bf16 hi + lo);
//  * wave w converts one 128-channel quarter of one tile of each tile pair
//    to bf16 into the shared LDS tile;
//  * wave w accumulates O for all rows over channels 64w .. 64w + 63: hi
//    and lo of P are two A operands of 16 full rows x 32 tokens against the
//    same V operand, accumulated into one accumulator.
// P (as ready MFMA A operands), the rescale factors and V pass through LDS,
// double-buffered by tile-pair parity: one barrier per pair.  Above 32 rows
// (three or four 16-row groups) decode512r_kernel splits the same work by
// role instead (four waves score, four accumulate), with bitwise the same
// partials.
#include <atomic>

#include "kvq_decode_common.h"

namespace kvq {
namespace {

constexpr int kD5 = 512;
constexpr int kT5 = 4;               // FP6 query terms
constexpr int kM5 = kT5 / 2;         // scaled MFMAs per 128-channel block (two terms each)
constexpr int kW5 = 8;               // waves per block
constexpr int kVRow5 = 2 * kD5 + 32;  // LDS bytes per bf16 token row (padded)
constexpr int kMaxRG5 = 4;           // 16-row groups (64 rows)
constexpr int kRoleSplitRG5 = 3;     // from three 16-row groups (33 rows) on, the role-split kernel
// tile pairs in flight per wave (one chunk each): three, fewer where the
// accumulators of 64 rows (and a separate V chunk, or the per-lane addresses
// of a gathered selection) leave no room
template <int RG, bool SHARED, bool SEL>
struct Ring5 {
  static constexpr int kN = RG >= 4 ? (SHARED && !SEL ? 2 : 1) : (SHARED || RG <= 2 ? 3 : 2);
};

// Raw codes of the one (tile, 128-channel chunk) of a tile pair this wave
// stages: lane l holds token l%16, channel group 4 chunk + l/16 (16 code
// bytes) and that group's scale byte; V likewise for a separate V cache.
struct Chunk5 {
  uint32_t k[4];
  uint32_t ksc;
  uint32_t v[4];
  uint32_t vsc;
};

// FLAT (cache arrays below 4 GiB): one buffer resource per array from this
// head on (loop-invariant), the page as the 32-bit scalar offset; else one
// resource per (page, head) block.
template <bool SHARED, bool SEL, bool FLAT>
__device__ __forceinline__ void load_chunk5(const DecodeParams& p, const int32_t* bt_row, const int32_t* sel_row,
                                            int L, int kvh, int tile, int chunk, int lane, Chunk5& t) {
  if constexpr (SEL) {
    // list entry tile*16 + token of this lane (clamped to the list; entries
    // past it are masked), gathered through the block table: every lane
    // addresses its own page
    const int j = min(tile * 16 + (lane & 15), L - 1);
    const int pos = sel_row[j];
    const int page = bt_row[pos >> p.p_shift];
    const int in_page = pos & (p.P - 1);
    const int grp = 4 * chunk + (lane >> 4);
    const int64_t coff = (int64_t)page * p.c_page + (int64_t)kvh * p.c_head + ((int64_t)grp * p.P + in_page) * 16;
    const int64_t soff = (int64_t)page * p.s_page + (int64_t)kvh * p.s_head + (int64_t)grp * p.P + in_page;
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p.kc + coff);
#pragma unroll
    for (int w = 0; w < 4; ++w) t.k[w] = a[w];
    t.ksc = p.ks[soff];
    if constexpr (!SHARED) {
      const u32x4_t c = *reinterpret_cast<const u32x4_t*>(p.vc + coff);
#pragma unroll
      for (int w = 0; w < 4; ++w) t.v[w] = c[w];
      t.vsc = p.vs[soff];
    }
    return;
  }
  const int tok = tile * 16;
  const int page = __builtin_amdgcn_readfirstlane(bt_row[tok >> p.p_shift]);
  const int in_page = tok & (p.P - 1);
  const int idx = (4 * chunk + (lane >> 4)) * p.P + (lane & 15);
  const int64_t ch = (int64_t)kvh * p.c_head, sh = (int64_t)kvh * p.s_head;
  int64_t cb, sb, cn, sn;
  int coff, soff;
  if constexpr (FLAT) {
    cb = ch;
    sb = sh;
    cn = p.c_total - ch;
    sn = p.s_total - sh;
    coff = (int)((uint32_t)page * (uint32_t)p.c_page + (uint32_t)in_page * 16u);
    soff = (int)((uint32_t)page * (uint32_t)p.s_page + (uint32_t)in_page);
  } else {
    cb = (int64_t)page * p.c_page + ch;
    sb = (int64_t)page * p.s_page + sh;
    cn = p.c_head;
    sn = p.s_head;
    coff = in_page * 16;
    soff = in_page;
  }
  const __amdgpu_buffer_rsrc_t rk = block_rsrc(p.kc, cb, cn);
  const __amdgpu_buffer_rsrc_t rks = block_rsrc(p.ks, sb, sn);
  const u32x4_t a = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, idx * 16, coff, 2));
#pragma unroll
  for (int w = 0; w < 4; ++w) t.k[w] = a[w];
  t.ksc = __builtin_amdgcn_raw_buffer_load_b8(rks, idx, soff, 0);
  if constexpr (!SHARED) {
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(p.vc, cb, cn);
    const __amdgpu_buffer_rsrc_t rvs = block_rsrc(p.vs, sb, sn);
    const u32x4_t c = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, idx * 16, coff, 2));
#pragma unroll
    for (int w = 0; w < 4; ++w) t.v[w] = c[w];
    t.vsc = __builtin_amdgcn_raw_buffer_load_b8(rvs, idx, soff, 0);
  }
}

// Query prologue for the 512-wide kernel, one wave per query row (rows of a
// KV head padded to 16 RG): load, rotate, pre-scale, split into kT5 FP6
// terms per 32-channel block and store the score B operands.  8-row owners
// (R16 false): [B][hkv][2 RG owners][4 blocks][kM5][64 lanes][8 dwords],
// two terms per MFMA in columns c and c + 8.  16-row groups (R16, the
// role-split kernel): [B][hkv][RG groups][4 blocks][kT5 terms][64 lanes][8
// dwords], one term of 16 rows per MFMA.  Lane l holds channels 8l .. 8l +
// 7; a 32-channel block is 4 lanes whose 8 six-bit codes (48 bits each) make
// the block's 192-bit stream.
template <int RG, bool CONV, bool R16 = false>
__global__ __launch_bounds__(256) void qprep512_kernel(const DecodeParams p) {
  constexpr int ROWS = 16 * RG;
  constexpr int NO = 2 * RG;  // score owners
  const int lane = threadIdx.x & 63;
  const int gr = blockIdx.x * 4 + (threadIdx.x >> 6);  // grid covers exactly B * hkv * ROWS
  const int r = gr % ROWS;
  const int bh = gr / ROWS;
  const int kvh = bh % p.hkv;
  const int b = bh / p.hkv;

  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.0f;
  if (r < p.rows) {
    const int j = r / p.group;
    const int hh = r - j * p.group;
    const uint16_t* src = p.q + (((size_t)b * p.n_q + j) * p.hq + (size_t)kvh * p.group + hh) * kD5 + 8 * lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = bf16_to_f32(src[i]);
  }
  if (p.rotate_q) wave_fwht<8>(x, lane, p.norm);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = x[i] * p.qscale;

  const int owner = r >> 3;
  if constexpr (CONV) {
    // bf16 hi + lo operands of the conversion route, [B][hkv][owners][4
    // chunks][4 k-steps][64 lanes][4 dwords]: k-step j of chunk c holds, in
    // operand lane 16 quad + col, channels 128 c + 32 quad + 8 j .. + 7 of the
    // owner's row col & 7 (hi for col < 8, lo for col >= 8) - exactly the
    // eight channels this lane holds (lane = 16 c + 4 quad + j)
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h0 = f32_to_bf16_rne(x[2 * i]), h1 = f32_to_bf16_rne(x[2 * i + 1]);
      const uint32_t l0 = f32_to_bf16_rne(x[2 * i] - bf16_to_f32((uint16_t)h0));
      const uint32_t l1 = f32_to_bf16_rne(x[2 * i + 1] - bf16_to_f32((uint16_t)h1));
      hi[i] = h0 | (h1 << 16);
      lo[i] = l0 | (l1 << 16);
    }
    const int c = lane >> 4, quad = (lane >> 2) & 3, j = lane & 3;
    uint32_t* dst = p.qops + (((((size_t)bh * NO + owner) * 4 + c) * 4 + j) * 64 + 16 * quad + (r & 7)) * 4;
    *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
    *reinterpret_cast<u32x4_t*>(dst + 8 * 4) = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
    return;
  }
  const int gi = lane >> 2;  // 32-channel group of the lane
  const int blk = gi >> 2;
  const int q = gi & 3;
  const int j4 = lane & 3;
  const int base = lane & ~3;
  const int sa = base + min(j4, 2);
#pragma unroll
  for (int t = 0; t < kT5; ++t) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
    am = fmaxf(am, dpp_f32<kDppXor1>(am));
    am = fmaxf(am, dpp_f32<kDppXor2>(am));
    const int byte = max((int)((as_u32(am) >> 23) & 0xFFu) - 2, 0);
    const int e = byte - 127;
    uint64_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v;
      const uint32_t c = e2m3_split(x[i], e, v);
      x[i] -= v;
      bits |= (uint64_t)c << (6 * i);
    }
    const uint32_t lo = (uint32_t)bits;
    const uint32_t hi = (uint32_t)(bits >> 32);  // 16 bits
    const uint32_t alo = (uint32_t)__shfl((int)lo, sa, 64);
    const uint32_t ahi = (uint32_t)__shfl((int)hi, sa, 64);
    const uint32_t blo = (uint32_t)__shfl((int)lo, sa + 1, 64);
    const uint32_t bhi = (uint32_t)__shfl((int)hi, sa + 1, 64);
    uint32_t d0, d1;
    if (j4 == 0) {
      d0 = alo;
      d1 = ahi | (blo << 16);
    } else if (j4 == 1) {
      d0 = (alo >> 16) | (ahi << 16);
      d1 = blo;
    } else if (j4 == 2) {
      d0 = ahi | (blo << 16);
      d1 = (blo >> 16) | (bhi << 16);
    } else {
      d0 = (uint32_t)byte;
      d1 = 0u;
    }
    uint32_t* dst;
    if constexpr (R16) {
      dst = p.qops + (((((size_t)bh * RG + (r >> 4)) * 4 + blk) * kT5 + t) * 64 + 16 * q + (r & 15)) * 8 + 2 * j4;
    } else {
      const int m = t >> 1;
      const int col = (r & 7) + 8 * (t & 1);
      dst = p.qops + (((((size_t)bh * NO + owner) * 4 + blk) * kM5 + m) * 64 + 16 * q + col) * 8 + 2 * j4;
    }
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{d0, d1};
  }
}

// Score contribution of one 128-channel chunk: K codes (FP4) and scale
// byte as the A operand, the two FP6 query-term MFMAs of that chunk as B;
// the query scale byte sits in byte 2 (C & 1) + m of register C / 2.
template <int C>
__device__ __forceinline__ f32x4_t qk_chunk5(f32x4_t acc, const u32x4_t kc, int ksc,
                                             const i32x8_t (&qb)[4][kM5], const int (&qs)[2]) {
  const i32x8_t A = {(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, qb[C][0], acc, 4, 2, 0, ksc, 2 * (C & 1), qs[C >> 1]);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, qb[C][1], acc, 4, 2, 0, ksc, 2 * (C & 1) + 1,
                                                         qs[C >> 1]);
  return acc;
}

// The conversion route's form of qk_chunk5: the chunk's K codes are
// converted with their scale to bf16 (kb, 16 dwords: channels 32 g .. 32 g
// + 31 of the lane's group g), and k-step j multiplies dwords 4 j .. 4 j + 3
// against the bf16 hi / lo query operand qv[j] (columns c < 8 hold hi of row
// c, c >= 8 lo of row c - 8, so x + its ror-8 partner is the row's score, as
// on the native route).
template <int J>
__device__ __forceinline__ f32x4_t qk_chunk5_conv(f32x4_t acc, const uint32_t (&kb)[16], const bf16x8_t (&qv)[J]) {
  static_assert(J == 4, "four k-steps per chunk");
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t a = {kb[4 * j], kb[4 * j + 1], kb[4 * j + 2], kb[4 * j + 3]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qv[j], acc, 0, 0, 0);
  }
  return acc;
}

// Query operands of one score owner on the conversion route.
template <int J>
__device__ __forceinline__ void load_qconv5(const DecodeParams& p, int bh, int NO, int owner, int lane,
                                            bf16x8_t (&qv)[4][J]) {
  static_assert(J == 4, "four k-steps per chunk");
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qv[c][j] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(p.qops + (((((size_t)bh * NO + owner) * 4 + c) * 4 + j) * 64 + lane) * 4));
}

// Byte J of a transposed code read (the channel pair of one token) to two
// bf16, with that token's scale: byte J of `sb`.
// (the scale operand byte << 23 in one SDWA shift)
template <int J>
__device__ __forceinline__ uint32_t cvt_token(int codes, uint32_t sb, uint32_t k23) {
  uint32_t s;
  if constexpr (J == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(s) : "v"(k23), "v"(sb));
  else if constexpr (J == 1)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(s) : "v"(k23), "v"(sb));
  else if constexpr (J == 2)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(s) : "v"(k23), "v"(sb));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(s) : "v"(k23), "v"(sb));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((uint32_t)codes, as_f32(s), J));
}

// Online softmax of one 8-row score owner over a tile pair, from its scores
// S (tile t, token 4 quad + i; column c of the MFMA output holds query-term
// half c / 8 of row c & 7, so x + its ror-8 partner is the row's score):
// masked past row_lim, lazy reference maximum (kLazyLog2), P split into bf16
// hi (lanes c < 8) and lo (c >= 8) and stored as PV A operands in the
// owner's slot of a 16-row group (`sp`: the group's two k-halves, `half`:
// the owner's 8 rows within it); the rows' rescale factors go to alpha[0..7]
// and whether any reference moved to *flag.
__device__ __forceinline__ void owner_softmax(const f32x4_t (&S)[2], int tile, int row_lim, int lane, int half,
                                              float& m_run, float& l_run, u32x4_t (*sp)[64], float* alpha,
                                              int* flag) {
  const int col = lane & 15;
  const int quad = lane >> 4;
  const bool hi_col = col < 8;
  float sc[8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = S[t][i];
      const int tok = (tile + t) * 16 + 4 * quad + i;
      sc[4 * t + i] = (tok <= row_lim) ? x + dpp_ror8(x) : -INFINITY;
    }
  }
  float mloc = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  mloc = quad_max(mloc);
  // lazy reference maximum (kLazyLog2): most pairs leave it, and so the
  // output rows, unchanged
  const float m_old = m_run;
  const float m_tgt = fmaxf(m_old, mloc);
  const bool grow = m_tgt > m_old + kLazyLog2;
  const float m_new = grow ? m_tgt : m_old;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  m_run = m_new;
  float psum = 0.0f;
  uint32_t pw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(sc[2 * e] - m_use);
    const float p1 = __builtin_amdgcn_exp2f(sc[2 * e + 1] - m_use);
    psum += p0 + p1;
    const uint32_t u0 = as_u32(p0), u1 = as_u32(p1);
    const uint32_t h = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    const uint32_t l = pack_bf16x2(p0 - as_f32(u0 & 0xFFFF0000u), p1 - as_f32(u1 & 0xFFFF0000u));
    pw[e] = hi_col ? h : l;
  }
  // A operand of the hi part (slot 0) or the lo part (slot 1) of the
  // 16-row group: lane k-group quad (tokens 4 quad .. 4 quad + 3 of both
  // tiles), row 8 half + (col & 7)
  sp[hi_col ? 0 : 1][16 * quad + 8 * half + (col & 7)] = u32x4_t{pw[0], pw[1], pw[2], pw[3]};
  const float a = __builtin_amdgcn_exp2f(m_old - m_use);
  l_run = l_run * a + psum;
  if (lane < 8) alpha[lane] = a;
  const bool moved = __builtin_amdgcn_ballot_w64(grow) != 0;
  if (lane == 0) *flag = moved ? 1 : 0;
}

// Online softmax of one 16-row score group over a tile pair (role-split
// kernel, native scores): S (tile t, token 4 quad + i) holds row `col` of
// the group in column col.  Masked past row_lim when `masked`; lazy
// reference maximum; P split into bf16 hi and lo, stored as the group's two
// PV A operands (slot 0: hi, slot 1: lo; lane 16 quad + col); the rows'
// rescale factors go to alpha[0..15] and whether any reference moved to
// flag[0] and flag[1] (the group's two 8-row halves).
__device__ __forceinline__ void group_softmax(const f32x4_t (&S)[2], int tile, int row_lim, bool masked, int lane,
                                              float& m_run, float& l_run, u32x4_t (*sp)[64], float* alpha,
                                              int* flag) {
  const int quad = lane >> 4;
  float sc[8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[4 * t + i] = S[t][i];
  if (masked) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * t + i] = ((tile + t) * 16 + 4 * quad + i <= row_lim) ? sc[4 * t + i] : -INFINITY;
  }
  float mloc = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  mloc = quad_max(mloc);
  const float m_old = m_run;
  const float m_tgt = fmaxf(m_old, mloc);
  const bool grow = m_tgt > m_old + kLazyLog2;
  const float m_new = grow ? m_tgt : m_old;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  m_run = m_new;
  float psum = 0.0f;
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(sc[2 * e] - m_use);
    const float p1 = __builtin_amdgcn_exp2f(sc[2 * e + 1] - m_use);
    psum += p0 + p1;
    const uint32_t u0 = as_u32(p0), u1 = as_u32(p1);
    h[e] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    l[e] = pack_bf16x2(p0 - as_f32(u0 & 0xFFFF0000u), p1 - as_f32(u1 & 0xFFFF0000u));
  }
  sp[0][lane] = u32x4_t{h[0], h[1], h[2], h[3]};
  sp[1][lane] = u32x4_t{l[0], l[1], l[2], l[3]};
  const float a = __builtin_amdgcn_exp2f(m_old - m_use);
  l_run = l_run * a + psum;
  if (lane < 16) alpha[lane] = a;
  const bool moved = __builtin_amdgcn_ballot_w64(grow) != 0;
  if (lane < 2) flag[lane] = moved ? 1 : 0;
}

// SEL: the scan runs over the list of selected positions of each sequence
// (p.sel; context_lens are the list lengths), one query position per
// sequence.
template <int RG, bool SHARED, bool SEL, bool CONV = false, bool FLAT = true>
__global__ __launch_bounds__(512) void decode512_kernel(const DecodeParams p) {
  constexpr int ROWS = 16 * RG;
  constexpr int NO = 2 * RG;
  // staged K codes / scales for the scores (by pair parity), bf16 V rows
  // (three buffers: a pair is staged while the previous one is still read),
  // P as PV A operands and the rescale factors (by pair parity)
  __shared__ __attribute__((aligned(16))) u32x4_t s_k[2][2][4][64];
  __shared__ uint32_t s_ks[2][2][4][64];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[3][2][16][kVRow5];
  __shared__ __attribute__((aligned(16))) u32x4_t s_p[2][RG][2][64];
  __shared__ float s_alpha[2][ROWS];
  __shared__ int s_flag[2][NO];

  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (staged tile and
  // chunk, buffer offsets) stays in SGPRs, with no per-lane loops
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int bh = b * p.hkv + kvh;
  const int L = p.context_lens[b];
  const int n_tiles = (L + 15) >> 4;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(n_tiles, t_begin + p.tiles_per_split);
  const int tok_limit = min(L, t_end * 16);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int32_t* bt_row = p.block_tables + (size_t)b * p.max_pages;
  const int32_t* sel_row = SEL ? p.sel + (size_t)b * p.sel_stride : nullptr;
  const int n_pairs = (t_end > t_begin) ? ((t_end - t_begin + 1) >> 1) : 0;
  constexpr int kRing5 = Ring5<RG, SHARED, SEL>::kN;
  const int n_iter = (n_pairs + kRing5 - 1) / kRing5;  // pairs padded to a multiple of kRing5
  const bool owner = (NO == kW5) || w < NO;  // every wave owns rows at 64 rows
  const int mtile = w & 1;   // tile of each pair this wave stages
  const int mchunk = w >> 1;  // ... and its 128-channel chunk

  // stage pair pi (codes in `c`): K codes and scales for the scores, V as
  // bf16 rows (zero past the context; branch-free)
  auto stage = [&](int pi, const Chunk5& c) {
    const int tile = t_begin + 2 * pi + mtile;
    s_k[pi & 1][mtile][mchunk][lane] = u32x4_t{c.k[0], c.k[1], c.k[2], c.k[3]};
    s_ks[pi & 1][mtile][mchunk][lane] = c.ksc;
    const bool dead = tile * 16 + col >= tok_limit;
    uint32_t vw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vw[i] = dead ? 0u : (SHARED ? c.k[i] : c.v[i]);
    const uint32_t vsc = dead ? 0u : (SHARED ? c.ksc : c.vsc);
    uint32_t vb[16];
    dequant_group<KVQ_FMT_FP4_E2M1>(vw, scale_operand(vsc), vb);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&s_v[pi % 3][mtile][col][2 * (128 * mchunk + 32 * quad)]);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{vb[4 * i], vb[4 * i + 1], vb[4 * i + 2], vb[4 * i + 3]};
  };
  // refill a ring slot with pair pi (clamped to the split's last tile)
  auto fetch = [&](int pi, Chunk5& c) {
    load_chunk5<SHARED, SEL, FLAT>(p, bt_row, sel_row, L, kvh, min(t_begin + 2 * pi + mtile, t_end - 1), mchunk, lane, c);
  };

  Chunk5 ring[kRing5];
  if (n_pairs > 0) {
#pragma unroll
    for (int u = 0; u < kRing5; ++u) fetch(u, ring[u]);
  }

  // score owner: query operands of rows 8w .. 8w + 7; their eight scale
  // bytes packed four to a register (the MFMA's scale op_sel picks the byte)
  i32x8_t qb[4][kM5];
  int qs[2] = {0, 0};
  bf16x8_t qv[4][CONV ? 4 : 1];
  if constexpr (CONV) {
    if (owner) load_qconv5(p, bh, NO, w, lane, qv);
  }
  if (owner && !CONV) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int m = 0; m < kM5; ++m) {
        const uint32_t* src = p.qops + (((((size_t)bh * NO + w) * 4 + c) * kM5 + m) * 64 + lane) * 8;
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(src);
        const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(src + 4);
        qb[c][m] = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], 0, 0};
        qs[c >> 1] |= (int)((a1[2] & 0xFFu) << (8 * (2 * (c & 1) + m)));
      }
    }
  }
  const int row = 8 * w + (col & 7);  // owner's row in this lane
  // last token this lane's row may see (context end, MTP causal rule)
  const int row_lim = (owner && row < p.rows) ? min(tok_limit - 1, L - p.n_q + row / p.group) : -1;
  float m_run = -INFINITY, l_run = 0.0f;

  // owner: scores of pair pi, online softmax, P hi / lo as PV A operands,
  // rescale factors (branch-free: one basic block with the PV product)
  auto scores = [&](int pi) {
    const int par = pi & 1;
    const int tile = t_begin + 2 * pi;
    f32x4_t S[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (CONV) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4_t kc = s_k[par][s][c][lane];
          const uint32_t kw[4] = {kc[0], kc[1], kc[2], kc[3]};
          uint32_t kb[16];
          dequant_group<KVQ_FMT_FP4_E2M1>(kw, scale_operand(s_ks[par][s][c][lane]), kb);
          acc = qk_chunk5_conv(acc, kb, qv[c]);
        }
      } else {
        acc = qk_chunk5<0>(acc, s_k[par][s][0][lane], (int)s_ks[par][s][0][lane], qb, qs);
        acc = qk_chunk5<1>(acc, s_k[par][s][1][lane], (int)s_ks[par][s][1][lane], qb, qs);
        acc = qk_chunk5<2>(acc, s_k[par][s][2][lane], (int)s_ks[par][s][2][lane], qb, qs);
        acc = qk_chunk5<3>(acc, s_k[par][s][3][lane], (int)s_ks[par][s][3][lane], qb, qs);
      }
      S[s] = acc;
    }
    owner_softmax(S, tile, row_lim, lane, w & 1, m_run, l_run, s_p[par][w >> 1], &s_alpha[par][8 * w], &s_flag[par][w]);
  };

  f32x4_t O[RG][4];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int n = 0; n < 4; ++n) O[g][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: stage pairs 0 and 1, scores of pair 0
  if (n_pairs > 0) {
    stage(0, ring[0]);
    fetch(kRing5, ring[0]);
  }
  __syncthreads();
  if (n_pairs > 0) {
    stage(1, ring[1 % kRing5]);
    fetch(1 + kRing5, ring[1 % kRing5]);
    if (owner) scores(0);
  }
  __syncthreads();

  // ---- segment pi: PV of pair pi, scores of pair pi + 1, staging of pair
  // pi + 2; one barrier per segment
#pragma unroll 1
  for (int it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int u = 0; u < kRing5; ++u) {
      const int pi = it * kRing5 + u;
      const int par = pi & 1;
      // rescale O by the factors of pair pi (rows 16g + 4 quad + i belong to
      // owner 2g + (quad >> 1)), then load its P operands
      bf16x8_t A[RG][2];
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        if (s_flag[par][2 * g] | s_flag[par][2 * g + 1]) {
          float ar[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ar[i] = s_alpha[par][16 * g + 4 * quad + i];
#pragma unroll
          for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[g][n][i] *= ar[i];
        }
        A[g][0] = __builtin_bit_cast(bf16x8_t, s_p[par][g][0][lane]);
        A[g][1] = __builtin_bit_cast(bf16x8_t, s_p[par][g][1][lane]);
      }
      // scores of the next pair (its codes were staged a segment ago); past
      // the last pair the staged tiles lie beyond the context and every
      // score is masked, so the call leaves the softmax state unchanged
      if (owner) scores(pi + 1);
      // PV over channels 64w .. 64w + 63 for every row group
      const int vb = pi % 3;
      const int rr = col >> 2;
      const int c4 = (col & 3) * 4;
      typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
      // one B operand (the pair's 32 tokens x 16 channels) serves the hi
      // and the lo MFMA of every row group
      // one LDS base per pair; the reads of tile 1 and of channel tile n
      // are constant offsets from it
      // (the buffer offset is made uniform so that the compiler keeps one
      // lane address instead of one per read)
      const int vbuf = __builtin_amdgcn_readfirstlane(vb * (int)sizeof(s_v[0]));
      __attribute__((address_space(3))) uint8_t* const vrow =
          (__attribute__((address_space(3))) uint8_t*)&s_v[0][0][4 * quad + rr][2 * (64 * w + c4)] + vbuf;
      auto read_b = [&](int n) {
        lds_bf16x4* a0 = (lds_bf16x4*)(vrow + 32 * n);
        lds_bf16x4* a1 = (lds_bf16x4*)(vrow + 16 * kVRow5 + 32 * n);
        const u32x2_t w0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a0));
        const u32x2_t w1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a1));
        return __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
      };
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8_t B = read_b(n);
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          O[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][0], B, O[g][n], 0, 0, 0);
          O[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][1], B, O[g][n], 0, 0, 0);
        }
      }
      // stage pair pi + 2 from the ring, refill the slot
      {
        const int su = (u + 2) % kRing5;
        stage(pi + 2, ring[su]);
        fetch(pi + 2 + kRing5, ring[su]);
      }
      __syncthreads();
    }
  }

  // ---- partials: O rows 16g + 4 quad + i, channel 64w + 16n + col; (m, l)
  const size_t base = ((size_t)bh * p.splits + split) * ROWS;
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.ws_o[(base + 16 * g + 4 * quad + i) * kD5 + 64 * w + 16 * n + col] = O[g][n][i];
  const float lrow = quad_sum(l_run);
  if (owner && lane < 8) {
    p.ws_ml[(base + 8 * w + lane) * 2 + 0] = m_run;
    p.ws_ml[(base + 8 * w + lane) * 2 + 1] = lrow;
  }
}

// Role-split form of the kernel above for 33..64 rows, with the same
// arithmetic per accumulator (its partials are bitwise those of
// decode512_kernel).  Waves 0..3 score: wave s owns the 8-row owners 2s and
// 2s + 1 (QK^T, online softmax, P hi / lo), so each K operand it reads from
// LDS serves two owners.  Waves 4..7 own the output: wave 4 + v accumulates
// O for all rows over channels 128v .. 128v + 127 and stages both tiles of
// chunk v of each pair.  Waves go round-robin onto the four SIMDs, so every
// SIMD holds one wave of each role: the softmax VALU of one runs beside the
// PV MFMAs of the other, and the LDS reads per pair drop by a third (K read
// by four owners' waves instead of eight, P by four output waves).  With
// fewer rows the score waves' two softmax chains are the longer path and
// the plain kernel is faster.
template <int RG, bool SHARED, bool SEL, bool CONV = false, bool FLAT = true>
__global__ __launch_bounds__(512) void decode512r_kernel(const DecodeParams p) {
  constexpr int ROWS = 16 * RG;
  constexpr int NO = 2 * RG;
  constexpr int kRing = 1;  // tile pairs in flight per staging wave (a deeper ring spills)
  // staged FP4 codes, three buffers (pair i + 2 is staged while the scores
  // read pair i + 1 and PV reads pair i): K as the score MFMA's A operand,
  // with its scale bytes; V (the K codes themselves when K = V) is read by
  // the PV waves straight from these codes, with its scale bytes in
  // s_vsb[buf][tile][chunk][token / 4][group][token % 4] (zero past the
  // context)
  __shared__ __attribute__((aligned(16))) u32x4_t s_k[3][2][4][64];
  __shared__ uint32_t s_ks[3][2][4][64];
  __shared__ __attribute__((aligned(16))) u32x4_t s_vc[SHARED ? 1 : 3][2][4][64];
  __shared__ __attribute__((aligned(16))) uint8_t s_vsb[3][2][4][64];
  __shared__ __attribute__((aligned(16))) u32x4_t s_p[2][RG][2][64];
  __shared__ float s_alpha[2][ROWS];
  __shared__ int s_flag[2][NO];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int bh = b * p.hkv + kvh;
  const int L = p.context_lens[b];
  const int n_tiles = (L + 15) >> 4;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(n_tiles, t_begin + p.tiles_per_split);
  const int tok_limit = min(L, t_end * 16);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int32_t* bt_row = p.block_tables + (size_t)b * p.max_pages;
  const int32_t* sel_row = SEL ? p.sel + (size_t)b * p.sel_stride : nullptr;
  const int n_pairs = (t_end > t_begin) ? ((t_end - t_begin + 1) >> 1) : 0;
  const int n_iter = (n_pairs + kRing - 1) / kRing;  // pairs padded to a multiple of kRing
  const size_t base = ((size_t)bh * p.splits + split) * ROWS;

  if (w < 4) {
    // ---------------- score wave: rows 16w .. 16w + 15 (owners 2w, 2w + 1)
    const int s = w;
    const bool active = 2 * s < NO;
    if constexpr (!CONV) {
      // native scores: one FP6 query term of the 16 rows per scaled MFMA
      // (column = row), four terms and four 128-channel chunks per tile
      i32x8_t qb[4][kT5];
      int qs[4] = {0, 0, 0, 0};
      if (active) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int tm = 0; tm < kT5; ++tm) {
            const uint32_t* src = p.qops + (((((size_t)bh * RG + s) * 4 + c) * kT5 + tm) * 64 + lane) * 8;
            const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(src);
            const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(src + 4);
            qb[c][tm] = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], 0, 0};
            qs[c] |= (int)((a1[2] & 0xFFu) << (8 * tm));
          }
      }
      const int row = 16 * s + col;
      const int row_lim = (active && row < p.rows) ? min(tok_limit - 1, L - p.n_q + row / p.group) : -1;
      // pairs ending at or below every real row's last visible token need
      // no mask (padding rows have zero queries and are never read back)
      int vis = row_lim >= 0 ? row_lim : 0x7FFFFFFF;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) vis = min(vis, __shfl_xor(vis, o, 64));
      vis = __builtin_amdgcn_readfirstlane(vis);
      float m_run = -INFINITY, l_run = 0.0f;
      auto scores = [&](int pi) {
        const int par = pi & 1;
        const int kbuf = pi % 3;
        const int tile = t_begin + 2 * pi;
        f32x4_t S[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          // two accumulators (even and odd chunks) halve the MFMA chain
          f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const u32x4_t kc = s_k[kbuf][tt][c][lane];
            const int ksc = (int)s_ks[kbuf][tt][c][lane];
            const i32x8_t A = {(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
            f32x4_t& acc = (c & 1) ? a1 : a0;
            // the query scale of term tm is byte tm of qs[c]
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, qb[c][0], acc, 4, 2, 0, ksc, 0, qs[c]);
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, qb[c][1], acc, 4, 2, 0, ksc, 1, qs[c]);
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, qb[c][2], acc, 4, 2, 0, ksc, 2, qs[c]);
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, qb[c][3], acc, 4, 2, 0, ksc, 3, qs[c]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) S[tt][i] = a0[i] + a1[i];
        }
        group_softmax(S, tile, row_lim, tile * 16 + 31 > vis, lane, m_run, l_run, s_p[par][s],
                      &s_alpha[par][16 * s], &s_flag[par][2 * s]);
      };
      __syncthreads();
      if (n_pairs > 0 && active) scores(0);
      __syncthreads();
#pragma unroll 1
      for (int pi = 0; pi < n_iter * kRing; ++pi) {
        // past the last pair the staged tiles lie beyond the context and
        // every score is masked: the softmax state stays unchanged
        if (active) scores(pi + 1);
        __syncthreads();
      }
      if (active) {
        const float lrow = quad_sum(l_run);
        if (lane < 16) {
          p.ws_ml[(base + 16 * s + lane) * 2 + 0] = m_run;
          p.ws_ml[(base + 16 * s + lane) * 2 + 1] = lrow;
        }
      }
      return;
    } else {
    // conversion route: 8-row owners 2w and 2w + 1, query hi / lo in
    // columns c and c + 8
    bf16x8_t qv[2][4][4];
    if (active) {
      load_qconv5(p, bh, NO, 2 * s, lane, qv[0]);
      load_qconv5(p, bh, NO, 2 * s + 1, lane, qv[1]);
    }
    int row_lim[2];
    float m_run[2], l_run[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int row = 8 * (2 * s + o) + (col & 7);
      row_lim[o] = (active && row < p.rows) ? min(tok_limit - 1, L - p.n_q + row / p.group) : -1;
      m_run[o] = -INFINITY;
      l_run[o] = 0.0f;
    }
    auto scores = [&](int pi) {
      const int par = pi & 1;
      const int kbuf = pi % 3;
      const int tile = t_begin + 2 * pi;
      f32x4_t S[2][2];
      // each chunk's K codes converted once, for both owners
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4_t kc = s_k[kbuf][tt][c][lane];
          const uint32_t kw[4] = {kc[0], kc[1], kc[2], kc[3]};
          uint32_t kb[16];
          dequant_group<KVQ_FMT_FP4_E2M1>(kw, scale_operand(s_ks[kbuf][tt][c][lane]), kb);
          a0 = qk_chunk5_conv(a0, kb, qv[0][c]);
          a1 = qk_chunk5_conv(a1, kb, qv[1][c]);
        }
        S[0][tt] = a0;
        S[1][tt] = a1;
      }
#pragma unroll
      for (int o = 0; o < 2; ++o)
        owner_softmax(S[o], tile, row_lim[o], lane, o, m_run[o], l_run[o], s_p[par][s], &s_alpha[par][8 * (2 * s + o)],
                      &s_flag[par][2 * s + o]);
    };
    // barrier schedule of the staging waves: pairs 0 and 1 staged, then
    // one barrier per pair
    __syncthreads();
    if (n_pairs > 0 && active) scores(0);
    __syncthreads();
#pragma unroll 1
    for (int pi = 0; pi < n_iter * kRing; ++pi) {
      if (active) scores(pi + 1);
      __syncthreads();
    }
    if (active) {
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const float lrow = quad_sum(l_run[o]);
        if (lane < 8) {
          p.ws_ml[(base + 8 * (2 * s + o) + lane) * 2 + 0] = m_run[o];
          p.ws_ml[(base + 8 * (2 * s + o) + lane) * 2 + 1] = lrow;
        }
      }
    }
    return;
    }
  }

  // ---------------- output wave: channels 128v .. 128v + 127, staging of chunk v
  const int v = w - 4;
  // stage pair pi: codes and scale bytes as they came (lane = token col,
  // group quad of chunk v); V's scale byte is zero past the context, so
  // whatever codes the cache holds there convert to zero
  auto stage = [&](int pi, int t, const Chunk5& c) {
    const int tile = t_begin + 2 * pi + t;
    const int buf = pi % 3;
    s_k[buf][t][v][lane] = u32x4_t{c.k[0], c.k[1], c.k[2], c.k[3]};
    s_ks[buf][t][v][lane] = c.ksc;
    if constexpr (!SHARED) s_vc[buf][t][v][lane] = u32x4_t{c.v[0], c.v[1], c.v[2], c.v[3]};
    const bool dead = tile * 16 + col >= tok_limit;
    s_vsb[buf][t][v][16 * (col >> 2) + 4 * quad + (col & 3)] = (uint8_t)(dead ? 0u : (SHARED ? c.ksc : c.vsc));
  };
  auto fetch = [&](int pi, int t, Chunk5& c) {
    load_chunk5<SHARED, SEL, FLAT>(p, bt_row, sel_row, L, kvh, min(t_begin + 2 * pi + t, t_end - 1), v, lane, c);
  };
  Chunk5 ring[kRing][2];
  if (n_pairs > 0) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      fetch(u, 0, ring[u][0]);
      fetch(u, 1, ring[u][1]);
    }
  }
  f32x4_t O[RG][8];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int n = 0; n < 8; ++n) O[g][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (n_pairs > 0) {
    stage(0, 0, ring[0][0]);
    stage(0, 1, ring[0][1]);
    fetch(kRing, 0, ring[0][0]);
    fetch(kRing, 1, ring[0][1]);
  }
  __syncthreads();
  if (n_pairs > 0) {
    stage(1, 0, ring[1 % kRing][0]);
    stage(1, 1, ring[1 % kRing][1]);
    fetch(1 + kRing, 0, ring[1 % kRing][0]);
    fetch(1 + kRing, 1, ring[1 % kRing][1]);
  }
  __syncthreads();

  // PV B operands from the staged FP4 codes: one transposing byte read per
  // 32-channel group gives lane (quad, col) byte col of the eight token
  // records 4 quad .. 4 quad + 3 of tile 0 and of tile 1 (the k order of the
  // P operands), i.e. channels 2 col and 2 col + 1 of eight tokens; row j of
  // the read (lanes 2j, 2j + 1 of the quad: the record's two halves) is
  // token 4 quad + j % 4 of tile j / 4.  Each byte is converted with its
  // token's scale; even and odd channels make two n-tiles.
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v2i_t lds_v2i;
  const int vlane = (col >> 3) * (int)sizeof(s_k[0][0]) + (4 * quad + ((col >> 1) & 3)) * 16 + 8 * (col & 1);
  const uint32_t k23 = 23;
#pragma unroll 1
  for (int it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int pi = it * kRing + u;
      const int par = pi & 1;
      bf16x8_t A[RG][2];
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        if (s_flag[par][2 * g] | s_flag[par][2 * g + 1]) {
          float ar[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ar[i] = s_alpha[par][16 * g + 4 * quad + i];
#pragma unroll
          for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[g][n][i] *= ar[i];
        }
        A[g][0] = __builtin_bit_cast(bf16x8_t, s_p[par][g][0][lane]);
        A[g][1] = __builtin_bit_cast(bf16x8_t, s_p[par][g][1][lane]);
      }
      const int kbuf = pi % 3;
      // (buffer offsets uniform, so that one lane address serves every read)
      const int cbuf = __builtin_amdgcn_readfirstlane(kbuf * (int)sizeof(s_k[0]) + v * (int)sizeof(s_k[0][0][0]));
      __attribute__((address_space(3))) uint8_t* const vrow =
          (__attribute__((address_space(3))) uint8_t*)(SHARED ? &s_k[0][0][0][0] : &s_vc[0][0][0][0]) + vlane + cbuf;
      v2i_t raw[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        raw[gg] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vrow + 256 * gg));
      // scale bytes of tokens 4 quad .. 4 quad + 3, groups 0..3, per tile
      const u32x4_t sb0 = *reinterpret_cast<const u32x4_t*>(&s_vsb[kbuf][0][v][16 * quad]);
      const u32x4_t sb1 = *reinterpret_cast<const u32x4_t*>(&s_vsb[kbuf][1][v][16 * quad]);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const uint32_t d[8] = {cvt_token<0>(raw[gg][0], sb0[gg], k23), cvt_token<1>(raw[gg][0], sb0[gg], k23),
                               cvt_token<2>(raw[gg][0], sb0[gg], k23), cvt_token<3>(raw[gg][0], sb0[gg], k23),
                               cvt_token<0>(raw[gg][1], sb1[gg], k23), cvt_token<1>(raw[gg][1], sb1[gg], k23),
                               cvt_token<2>(raw[gg][1], sb1[gg], k23), cvt_token<3>(raw[gg][1], sb1[gg], k23)};
        uint32_t be[4], bo[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          be[m] = __builtin_amdgcn_perm(d[2 * m + 1], d[2 * m], 0x05040100u);
          bo[m] = __builtin_amdgcn_perm(d[2 * m + 1], d[2 * m], 0x07060302u);
        }
        const bf16x8_t Be = __builtin_bit_cast(bf16x8_t, u32x4_t{be[0], be[1], be[2], be[3]});
        const bf16x8_t Bo = __builtin_bit_cast(bf16x8_t, u32x4_t{bo[0], bo[1], bo[2], bo[3]});
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          O[g][2 * gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][0], Be, O[g][2 * gg], 0, 0, 0);
          O[g][2 * gg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][1], Be, O[g][2 * gg], 0, 0, 0);
          O[g][2 * gg + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][0], Bo, O[g][2 * gg + 1], 0, 0, 0);
          O[g][2 * gg + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][1], Bo, O[g][2 * gg + 1], 0, 0, 0);
        }
      }
      {
        const int su = (u + 2) % kRing;
        stage(pi + 2, 0, ring[su][0]);
        stage(pi + 2, 1, ring[su][1]);
        fetch(pi + 2 + kRing, 0, ring[su][0]);
        fetch(pi + 2 + kRing, 1, ring[su][1]);
      }
      __syncthreads();
    }
  }
  // n-tile n holds channels 128 v + 32 (n / 2) + 2 col + n % 2
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.ws_o[(base + 16 * g + 4 * quad + i) * kD5 + 128 * v + 32 * (n >> 1) + 2 * col + (n & 1)] = O[g][n][i];
}

constexpr int kMinTilesPerSplit5 = 8;
constexpr int kDefaultSlots5 = 256;  // MI355X: 256 CUs x 1 block
constexpr int kMaxDevices5 = 64;

template <int RG, bool SHARED, bool CONV>
int resident_blocks5(int dev) {
  static std::atomic<int> cache[kMaxDevices5];
  if (dev < kMaxDevices5) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0, blocks = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) {
    if constexpr (RG >= kRoleSplitRG5)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode512r_kernel<RG, SHARED, false, CONV>, 512, 0);
    else
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode512_kernel<RG, SHARED, false, CONV>, 512, 0);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int v = cus * blocks;
  if (dev < kMaxDevices5) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <bool CONV>
int resident_slots5_c(int dev, int rg, bool shared) {
  switch (rg) {
    case 1: return shared ? resident_blocks5<1, true, CONV>(dev) : resident_blocks5<1, false, CONV>(dev);
    case 2: return shared ? resident_blocks5<2, true, CONV>(dev) : resident_blocks5<2, false, CONV>(dev);
    case 3: return shared ? resident_blocks5<3, true, CONV>(dev) : resident_blocks5<3, false, CONV>(dev);
    case 4: return shared ? resident_blocks5<4, true, CONV>(dev) : resident_blocks5<4, false, CONV>(dev);
    default: return 0;
  }
}

int resident_slots5(int rg, bool shared, bool conv) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return conv ? resident_slots5_c<true>(dev, rg, shared) : resident_slots5_c<false>(dev, rg, shared);
}

template <int RG, bool SHARED, bool SEL, bool CONV = false>
hipError_t launch5(const DecodeParams& p, int batch, hipStream_t stream) {
  const unsigned qblocks = (unsigned)((size_t)batch * p.hkv * 16 * RG / 4);
  hipLaunchKernelGGL((qprep512_kernel<RG, CONV, (RG >= kRoleSplitRG5) && !CONV>), dim3(qblocks), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)p.splits, (unsigned)p.hkv, (unsigned)batch);
  // the gathered selection (SEL) addresses every lane's page on its own
  const bool flat = p.flat && !SEL;
  if constexpr (RG >= kRoleSplitRG5) {
    if (flat)
      hipLaunchKernelGGL((decode512r_kernel<RG, SHARED, SEL, CONV, true>), grid, dim3(64 * kW5), 0, stream, p);
    else
      hipLaunchKernelGGL((decode512r_kernel<RG, SHARED, SEL, CONV, false>), grid, dim3(64 * kW5), 0, stream, p);
  } else {
    if (flat)
      hipLaunchKernelGGL((decode512_kernel<RG, SHARED, SEL, CONV, true>), grid, dim3(64 * kW5), 0, stream, p);
    else
      hipLaunchKernelGGL((decode512_kernel<RG, SHARED, SEL, CONV, false>), grid, dim3(64 * kW5), 0, stream, p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<16 * RG, 8>), dim3(qblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <bool SHARED, bool SEL, bool CONV = false>
hipError_t launch5_rg(const DecodeParams& p, int rg, int batch, hipStream_t stream) {
  switch (rg) {
    case 1: return launch5<1, SHARED, SEL, CONV>(p, batch, stream);
    case 2: return launch5<2, SHARED, SEL, CONV>(p, batch, stream);
    case 3: return launch5<3, SHARED, SEL, CONV>(p, batch, stream);
    case 4: return launch5<4, SHARED, SEL, CONV>(p, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int plan_decode512(const CacheGeom& c, int batch, int hq, int n_q, int max_context_len, uint32_t flags,
                   DecodePlan* plan) {
  if (c.d != kD5) return KVQ_ERR_UNSUPPORTED;
  if (c.fmt != KVQ_FMT_FP4_E2M1) return KVQ_ERR_UNSUPPORTED;
  // 64-bit before any narrowing: an int product of group and n_q could wrap
  // to a small row count
  const long long rows_ll = (long long)(hq / c.hkv) * n_q;
  if (rows_ll < 1 || rows_ll > 16LL * kMaxRG5) return KVQ_ERR_UNSUPPORTED;
  const int rows = (int)rows_ll;
  const int rg = (rows + 15) / 16;
  const int n_tiles = (int)(((long long)max_context_len + 15) / 16);
  int splits = (int)((flags & KVQ_SPLITS_MASK) >> KVQ_SPLITS_SHIFT);
  if (splits <= 0) {
    // one round of blocks over the device (one block per compute unit)
    int slots = resident_slots5(rg, c.kv_shared != 0, (flags & KVQ_QK_CONVERT) != 0);
    if (slots <= 0) slots = kDefaultSlots5;
    const long long units = (long long)batch * c.hkv;
    long long want = units >= slots ? 1 : slots / units;
    const long long by_len = n_tiles / kMinTilesPerSplit5;
    if (want > by_len) want = by_len;
    splits = (int)(want < 1 ? 1 : want);
  }
  if (splits > kMaxSplits) splits = kMaxSplits;
  int per = (n_tiles + splits - 1) / splits;
  per = (per + 1) & ~1;
  if (per < 2) per = 2;
  splits = (n_tiles + per - 1) / per;
  if (splits < 1) splits = 1;
  plan->rows = rows;
  plan->row_tiles = rg;
  plan->splits = splits;
  plan->tiles_per_split = per;
  plan->qk_convert = (flags & KVQ_QK_CONVERT) ? 1 : 0;
  // query operands: FP6 terms (4 chunks x kM5 x 8 dwords per lane) or, on
  // the conversion route, bf16 hi / lo (4 chunks x 4 k-steps x 4 dwords):
  // the same size
  plan->qops_bytes = (size_t)batch * c.hkv * (2 * rg) * 4 * kM5 * 64 * 8 * sizeof(uint32_t);
  plan->workspace = plan->qops_bytes + (size_t)batch * c.hkv * splits * (16 * rg) * (kD5 + 2) * sizeof(float);
  return KVQ_OK;
}

hipError_t launch_decode512(const DecodeArgs& a, hipStream_t stream) {
  DecodeParams p{};
  p.kc = a.c.kc;
  p.ks = a.c.ks;
  p.vc = a.c.kv_shared ? a.c.kc : a.c.vc;
  p.vs = a.c.kv_shared ? a.c.ks : a.c.vs;
  p.c_head = a.c.c_head;
  p.c_page = a.c.c_page;
  p.s_head = a.c.s_head;
  p.s_page = a.c.s_page;
  p.c_total = (int64_t)a.c.num_pages * a.c.c_page;
  p.s_total = (int64_t)a.c.num_pages * a.c.s_page;
  p.flat = flat_ok(p.c_total, p.s_total);
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
  p.norm = fwht_norm(kD5);
  p.rotate_q = a.rotate_q;
  p.rotate_out = a.rotate_out;
  p.splits = a.plan.splits;
  p.tiles_per_split = a.plan.tiles_per_split;
  p.out = a.out;
  const size_t n_o = (size_t)a.batch * a.c.hkv * a.plan.splits * (16 * a.plan.row_tiles) * kD5;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.workspace);
  p.qops = reinterpret_cast<uint32_t*>(ws);
  p.ws_o = reinterpret_cast<float*>(ws + a.plan.qops_bytes);
  p.ws_ml = p.ws_o + n_o;
  p.sel = a.sel;
  p.sel_stride = a.sel_stride;
  if (a.sel) {
    if (a.c.kv_shared) return launch5_rg<true, true>(p, a.plan.row_tiles, a.batch, stream);
    return launch5_rg<false, true>(p, a.plan.row_tiles, a.batch, stream);
  }
  if (a.plan.qk_convert) {
    if (a.c.kv_shared) return launch5_rg<true, false, true>(p, a.plan.row_tiles, a.batch, stream);
    return launch5_rg<false, false, true>(p, a.plan.row_tiles, a.batch, stream);
  }
  if (a.c.kv_shared) return launch5_rg<true, false>(p, a.plan.row_tiles, a.batch, stream);
  return launch5_rg<false, false>(p, a.plan.row_tiles, a.batch, stream);
}

}  // namespace kvq

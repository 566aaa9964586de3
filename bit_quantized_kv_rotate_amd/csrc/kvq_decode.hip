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
// Design (gfx950, wave64).  Three kernels per call:
//  * qprep_kernel, one wave per query row: load, rotate (lane-shuffle
//    butterfly), pre-scale by sm_scale * log2 e, and store each page-scan
//    lane's score operands in the workspace.  FP4 cache: the query is split
//    into kQTerms FP6 (E2M3) terms with their own per-32 UE8M0 scales, each
//    term carrying the previous residual; FP4 x FP6 products are exact in
//    the scaled MFMA, and four terms leave a residual of about 2^-16 of the
//    block maximum.  FP8 cache: bf16 hi + lo parts.
//  * decode_kernel, one wave per (sequence, KV head, context split): the
//    page scan streams 16-token tiles.  Lane l loads the code bytes of token
//    l%16, channel group l/16, plus that group's scale byte.  For the FP4
//    cache, QK^T runs on v_mfma_scale_f32_16x16x128_f8f6f4 with the K codes
//    and their UE8M0 bytes as the A operand and A scale exactly as loaded:
//    the FP4 operand layout of that instruction is one (token, 32-channel
//    group) per lane.  Two query terms per MFMA sit in columns c and c + 8;
//    one DPP row rotate adds the halves.  The FP8 comparator converts K to
//    bf16 (exact) for bf16 MFMAs against the hi/lo query.  Scores come out
//    transposed (S^T: tokens x query rows), which is directly the A operand
//    layout of the PV product.
//  * V codes are converted with their scale (gfx950 scaled converts, two
//    values per instruction) into a wave-private bf16 LDS tile and read back
//    transposed with ds_read_b64_tr_b16 as the B operand of PV; P is split
//    into bf16 hi + lo (8 rows each in the 16 MFMA rows).  fp32 accumulation.
//  * Online softmax in base 2 with lane-swap reductions; the O rescale runs
//    only when a row's maximum passes its lagging reference (kLazyLog2).
//  * Codes are prefetched through a ring of kRing tile pairs held in
//    registers; refills are unconditional (clamped to the last tile) so the
//    memory wait counts stay exact.
//  * merge_kernel, one wave per query row: partial (m, l, O) of the context
//    splits are combined, normalised and rotated back.  The planner picks
//    the split count that fills the device's resident wave slots once.
#include <atomic>
#include <type_traits>

#include "kvq_append_dev.h"
#include "kvq_decode_common.h"

namespace kvq {
namespace {

constexpr int kD = 128;              // head_dim handled by this kernel
constexpr int kQTerms = 4;           // FP6 (E2M3) terms of the pre-scaled query (FP4 cache)
constexpr int kQMfma = kQTerms / 2;  // scaled MFMAs per tile and row tile
constexpr int kVRow = 2 * kD + 32;   // LDS bytes per token row of V (bf16, padded)
// tile pairs held in registers per wave: one at 8 and 16 rows, with two
// waves per SIMD (on b32_l32k a second pair in flight per wave made the
// scan 2% slower and a third 4%: more outstanding random blocks cost HBM
// row conflicts); two at 24 rows (FP8 cache only), where one wave per SIMD
// fits either way and the deeper ring wins
template <int NT>
struct Ring {
  static constexpr int kN = NT == 3 ? 2 : 1;
};

// bf16 terms of the query on the conversion score route.  The FP8 cache is
// not rotated, so outlier channels of q and K put large products into the
// scores (log2 units beyond 250 on the outlier test inputs), where two bf16
// terms (residual 2^-18 of each channel) move softmax weights enough to
// breach 2e-3 on outputs near 50; a third term leaves 2^-27.  The FP4
// conversion route works on the rotated cache and keeps two.
template <int FMT>
struct Bf16QTerms {
  static constexpr int kN = FMT == KVQ_FMT_FP8_E4M3 ? 3 : 2;
};

// Workspace image of the query operands: per (sequence, KV head, row tile)
// kSlots operands of kDwords per lane (FP6 terms: 6 packed dwords + scale +
// pad; bf16 terms: one bf16x8 = 4 dwords per k-step of 32 channels, four
// k-steps per set of 16 MFMA columns: hi in columns 0..7 and lo in 8..15,
// then, with three terms, a second set with the third term in columns 0..7
// and zeros in 8..15).
template <int FMT>
struct QOpsLayout {
  static constexpr int kSlots = Fmt<FMT>::kNativeQK ? kQMfma : (Bf16QTerms<FMT>::kN == 3 ? 8 : 4);
  static constexpr int kDwords = Fmt<FMT>::kNativeQK ? 8 : 4;
};

// Query operands of the score product.
//  Native FP4 scores: kQTerms FP6 terms for the scaled MFMA (6 packed dwords
//  + scale).  FP8 cache, and FP4 through the conversion route: bf16 terms
//  for the bf16 MFMA.
template <int FMT, int NT>
struct QOps {
  bf16x8_t b[NT][QOpsLayout<FMT>::kSlots];
};
template <int NT>
struct QOps<KVQ_FMT_FP4_E2M1, NT> {
  i32x8_t b[NT][kQMfma];
  int sc[NT][kQMfma];
};

template <int FMT>
struct RawTile {
  uint32_t k[Fmt<FMT>::kWords];
  uint32_t v[Fmt<FMT>::kWords];
  uint32_t ksc, vsc;
};

// Per-lane byte offsets inside one (page, KV head) block, fixed for the
// whole scan: lane l reads token l%16 (of a 16-token tile) in group l/16.
// Blocked addressing builds four buffer resources per tile, bounded to the
// (page, head) block; flat addressing (cache arrays below 4 GiB) builds
// them once per wave over the whole array from this head on, and a tile
// only adds its page offset as the scalar offset, a quarter of the scalar
// instructions per tile (b32_l32k: cold-start steps 0.215-0.225 -> 0.198-
// 0.202 ms).
struct LaneOffsets {
  uint32_t code;   // into the code block
  uint32_t scale;  // into the scale block
};
struct FlatOffsets {
  uint32_t code;
  uint32_t scale;
  __amdgpu_buffer_rsrc_t rk, rv, rks, rvs;
};

template <int FMT>
__device__ __forceinline__ LaneOffsets lane_offsets(const DecodeParams& p, int lane) {
  constexpr int kBytes = Fmt<FMT>::kWords * 4;
  const uint32_t idx = (uint32_t)((lane >> 4) * p.P + (lane & 15));
  return LaneOffsets{idx * kBytes, idx};
}

template <int FMT>
__device__ __forceinline__ FlatOffsets flat_offsets(const DecodeParams& p, int lane, int kvh) {
  const LaneOffsets l = lane_offsets<FMT>(p, lane);
  const int64_t ch = (int64_t)kvh * p.c_head, sh = (int64_t)kvh * p.s_head;
  return FlatOffsets{l.code, l.scale, block_rsrc(p.kc, ch, p.c_total - ch), block_rsrc(p.vc, ch, p.c_total - ch),
                     block_rsrc(p.ks, sh, p.s_total - sh), block_rsrc(p.vs, sh, p.s_total - sh)};
}

// Loads of one 16-token tile (all addressing scalar except the lane offset).
template <int FMT>
__device__ __forceinline__ void load_tile(const DecodeParams& p, const int32_t* bt_row, int kvh,
                                          int tile, const FlatOffsets& lo, RawTile<FMT>& t) {
  constexpr int kBytes = Fmt<FMT>::kWords * 4;
  const int tok = tile * 16;
  const uint32_t page = (uint32_t)__builtin_amdgcn_readfirstlane(bt_row[tok >> p.p_shift]);
  const uint32_t in_page = (uint32_t)(tok & (p.P - 1));
  const int coff = (int)(page * (uint32_t)p.c_page + in_page * kBytes);
  const int soff = (int)(page * (uint32_t)p.s_page + in_page);
#pragma unroll
  for (int i = 0; i < kBytes / 16; ++i) {
    const u32x4_t a = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lo.rk, (int)lo.code + 16 * i, coff, 2));
    const u32x4_t c = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lo.rv, (int)lo.code + 16 * i, coff, 2));
#pragma unroll
    for (int w = 0; w < 4; ++w) { t.k[4 * i + w] = a[w]; t.v[4 * i + w] = c[w]; }
  }
  t.ksc = __builtin_amdgcn_raw_buffer_load_b8(lo.rks, (int)lo.scale, soff, 0);
  t.vsc = __builtin_amdgcn_raw_buffer_load_b8(lo.rvs, (int)lo.scale, soff, 0);
}

template <int FMT>
__device__ __forceinline__ void load_tile(const DecodeParams& p, const int32_t* bt_row, int kvh,
                                          int tile, const LaneOffsets& lo, RawTile<FMT>& t) {
  constexpr int kBytes = Fmt<FMT>::kWords * 4;
  const int tok = tile * 16;
  const int page = __builtin_amdgcn_readfirstlane(bt_row[tok >> p.p_shift]);
  const int in_page = tok & (p.P - 1);
  const int64_t cb = (int64_t)page * p.c_page + (int64_t)kvh * p.c_head;
  const int64_t sb = (int64_t)page * p.s_page + (int64_t)kvh * p.s_head;
  const __amdgpu_buffer_rsrc_t rk = block_rsrc(p.kc, cb, p.c_head);
  const __amdgpu_buffer_rsrc_t rv = block_rsrc(p.vc, cb, p.c_head);
  const __amdgpu_buffer_rsrc_t rks = block_rsrc(p.ks, sb, p.s_head);
  const __amdgpu_buffer_rsrc_t rvs = block_rsrc(p.vs, sb, p.s_head);
  const int coff = in_page * kBytes;
  // slc (bit 1 of aux): streaming, the codes are read once per step
#pragma unroll
  for (int i = 0; i < kBytes / 16; ++i) {
    const u32x4_t a = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)lo.code + 16 * i, coff, 2));
    const u32x4_t c = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)lo.code + 16 * i, coff, 2));
#pragma unroll
    for (int w = 0; w < 4; ++w) { t.k[4 * i + w] = a[w]; t.v[4 * i + w] = c[w]; }
  }
  t.ksc = __builtin_amdgcn_raw_buffer_load_b8(rks, (int)lo.scale, in_page, 0);
  t.vsc = __builtin_amdgcn_raw_buffer_load_b8(rvs, (int)lo.scale, in_page, 0);
}

// Per-wave softmax / accumulator state.
template <int NT>
struct WaveState {
  f32x4_t O[NT][8];
  float m_run[NT];
  float l_run[NT];
};

template <int FMT, class LO>
__device__ __forceinline__ void issue_pair(const DecodeParams& p, const int32_t* bt_row, int kvh,
                                           int tile, int t_end, const LO& lo,
                                           RawTile<FMT> (&r)[2]) {
  load_tile<FMT>(p, bt_row, kvh, min(tile, t_end - 1), lo, r[0]);
  load_tile<FMT>(p, bt_row, kvh, min(tile + 1, t_end - 1), lo, r[1]);
}

// One pair of 16-token tiles: scores, V staging, softmax update, PV.
// Once the codes of `r` are consumed, the loads of tile pair `refill` are
// issued into the same registers (clamped to the split's last tile).
// Boundary pairs (the split's last tokens, padding pairs, MTP verify
// tokens) mask scores and clear values of tokens past the end; interior
// pairs skip all of that.
template <int FMT, int NT, bool Boundary, class LO>
__device__ __forceinline__ void compute_pair(const DecodeParams& p, const int32_t* bt_row, int kvh,
                                             int tile, int t_end, int refill, int tok_limit,
                                             int interior_limit, const int (&row_last)[NT],
                                             const QOps<FMT, NT>& q, RawTile<FMT> (&r)[2],
                                             uint8_t (*s_v)[16][kVRow], int lane,
                                             const LO& lo, WaveState<NT>& st) {
  const int col = lane & 15;
  const int quad = lane >> 4;
  const bool hi_col = col < 8;

  // ---- scores S^T = K q^T for row tile t.  With 8 rows they are all
  // computed up front; with 16 or 24 rows one row tile at a time, inside the
  // softmax loop, to keep register pressure down.
  constexpr bool kLate = NT >= 2;
  auto scores_t = [&](int s, int t) -> f32x4_t {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Fmt<FMT>::kNativeQK) {
      // FP4 codes and UE8M0 scales straight into the scaled MFMA (A operand)
      const i32x8_t A = {(int)r[s].k[0], (int)r[s].k[1], (int)r[s].k[2], (int)r[s].k[3], 0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < kQMfma; ++m)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, q.b[t][m], acc, 4, 2, 0, (int)r[s].ksc, 0,
                                                               q.sc[t][m]);
    } else {
      // E4M3 (or, on the conversion route, E2M1) codes dequantised with their
      // scale to bf16 (exact) as the A operand of bf16 MFMAs
      uint32_t kb[16];
      dequant_group<FMT>(r[s].k, scale_operand(r[s].ksc), kb);
#pragma unroll
      for (int ks = 0; ks < QOpsLayout<FMT>::kSlots; ++ks) {
        const u32x4_t a = {kb[4 * (ks & 3)], kb[4 * (ks & 3) + 1], kb[4 * (ks & 3) + 2], kb[4 * (ks & 3) + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), q.b[t][ks], acc, 0, 0, 0);
      }
    }
    return acc;
  };
  f32x4_t S[2][kLate ? 1 : NT];
  if constexpr (!kLate) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) S[s][t] = scores_t(s, t);
  }

  // ---- V tiles -> LDS as bf16 token rows.  Past the end of the context the
  // cache may hold anything: clear those codes and use the smallest scale so
  // the (zero-weighted) values are exactly zero.
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint32_t vw[Fmt<FMT>::kWords];
    uint32_t vsc = r[s].vsc;
#pragma unroll
    for (int i = 0; i < Fmt<FMT>::kWords; ++i) vw[i] = r[s].v[i];
    if constexpr (Boundary) {
      const bool dead = (tile + s) * 16 + col >= tok_limit;
#pragma unroll
      for (int i = 0; i < Fmt<FMT>::kWords; ++i) vw[i] = dead ? 0u : vw[i];
      vsc = dead ? 0u : vsc;
    }
    uint32_t vb[16];
    dequant_group<FMT>(vw, scale_operand(vsc), vb);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&s_v[s][col][64 * quad]);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{vb[4 * i], vb[4 * i + 1], vb[4 * i + 2], vb[4 * i + 3]};
  }

  // the raw codes are consumed: start the next loads into the same registers
  if constexpr (!kLate) issue_pair<FMT>(p, bt_row, kvh, refill, t_end, lo, r);

  // ---- softmax update and P (bf16 hi/lo) per row tile
  bf16x8_t A[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4_t St[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) St[s] = kLate ? scores_t(s, t) : S[s][kLate ? 0 : t];
    if (kLate && t == NT - 1) issue_pair<FMT>(p, bt_row, kvh, refill, t_end, lo, r);
    // Row col & 7's scores: the two query-term halves (columns c and c + 8)
    // summed.  Lanes c < 8 then keep tile 0's four tokens 4 quad + i, lanes
    // c >= 8 tile 1's, so each score's softmax runs once.
    const int ts = hi_col ? 0 : 1;  // this lane's tile of the pair
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = St[0][i] + dpp_ror8(St[0][i]);
      const float x1 = St[1][i] + dpp_ror8(St[1][i]);
      sc[i] = hi_col ? x0 : x1;
    }
    if constexpr (Boundary) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = (tile + ts) * 16 + 4 * quad + i;
        const bool ok = (tok < tok_limit) && (tok <= row_last[t]);
        sc[i] = ok ? sc[i] : -INFINITY;
      }
    }
    float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mloc = fmaxf(mloc, dpp_ror8(mloc));
    mloc = quad_max(mloc);
    // lazy reference maximum: a row's reference moves only when its running
    // maximum passes it by more than kLazyLog2, so most tiles skip the
    // rescale; the weights stay below 2^kLazyLog2
    const float m_old = st.m_run[t];
    const float m_tgt = fmaxf(m_old, mloc);
    const bool grow = m_tgt > m_old + kLazyLog2;
    const float m_new = grow ? m_tgt : m_old;
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    st.m_run[t] = m_new;
    float psum = 0.0f;
    uint32_t h[2], l[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(sc[2 * e] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(sc[2 * e + 1] - m_use);
      psum += p0 + p1;
      // hi: the upper halves of p0, p1 (bf16 by truncation, one byte permute);
      // lo: the exact remainders rounded to bf16.  |p - hi - lo| <= 2^-16 |p|.
      const uint32_t u0 = as_u32(p0), u1 = as_u32(p1);
      h[e] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
      l[e] = pack_bf16x2(p0 - as_f32(u0 & 0xFFFF0000u), p1 - as_f32(u1 & 0xFFFF0000u));
    }
    // PV A operand: lane c < 8 holds hi of row c for tile 0 then tile 1,
    // lane c >= 8 lo of row c - 8; each lane passes its partner (lane c ^ 8)
    // the half it lacks
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t give = hi_col ? l[e] : h[e];
      const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0x128, 0xF, 0xF, false);
      pw[e] = hi_col ? h[e] : got;
      pw[2 + e] = hi_col ? got : l[e];
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
      // a row reference moved in some lane: rescale (rare once the scan settles)
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
    A[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]});
  }

  // ---- PV: B operands read transposed from the LDS V tiles, one n-tile
  // ahead of the MFMA that consumes it
  {
    const int rr = col >> 2;
    const int c4 = (col & 3) * 4;
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    auto read_b = [&](int n) {
      lds_bf16x4* a0 = (lds_bf16x4*)((__attribute__((address_space(3))) uint8_t*)&s_v[0][4 * quad + rr][2 * (16 * n + c4)]);
      lds_bf16x4* a1 = (lds_bf16x4*)((__attribute__((address_space(3))) uint8_t*)&s_v[1][4 * quad + rr][2 * (16 * n + c4)]);
      const u32x2_t w0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a0));
      const u32x2_t w1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(a1));
      return __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
    };
    bf16x8_t B0 = read_b(0);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const bf16x8_t C0 = (n + 1 < 8) ? read_b(n + 1) : B0;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        st.O[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], B0, st.O[t][n], 0, 0, 0);
      B0 = C0;
    }
  }
}

// Query prologue, once per query row: load the row, rotate it with the fp32
// transform, pre-scale by sm_scale * log2 e, and store the score-MFMA
// operands the page-scan lanes will hold (FP6 terms for the FP4 cache, bf16
// hi/lo for the FP8 cache) in the workspace, for all context splits.
// One wave per row (rows of a KV head padded to 8 * NT with zeros); lane l
// holds channels 2l and 2l + 1, so the butterfly stage of distance h >= 2
// pairs lane l with lane l ^ (h / 2); every stage is the fp32 add or
// subtract of the append kernel's transform, in the same order.
template <int FMT, int NT>
__device__ __forceinline__ void qprep_row(const DecodeParams& p, int gr, int lane) {
  constexpr int ROWS = 8 * NT;
  constexpr int kS = QOpsLayout<FMT>::kSlots;
  constexpr int kW = QOpsLayout<FMT>::kDwords;
  const int r = gr % ROWS;
  const int bh = gr / ROWS;
  const int kvh = bh % p.hkv;
  const int b = bh / p.hkv;

  float x0 = 0.0f, x1 = 0.0f;
  if (r < p.rows) {
    const int j = r / p.group;
    const int hh = r - j * p.group;
    const uint16_t* src = p.q + (((size_t)b * p.n_q + j) * p.hq + (size_t)kvh * p.group + hh) * kD + 2 * lane;
    x0 = bf16_to_f32(src[0]);
    x1 = bf16_to_f32(src[1]);
  }
  if (p.rotate_q) {
    float xr[2] = {x0, x1};
    wave_fwht<2>(xr, lane, p.norm);
    x0 = xr[0];
    x1 = xr[1];
  }
  x0 = x0 * p.qscale;
  x1 = x1 * p.qscale;

  const int t = r >> 3;
  const int c7 = r & 7;
  uint32_t* base = p.qops + (size_t)bh * NT * kS * 64 * kW;
  if constexpr (Fmt<FMT>::kNativeQK) {
    // kQTerms FP6 (E2M3) terms per 32-channel block (16 lanes), each with its
    // own UE8M0 scale and carrying the previous residual.  The block's 32
    // six-bit codes form a 192-bit little-endian stream: lane i of the block
    // holds bits 12i .. 12i + 11; lanes 0..5 assemble its dwords, lane 6
    // the scale byte, lane 7 a zero pad.
    const int blk = lane >> 4;
    const int li = lane & 15;
    const int w = min(li, 5);
    const int src_a = 16 * blk + 8 * (w / 3) + 2 * (w % 3);
    const int sh = 8 * (w % 3);
#pragma unroll
    for (int tm = 0; tm < kQTerms; ++tm) {
      float am = fmaxf(fabsf(x0), fabsf(x1));
      am = row16_max(am);
      const int byte = max((int)((as_u32(am) >> 23) & 0xFFu) - 2, 0);
      const int e = byte - 127;
      float v0, v1;
      const uint32_t c0 = e2m3_split(x0, e, v0);
      const uint32_t c1 = e2m3_split(x1, e, v1);
      x0 -= v0;
      x1 -= v1;
      const uint32_t v12 = c0 | (c1 << 6);
      const uint32_t u24 = v12 | ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v12, kDppXor1, 0xF, 0xF, true) << 12);  // valid on even li
      const uint32_t ua = (uint32_t)__shfl((int)u24, src_a, 64);
      const uint32_t ub = (uint32_t)__shfl((int)u24, src_a + 2, 64);
      const uint32_t d = (ua >> sh) | (ub << (24 - sh));
      const int m = tm >> 1;
      const int col = c7 + 8 * (tm & 1);
      uint32_t* dst = base + ((size_t)(t * kS + m) * 64 + 16 * blk + col) * kW;
      if (li < 8) dst[li] = (li < 6) ? d : (li == 6 ? (uint32_t)byte : 0u);
    }
  } else {
    // bf16 terms, each the previous residual (exact in fp32) rounded; the
    // operand lane (col, quad) of k-step s holds channels 32 quad + 8 s .. + 7
    // of row 8t + (col & 7): hi for col < 8, lo for col >= 8, and in the
    // second set (k-steps 4..7, three terms) the third term for col < 8 and
    // zero for col >= 8.
    const uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
    const float r0 = x0 - bf16_to_f32((uint16_t)h0), r1 = x1 - bf16_to_f32((uint16_t)h1);
    const uint32_t l0 = f32_to_bf16_rne(r0), l1 = f32_to_bf16_rne(r1);
    const int quad = lane >> 4;
    const int s4 = (lane & 15) >> 2;
    const int e = lane & 3;
    uint32_t* dst = base + ((size_t)(t * kS + s4) * 64 + 16 * quad + c7) * kW + e;
    dst[0] = h0 | (h1 << 16);
    dst[8 * kW] = l0 | (l1 << 16);
    if constexpr (Bf16QTerms<FMT>::kN == 3) {
      const uint32_t m0 = f32_to_bf16_rne(r0 - bf16_to_f32((uint16_t)l0));
      const uint32_t m1 = f32_to_bf16_rne(r1 - bf16_to_f32((uint16_t)l1));
      dst[4 * 64 * kW] = m0 | (m1 << 16);
      dst[4 * 64 * kW + 8 * kW] = 0u;
    }
  }
}

template <int FMT, int NT>
__global__ __launch_bounds__(256) void qprep_kernel(const DecodeParams p) {
  // grid covers exactly B * hkv * 8 NT rows, four per block
  qprep_row<FMT, NT>(p, blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

// The query prologue and the append of the step's new tokens in one launch
// (head_dim 128, G = 4 groups): blocks below qblocks prepare query rows, the
// others are append waves, axb blocks per (KV head, tensor).  The page scan,
// the next launch on the stream, then finds the new tokens in the cache.
template <int FMT, int NT>
__global__ __launch_bounds__(256) void qprep_append_kernel(const DecodeParams p, const AppendParams ap,
                                                           unsigned qblocks, unsigned axb) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (blockIdx.x < qblocks) {
    qprep_row<FMT, NT>(p, blockIdx.x * 4 + wave, lane);
    return;
  }
  const unsigned b2 = blockIdx.x - qblocks;
  const unsigned ht = b2 / axb;
  append_wave<kD / 32>(ap, (int)(b2 - ht * axb) * 4 + wave, (int)(ht % (unsigned)ap.c.hkv),
                       (int)(ht / (unsigned)ap.c.hkv), lane);
}

// FLAT: flat addressing (cache arrays below 4 GiB), else blocked
template <int FMT, int NT, bool FLAT>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeParams p) {
  constexpr int ROWS = 8 * NT;
  // s_rows: output rows (epilogue); s_v: the V tiles of the page scan
  __shared__ __attribute__((aligned(16))) float s_rows[ROWS * kD];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][16][kVRow];

  const int lane = threadIdx.x;
  // 1-D grid, the splits of one (sequence, KV head) unit consecutive, the
  // split index rotated by the sequence: blocks go to the XCDs round-robin,
  // and with ragged contexts only the low splits of short sequences have
  // work, so without the rotation a split count divisible by 8 would pile
  // that work onto a few XCDs.  The KV head of grid unit u is rotated by
  // u / 32, so that units 32 apart (at 8 splits, the waves an XCD's 32
  // compute units receive in turn) read different heads' slices of the
  // pages: b32_l32k decode 0.1787-0.1791 against 0.1797-0.1803 ms unrotated
  // (three ABBA pairs on one device).
  const int u = blockIdx.x / p.splits;
  const int b = u / p.hkv;
  const int kvh = (u % p.hkv + u / 32) % p.hkv;
  const int split = (blockIdx.x - u * p.splits + b) % p.splits;
  const int L = p.context_lens[b];
  const int n_tiles = (L + 15) >> 4;
  // a shared-prefix suffix scan starts past the prefix (a multiple of 16)
  const int t0 = p.tok_start ? (p.tok_start[b] >> 4) : 0;
  const int t_begin = t0 + split * p.tiles_per_split;
  const int t_end = min(n_tiles, t_begin + p.tiles_per_split);
  const int tok_limit = min(L, t_end * 16);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const int32_t* bt_row = p.block_tables + (size_t)b * p.max_pages;
  const bool has_work = t_end > t_begin;
  if (!has_work && (p.splits > 1 || p.keep_partials)) {
    // an empty split (a short sequence of a ragged batch): (m, l) = (-inf, 0)
    // only; a merge never reads the O of a split with zero weight
    if (lane < ROWS) {
      const size_t base = (((size_t)b * p.hkv + kvh) * p.splits + split) * ROWS;
      p.ws_ml[(base + lane) * 2 + 0] = -INFINITY;
      p.ws_ml[(base + lane) * 2 + 1] = 0.0f;
    }
    return;
  }
  const int n_pairs = has_work ? ((t_end - t_begin + 1) >> 1) : 0;
  constexpr int kRing = Ring<NT>::kN;
  const int n_iter = (n_pairs + kRing - 1) / kRing;

  // ---- start streaming the first tile pairs
  using LO = std::conditional_t<FLAT, FlatOffsets, LaneOffsets>;
  LO lo;
  if constexpr (FLAT) lo = flat_offsets<FMT>(p, lane, kvh);
  else lo = lane_offsets<FMT>(p, lane);
  RawTile<FMT> ring[kRing][2];
  if (has_work) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) issue_pair<FMT>(p, bt_row, kvh, t_begin + 2 * u, t_end, lo, ring[u]);
  }

  // ---- this lane's query operands, prepared once per (sequence, KV head)
  QOps<FMT, NT> q;
  {
    constexpr int kS = QOpsLayout<FMT>::kSlots;
    constexpr int kW = QOpsLayout<FMT>::kDwords;
    const uint32_t* src = p.qops + ((size_t)(b * p.hkv + kvh) * NT * kS * 64 + lane) * kW;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int m = 0; m < kS; ++m) {
        const uint32_t* w = src + (size_t)(t * kS + m) * 64 * kW;
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(w);
        if constexpr (Fmt<FMT>::kNativeQK) {
          const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(w + 4);
          q.b[t][m] = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], 0, 0};
          q.sc[t][m] = (int)a1[2];
        } else {
          q.b[t][m] = __builtin_bit_cast(bf16x8_t, a0);
        }
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
  // multiple of kRing with fully masked pairs so every refill is unconditional.
  // Iterations whose pairs all lie below interior_limit run without masks;
  // the rest (the split's last pairs) run masked.  Two loops rather than a
  // per-pair branch keep the loop-carried registers in place.
  const int n_int_pairs = (interior_limit >= 16 * t_begin + 32) ? (interior_limit - 16 * t_begin - 32) / 32 + 1 : 0;
  const int n_int_iter = min(n_int_pairs, n_pairs) / kRing;
#pragma unroll 1
  for (int it = 0; it < n_int_iter; ++it) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int tile = t_begin + 2 * (it * kRing + u);
      compute_pair<FMT, NT, false>(p, bt_row, kvh, tile, t_end, tile + 2 * kRing, tok_limit,
                                   interior_limit, row_last, q, ring[u], s_v, lane, lo, st);
    }
  }
#pragma unroll 1
  for (int it = n_int_iter; it < n_iter; ++it) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int tile = t_begin + 2 * (it * kRing + u);
      compute_pair<FMT, NT, true>(p, bt_row, kvh, tile, t_end, tile + 2 * kRing, tok_limit,
                                  interior_limit, row_last, q, ring[u], s_v, lane, lo, st);
    }
  }

  // ---- epilogue: full row sums, hi + lo halves of O
  float lrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    lrow[t] = quad_sum(st.l_run[t]);
    lrow[t] += dpp_ror8(lrow[t]);  // lanes c and c + 8 summed different tiles
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st.O[t][n][i] = add_half_swap(st.O[t][n][i]);
    }
  }

  // lanes 0..31 hold row 8t + 4*quad + i, channel 16n + col
  if (p.splits == 1 && !p.keep_partials) {
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

constexpr int kMinTilesPerSplit = 8;     // 128 tokens
constexpr int kMaxTilesPerSplit = 256;   // 4096 tokens
constexpr int kMaxWavesPerCU = 8;        // two page-scan waves per SIMD
// The FP8 comparator moves twice the bytes per tile and is fastest with
// fewer concurrent page streams: six waves per CU measured best both at
// 32K (b32_l32k: 6 splits 0.3838 ms, 7 0.3900, 8 0.4032) and at 8K (b8_l8k:
// 24 splits 0.0383 ms, 32 0.0411), where FP4 is best at eight (b32_l32k 8
// splits 0.1787 ms against 0.1883 at 6; b8_l8k 32 splits 0.0255 against
// 0.0259 at 24).
constexpr int kMaxWavesPerCUFP8 = 6;
// ... and so with longer splits, up to 16 rows (the shapes measured): at
// most 384 tiles each (6K tokens), which lets b32_l32k run its 6 splits.
// At 24 rows the kernel holds one wave per SIMD, the wave cap does not bind,
// and the FP8 plan keeps the 256-tile cap.
constexpr int kMaxTilesPerSplitFP8 = 384;
constexpr int kDefaultWaveSlots = 2048;  // MI355X: 256 CUs x kMaxWavesPerCU
constexpr int kMaxDevices = 64;

template <int FMT, int NT>
hipError_t launch_nt(const DecodeParams& p, int batch, const AppendParams* ap, hipStream_t stream) {
  // 8 * NT rows per (sequence, KV head), four row-waves per block
  const unsigned qblocks = (unsigned)((size_t)batch * p.hkv * 8 * NT / 4);
  if (ap && ap->n_tokens > 0) {
    const unsigned axb = (unsigned)((append_waves(ap->c, ap->n_tokens) + 3) / 4);
    const unsigned ablocks = axb * (unsigned)p.hkv * (ap->c.kv_shared ? 1u : 2u);
    hipLaunchKernelGGL((qprep_append_kernel<FMT, NT>), dim3(qblocks + ablocks), dim3(256), 0, stream, p, *ap,
                       qblocks, axb);
  } else {
    hipLaunchKernelGGL((qprep_kernel<FMT, NT>), dim3(qblocks), dim3(256), 0, stream, p);
  }
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  const dim3 grid((unsigned)((size_t)p.splits * p.hkv * batch));
  // the FP8 comparator keeps blocked addressing: flat read 2.5-3% slower on
  // its 2 KB code tiles (b32_l32k 0.417-0.421 against 0.407-0.409 ms)
  if (p.flat && FMT != KVQ_FMT_FP8_E4M3)
    hipLaunchKernelGGL((decode_kernel<FMT, NT, true>), grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<FMT, NT, false>), grid, dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1 || p.keep_partials) return e;
  // past the first eight splits, the nonzero-weight ones in rounds of 32
  // rather than of eight (b8_l8k's 32 splits: two memory round trips, not four)
  hipLaunchKernelGGL((merge_kernel<8 * NT, 2, 32>), dim3(qblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const DecodeParams& p, int row_tiles, int batch, const AppendParams* ap, hipStream_t stream) {
  switch (row_tiles) {
    case 1: return launch_nt<FMT, 1>(p, batch, ap, stream);
    case 2: return launch_nt<FMT, 2>(p, batch, ap, stream);
    case 3: return launch_nt<FMT, 3>(p, batch, ap, stream);
    default: return hipErrorInvalidValue;
  }
}

// Page-scan waves the current device holds at once: compute units times
// resident 64-thread blocks per unit for this kernel; 0 without a device.
// Cached per (device, format, row tiles).
template <int FMT, int NT>
int resident_waves_nt(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  if (dev < kMaxDevices) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0, blocks = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_kernel<FMT, NT, true>, 64, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  // at most kMaxWavesPerCU page streams per CU: the scan's random 1 KB
  // blocks lose HBM bandwidth to row conflicts as concurrent streams grow
  // (three waves per SIMD were a third slower than two on b32_l32k, with
  // the same bytes in flight per wave)
  const int cap = FMT == KVQ_FMT_FP8_E4M3 ? kMaxWavesPerCUFP8 : kMaxWavesPerCU;
  const int v = cus * (blocks < cap ? blocks : cap);
  if (dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int FMT>
int resident_waves_fmt(int dev, int row_tiles) {
  switch (row_tiles) {
    case 1: return resident_waves_nt<FMT, 1>(dev);
    case 2: return resident_waves_nt<FMT, 2>(dev);
    case 3: return resident_waves_nt<FMT, 3>(dev);
    default: return 0;
  }
}

// kernel format: the cache's, or the FP4 conversion route
int resident_waves(int kfmt, int row_tiles) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (kfmt == KVQ_FMT_FP4_E2M1) return resident_waves_fmt<KVQ_FMT_FP4_E2M1>(dev, row_tiles);
  if (kfmt == kFmtFP4Conv) return resident_waves_fmt<kFmtFP4Conv>(dev, row_tiles);
  return resident_waves_fmt<KVQ_FMT_FP8_E4M3>(dev, row_tiles);
}

}  // namespace

int plan_decode(const CacheGeom& c, int batch, int hq, int n_q, int max_context_len, uint32_t flags,
                DecodePlan* plan) {
  if (c.d == 512) {
    plan->kind = kDecodeLatent;
    return plan_decode512(c, batch, hq, n_q, max_context_len, flags, plan);
  }
  if (c.d != kD) return KVQ_ERR_UNSUPPORTED;
  const int group = hq / c.hkv;
  const long long rows_ll = (long long)group * n_q;
  // FP4 above 16 rows: the many-row kernel (32-row blocks of 2 waves, each
  // wave 16 full rows per MFMA tile) needs about half the VALU work per score
  // of one wave holding 24 rows in 8-row tiles (agentic mix 0.58 -> 0.51 ms)
  if (rows_ll > 24 || (rows_ll > 16 && c.fmt == KVQ_FMT_FP4_E2M1)) {
    plan->kind = kDecodeMany;
    return plan_extend(c, batch, hq, n_q, max_context_len, flags, plan);
  }
  plan->kind = kDecodeFew;
  const bool convert = c.fmt == KVQ_FMT_FP4_E2M1 && (flags & KVQ_QK_CONVERT);
  plan->qk_convert = convert ? 1 : 0;
  const int kfmt = convert ? kFmtFP4Conv : c.fmt;
  const int rows = (int)rows_ll;
  const int row_tiles = (rows + 7) / 8;
  const int n_tiles = (int)(((long long)max_context_len + 15) / 16);
  int splits = (int)((flags & KVQ_SPLITS_MASK) >> KVQ_SPLITS_SHIFT);
  if (splits <= 0) {
    // One round of waves: as many splits as fill the device's resident wave
    // slots once (a second, partial round costs more than the larger
    // partials save), but at least kMinTilesPerSplit tiles per split and at
    // most kMaxTilesPerSplit: with ragged context lengths only the maximum
    // is known here, and long splits of the longest sequences would then
    // set the time of the whole call.
    int slots = resident_waves(kfmt, row_tiles);
    if (slots <= 0) slots = kfmt == KVQ_FMT_FP8_E4M3 ? kDefaultWaveSlots / kMaxWavesPerCU * kMaxWavesPerCUFP8
                                                      : kDefaultWaveSlots;
    const long long units = (long long)batch * c.hkv;
    long long want = units >= slots ? 1 : slots / units;
    const long long by_len = n_tiles / kMinTilesPerSplit;
    if (want > by_len) want = by_len;
    const int max_per = (kfmt == KVQ_FMT_FP8_E4M3 && row_tiles <= 2) ? kMaxTilesPerSplitFP8 : kMaxTilesPerSplit;
    const long long by_cap = (n_tiles + max_per - 1) / max_per;
    if (want < by_cap) want = by_cap;
    // FP8 at 24 rows (one wave per SIMD) on a ragged batch ran split counts
    // that are multiples of 16 far slower than their neighbours (agentic mix:
    // 31 splits 0.720 ms, 32 1.100, 33 0.691, 47 0.671, 48 0.791, 63 0.758,
    // 64 0.959), and a 128K maximum context plans exactly 32
    if (kfmt == KVQ_FMT_FP8_E4M3 && row_tiles == 3 && want > 16 && want % 16 == 0) --want;
    splits = (int)(want < 1 ? 1 : want);
  }
  if (splits > kMaxSplits) splits = kMaxSplits;
  int per = (n_tiles + splits - 1) / splits;
  per = (per + 1) & ~1;  // tiles are processed in pairs
  if (per < 2) per = 2;
  splits = (n_tiles + per - 1) / per;
  if (splits < 1) splits = 1;
  plan->rows = rows;
  plan->row_tiles = row_tiles;
  plan->splits = splits;
  plan->tiles_per_split = per;
  const int per_lane = (kfmt == KVQ_FMT_FP4_E2M1)
                           ? QOpsLayout<KVQ_FMT_FP4_E2M1>::kSlots * QOpsLayout<KVQ_FMT_FP4_E2M1>::kDwords
                       : (kfmt == kFmtFP4Conv)
                           ? QOpsLayout<kFmtFP4Conv>::kSlots * QOpsLayout<kFmtFP4Conv>::kDwords
                           : QOpsLayout<KVQ_FMT_FP8_E4M3>::kSlots * QOpsLayout<KVQ_FMT_FP8_E4M3>::kDwords;
  const size_t qops = (size_t)batch * c.hkv * row_tiles * 64 * sizeof(uint32_t) * per_lane;
  plan->qops_bytes = qops;
  plan->workspace =
      qops + ((splits > 1) ? (size_t)batch * c.hkv * splits * (8 * row_tiles) * (kD + 2) * sizeof(float) : 0);
  return KVQ_OK;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.append && a.append->n_tokens > 0 && a.plan.kind != kDecodeFew) {
    // the other kernel families append in a launch of their own first
    const AppendArgs& ap = *a.append;
    const hipError_t e = launch_append(a.c, ap.kc, ap.ks, ap.vc, ap.vs, ap.k_new, ap.v_new, ap.slots,
                                       ap.n_tokens, stream);
    if (e != hipSuccess) return e;
  }
  if (a.plan.kind == kDecodeLatent) return launch_decode512(a, stream);
  if (a.plan.kind == kDecodeMany) return launch_extend(a, stream);
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
  p.norm = fwht_norm(kD);
  p.rotate_q = a.rotate_q;
  p.rotate_out = a.rotate_out;
  p.splits = a.plan.splits;
  p.tiles_per_split = a.plan.tiles_per_split;
  p.out = a.out;
  p.tok_start = a.tok_start;
  p.keep_partials = a.keep_partials;
  const size_t n_o = (size_t)a.batch * a.c.hkv * a.plan.splits * (8 * a.plan.row_tiles) * kD;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.workspace);
  p.qops = reinterpret_cast<uint32_t*>(ws);
  p.ws_o = reinterpret_cast<float*>(ws + a.plan.qops_bytes);
  p.ws_ml = p.ws_o + n_o;
  AppendParams ap;
  const AppendParams* app = nullptr;
  if (a.append && a.append->n_tokens > 0) {
    ap = make_append_params(a.c, *a.append);
    app = &ap;
  }
  if (a.c.fmt == KVQ_FMT_FP4_E2M1) {
    if (a.plan.qk_convert) return launch_fmt<kFmtFP4Conv>(p, a.plan.row_tiles, a.batch, app, stream);
    return launch_fmt<KVQ_FMT_FP4_E2M1>(p, a.plan.row_tiles, a.batch, app, stream);
  }
  return launch_fmt<KVQ_FMT_FP8_E4M3>(p, a.plan.row_tiles, a.batch, app, stream);
}

}  // namespace kvq

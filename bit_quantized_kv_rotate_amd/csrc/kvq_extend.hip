// Attention of many query rows per KV head over the FP4 cache, head_dim 128:
// prefill / extend chunks (n_q new tokens already appended, position j of the
// chunk sees tokens 0 .. L - n_q + j) and decode shapes with more than 16 rows
// per KV head (wide query groups x MTP positions).
//
// Method: ROCm blog "UltraQuant on AMD Instinct", section "What is
// UltraQuant?" (FP4 codes and power-of-two scales straight into the scaled
// MFMA); the blog's key results include the time to first token, which is
// this step.  With hundreds of rows per KV head the work is MFMA-bound: one
// block of 8 waves per (row block of 128 rows, sequence, KV head, context
// split) stages each 16-token tile once in LDS -- the K codes as the scaled
// MFMA's A operand, V as bf16 rows -- and every wave runs its own 16 rows
// against it:
//  * scores S^T = K q^T with the FP4 K codes and scale bytes as A and four
//    FP6 query terms accumulated in the same 16 x 16 tile (16 full rows);
//  * online softmax per row, P split into bf16 hi + lo;
//  * PV against hi and then lo into one accumulator set (the wave's 16 rows
//    the MFMA rows of both), so each V operand read serves two MFMAs and the
//    accumulators take 32 VGPRs: at 112 VGPRs two wide blocks fit a CU.
// One barrier per tile pair; LDS is double-buffered by pair parity.
#include <atomic>

#include "kvq_decode_common.h"

namespace kvq {
namespace {

constexpr int kDX = 128;
constexpr int kTX = 4;                // FP6 query terms
// Waves per block: 8 (128 rows) for hundreds of rows per KV head, 2 (32
// rows) for a few dozen, where a 128-row block would mostly hold padding.
constexpr int kWideX = 8;
constexpr int kNarrowX = 2;
constexpr int kNarrowMaxRows = 64;    // plain calls up to this many rows use 2-wave blocks
static_assert(16 * kWideX == kExtendRowBlock, "row block of the many-row kernel");
constexpr int kVRowX = 2 * kDX + 32;  // LDS bytes per bf16 token row (padded)
constexpr int kRingX = 2;             // tile pairs in flight per staging wave

// Query prologue, one wave per query row (rows of a KV head padded to a
// multiple of 128): load, rotate, pre-scale, split into kTX FP6 terms per
// 32-channel block and store the B operands [B][hkv][rows_pad / 16]
// [kTX][64 lanes][8 dwords]: lane (k-group j, column n) holds term t of row
// 16 g + n, channels 32 j .. 32 j + 31 (6 packed dwords), its scale, a pad.
template <bool CONV>
__global__ __launch_bounds__(256) void qprep_ext_kernel(const DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const long long gr = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // grid covers B * hkv * rows_pad
  const int r = (int)(gr % p.rows_pad);
  const long long bh = gr / p.rows_pad;
  const int kvh = (int)(bh % p.hkv);
  const int b = (int)(bh / p.hkv);

  float x[2] = {0.0f, 0.0f};
  if (r < p.rows) {
    // row r of a sequence, or of a prefix group: member r / rows_seq, its
    // row r % rows_seq; rows past the group's members stay zero
    int seq = b, rr = r;
    bool live = true;
    if (p.grp_ptr) {
      const int k = r / p.rows_seq;
      const int m0 = p.grp_ptr[b];
      live = k < p.grp_ptr[b + 1] - m0;
      seq = live ? p.grp_seq[m0 + k] : 0;
      rr = r - k * p.rows_seq;
    }
    if (live) {
      const int j = rr / p.group;
      const int hh = rr - j * p.group;
      const uint16_t* src = p.q + (((size_t)seq * p.n_q + j) * p.hq + (size_t)kvh * p.group + hh) * kDX + 2 * lane;
      x[0] = bf16_to_f32(src[0]);
      x[1] = bf16_to_f32(src[1]);
    }
  }
  if (p.rotate_q) wave_fwht<2>(x, lane, p.norm);
  x[0] = x[0] * p.qscale;
  x[1] = x[1] * p.qscale;

  if constexpr (CONV) {
    // conversion route: bf16 hi and lo operands [B][hkv][rows_pad / 16][hi,
    // lo][4 k-steps][64 lanes][4 dwords]; operand lane (quad, n) of k-step j
    // holds channels 32 quad + 8 j .. + 7 of row 16 g + n, the order in which
    // a K lane of group quad offers its converted channels.  This lane's two
    // channels 2 lane, 2 lane + 1 are dword lane & 3 of k-step (lane >> 2) & 3,
    // operand lane 16 (lane >> 4) + n.
    const uint32_t h0 = f32_to_bf16_rne(x[0]), h1 = f32_to_bf16_rne(x[1]);
    const uint32_t l0 = f32_to_bf16_rne(x[0] - bf16_to_f32((uint16_t)h0));
    const uint32_t l1 = f32_to_bf16_rne(x[1] - bf16_to_f32((uint16_t)h1));
    const int g = r >> 4, n = r & 15;
    uint32_t* dst = p.qops + ((((size_t)bh * (p.rows_pad / 16) + g) * 2 * 4 + ((lane >> 2) & 3)) * 64 +
                              16 * (lane >> 4) + n) * 4 + (lane & 3);
    dst[0] = h0 | (h1 << 16);
    dst[4 * 64 * 4] = l0 | (l1 << 16);
    return;
  }

  // 16 lanes per 32-channel block; lane i of the block holds bits 12i ..
  // 12i + 11 of the block's 192-bit stream; lanes 0..5 assemble its dwords,
  // lane 6 the scale byte, lane 7 a zero pad
  const int blk = lane >> 4;
  const int li = lane & 15;
  const int w = min(li, 5);
  const int src_a = 16 * blk + 8 * (w / 3) + 2 * (w % 3);
  const int sh = 8 * (w % 3);
  const int g = r >> 4;
  const int n = r & 15;
  uint32_t* base = p.qops + (size_t)bh * (p.rows_pad / 16) * kTX * 64 * 8;
#pragma unroll
  for (int t = 0; t < kTX; ++t) {
    float am = fmaxf(fabsf(x[0]), fabsf(x[1]));
    am = row16_max(am);
    const int byte = max((int)((as_u32(am) >> 23) & 0xFFu) - 2, 0);
    const int e = byte - 127;
    float v0, v1;
    const uint32_t c0 = e2m3_split(x[0], e, v0);
    const uint32_t c1 = e2m3_split(x[1], e, v1);
    x[0] -= v0;
    x[1] -= v1;
    const uint32_t v12 = c0 | (c1 << 6);
    const uint32_t u24 = v12 | ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v12, kDppXor1, 0xF, 0xF, true) << 12);  // valid on even li
    const uint32_t ua = (uint32_t)__shfl((int)u24, src_a, 64);
    const uint32_t ub = (uint32_t)__shfl((int)u24, src_a + 2, 64);
    const uint32_t d = (ua >> sh) | (ub << (24 - sh));
    uint32_t* dst = base + (((size_t)g * kTX + t) * 64 + 16 * blk + n) * 8;
    if (li < 8) dst[li] = (li < 6) ? d : (li == 6 ? (uint32_t)byte : 0u);
  }
}

// Raw codes a staging wave holds for one tile pair: its one 16-token tile of
// K (codes + scale byte) or of V, lane l = token l%16, group l/16.
struct Stage {
  uint32_t c[4];
  uint32_t sc;
};

// FLAT (cache arrays below 4 GiB): one buffer resource per array from this
// head on (loop-invariant, built once), the page as the 32-bit scalar
// offset; else one resource per (page, head) block.
template <bool FLAT>
__device__ __forceinline__ void load_stage(const DecodeParams& p, const int32_t* bt_row, int kvh, int tile,
                                           bool v, int lane, Stage& t) {
  const int tok = tile * 16;
  const int page = __builtin_amdgcn_readfirstlane(bt_row[tok >> p.p_shift]);
  const int in_page = tok & (p.P - 1);
  const int idx = (lane >> 4) * p.P + (lane & 15);
  __amdgpu_buffer_rsrc_t rc, rs;
  int coff, soff;
  if constexpr (FLAT) {
    const int64_t ch = (int64_t)kvh * p.c_head, sh = (int64_t)kvh * p.s_head;
    rc = block_rsrc(v ? p.vc : p.kc, ch, p.c_total - ch);
    rs = block_rsrc(v ? p.vs : p.ks, sh, p.s_total - sh);
    coff = (int)((uint32_t)page * (uint32_t)p.c_page + (uint32_t)in_page * 16u);
    soff = (int)((uint32_t)page * (uint32_t)p.s_page + (uint32_t)in_page);
  } else {
    const int64_t cb = (int64_t)page * p.c_page + (int64_t)kvh * p.c_head;
    const int64_t sb = (int64_t)page * p.s_page + (int64_t)kvh * p.s_head;
    rc = block_rsrc(v ? p.vc : p.kc, cb, p.c_head);
    rs = block_rsrc(v ? p.vs : p.ks, sb, p.s_head);
    coff = in_page * 16;
    soff = in_page;
  }
  const u32x4_t a = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, idx * 16, coff, 2));
#pragma unroll
  for (int w = 0; w < 4; ++w) t.c[w] = a[w];
  t.sc = __builtin_amdgcn_raw_buffer_load_b8(rs, idx, soff, 0);
}

// GRP: prefix level of a shared-prefix decode (units are prefix groups; see
// DecodeParams); otherwise units are sequences, optionally scanned from
// p.tok_start[b] on.
template <bool GRP, int WAVES, bool CONV = false, bool FLAT = true>
__global__ __launch_bounds__(64 * WAVES) void extend_kernel(const DecodeParams p) {
  constexpr int kRowsX = 16 * WAVES;                // rows per block
  constexpr int kJobs = WAVES >= 4 ? 1 : 4 / WAVES;  // staging jobs per staging wave
  __shared__ __attribute__((aligned(16))) u32x4_t s_k[2][2][64];
  __shared__ uint32_t s_ks[2][2][64];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][2][16][kVRowX];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int col = lane & 15;
  const int quad = lane >> 4;
  const bool hi_col = col < 8;
  // 1-D grid: split fastest, then (sequence or group, KV head), then row
  // block.  Blocks go to the XCDs round-robin; when contexts are ragged only
  // the low splits of a short unit have work, so the split index is rotated
  // by (unit, row block): otherwise a split count divisible by 8 would put
  // all of that work on a few XCDs
  const int units = p.hkv * p.batch;
  const int u = (blockIdx.x / p.splits) % units;
  const int rb = blockIdx.x / (p.splits * units);
  const int split = (int)((blockIdx.x % p.splits + (unsigned)u + (unsigned)rb * units) % p.splits);
  const int kvh = u % p.hkv;
  const int b = u / p.hkv;  // sequence, or prefix group (GRP)
  const int r_last_blk = min(p.rows, (rb + 1) * kRowsX) - 1;
  // blk_tok: tokens 0 .. blk_tok - 1 hold every token a row of this block may
  // see (and are valid cache entries)
  int blk_tok, t0 = 0, m0 = 0, n_mem = 0, L = 0;
  if constexpr (GRP) {
    m0 = p.grp_ptr[b];
    n_mem = p.grp_ptr[b + 1] - m0;
    const int k_hi = min(n_mem, r_last_blk / p.rows_seq + 1);
    blk_tok = 0;
    for (int k = (rb * kRowsX) / p.rows_seq; k < k_hi; ++k) blk_tok = max(blk_tok, p.shared_lens[p.grp_seq[m0 + k]]);
  } else {
    L = p.context_lens[b];
    blk_tok = min(L, L - p.n_q + r_last_blk / p.group + 1);
    if (p.tok_start) t0 = p.tok_start[b] >> 4;
  }
  const int t_begin = t0 + split * p.tiles_per_split;
  const int t_end = min(t_begin + p.tiles_per_split, (blk_tok + 15) >> 4);
  const int tok_limit = min(blk_tok, t_end * 16);
  const int32_t* bt_row = p.block_tables + (size_t)b * p.max_pages;
  // where row r of this unit stores its split partial: per unit, padded
  // rows included, or (GRP) per member sequence (-1: no member)
  auto part_row = [&](int r) -> long long {
    if constexpr (GRP) {
      const int k = r / p.rows_seq;
      if (r >= p.rows || k >= n_mem) return -1;
      const int sq = p.grp_seq[m0 + k];
      return (((long long)sq * p.hkv + kvh) * p.splits + split) * p.rows_seq + (r - k * p.rows_seq);
    } else {
      return ((long long)u * p.splits + split) * p.rows_pad + r;
    }
  };
  if (t_end <= t_begin) {
    // an empty split: (m, l) = (-inf, 0) for the block's rows; a merge never
    // reads the O of a split with zero weight
    if (threadIdx.x < kRowsX) {
      const long long d = part_row(rb * kRowsX + (int)threadIdx.x);
      if (d >= 0) {
        p.ws_ml[d * 2 + 0] = -INFINITY;
        p.ws_ml[d * 2 + 1] = 0.0f;
      }
    }
    return;
  }
  const int n_pairs = (t_end - t_begin + 1) >> 1;
  const int n_iter = (n_pairs + kRingX - 1) / kRingX;  // pairs padded to a multiple of kRingX

  // staging jobs j = 0..3: K tile 0, K tile 1, V tile 0, V tile 1; wave w
  // takes jobs w + WAVES jj (jj < kJobs), so waves 0..3 of a wide block take
  // one each and both waves of a narrow block take two
  const bool stager = w < 4;
  auto fetch = [&](int pi, int j, Stage& c) {
    load_stage<FLAT>(p, bt_row, kvh, min(t_begin + 2 * pi + (j & 1), t_end - 1), j >= 2, lane, c);
  };
  auto stage = [&](int pi, int j, const Stage& c) {
    const int st_tile = j & 1;
    const bool st_v = j >= 2;
    const int par = pi & 1;
    if (!st_v) {
      s_k[par][st_tile][lane] = u32x4_t{c.c[0], c.c[1], c.c[2], c.c[3]};
      s_ks[par][st_tile][lane] = c.sc;
    } else {
      // zero values past the context (their weights are zero; the cache may
      // hold anything there)
      const bool dead = (t_begin + 2 * pi + st_tile) * 16 + col >= tok_limit;
      uint32_t vw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vw[i] = dead ? 0u : c.c[i];
      uint32_t vb[16];
      dequant_group<KVQ_FMT_FP4_E2M1>(vw, scale_operand(dead ? 0u : c.sc), vb);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(&s_v[par][st_tile][col][64 * quad]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{vb[4 * i], vb[4 * i + 1], vb[4 * i + 2], vb[4 * i + 3]};
    }
  };

  Stage ring[kJobs][kRingX];
  if (stager) {
#pragma unroll
    for (int jj = 0; jj < kJobs; ++jj)
#pragma unroll
      for (int k = 0; k < kRingX; ++k) fetch(k, w + WAVES * jj, ring[jj][k]);
  }

  // this wave's 16 rows: query operands (four terms, one per MFMA)
  const int r0 = rb * kRowsX + 16 * w;
  const int g = r0 >> 4;
  i32x8_t qb[kTX];
  int qs[kTX];
  bf16x8_t qv[CONV ? 2 : 1][4];   // conversion route: hi, lo per k-step
  if constexpr (CONV) {
    const uint32_t* src = p.qops + (((size_t)u * (p.rows_pad / 16) + g) * 2 * 4 * 64 + lane) * 4;
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        qv[hl][j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(src + (size_t)(4 * hl + j) * 64 * 4));
  } else {
    const uint32_t* src = p.qops + (((size_t)u * (p.rows_pad / 16) + g) * kTX * 64 + lane) * 8;
#pragma unroll
    for (int t = 0; t < kTX; ++t) {
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(src + (size_t)t * 64 * 8);
      const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(src + (size_t)t * 64 * 8 + 4);
      qb[t] = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], 0, 0};
      qs[t] = (int)a1[2];
    }
  }
  const int row = r0 + col;  // this lane's row (scores and softmax)
  int row_lim = -1;
  if constexpr (GRP) {
    const int k = row / p.rows_seq;
    if (row < p.rows && k < n_mem) {
      const int sq = p.grp_seq[m0 + k];
      const int j = (row - k * p.rows_seq) / p.group;
      row_lim = min(tok_limit - 1, min(p.shared_lens[sq] - 1, p.context_lens[sq] - p.n_q + j));
    }
  } else {
    if (row < p.rows) row_lim = min(tok_limit - 1, L - p.n_q + row / p.group);
  }
  // last token any row of this wave sees: pairs past it leave the wave's
  // state unchanged and are skipped (members of a prefix group may share
  // prefixes of very different lengths)
  int wave_lim = row_lim;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) wave_lim = max(wave_lim, __shfl_xor(wave_lim, o, 64));
  wave_lim = __builtin_amdgcn_readfirstlane(wave_lim);
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t O[8];  // the wave's 16 rows: PV of the hi part of P, then of the lo part
#pragma unroll
  for (int n = 0; n < 8; ++n) O[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (stager) {
#pragma unroll
    for (int jj = 0; jj < kJobs; ++jj) {
      stage(0, w + WAVES * jj, ring[jj][0]);
      fetch(kRingX, w + WAVES * jj, ring[jj][0]);
    }
  }
  __syncthreads();

  // Pairs whose 32 tokens every real row of the wave sees run without
  // score masks (the iterations before n_int_iter); padding rows have zero
  // queries (exact zero scores) and are never read back, so they need none
  // either.
  int vis_all = row_lim >= 0 ? row_lim : 0x7FFFFFFF;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) vis_all = min(vis_all, __shfl_xor(vis_all, o, 64));
  vis_all = __builtin_amdgcn_readfirstlane(vis_all);
  const int int_tok = wave_lim < 0 ? 0 : vis_all + 1;
  const int n_int_pairs = (int_tok >= 16 * t_begin + 32) ? (int_tok - 16 * t_begin - 32) / 32 + 1 : 0;
  const int n_int_iter = min(n_int_pairs, n_pairs) / kRingX;

  auto pair_step = [&](int it, int k, bool masked) {
    const int pi = it * kRingX + k;
    const int par = pi & 1;
    const int tile = t_begin + 2 * pi;
    // ---- stage the next pair (its buffer was last read before the
    // previous barrier), refill the ring slot
    if (stager) {
      const int nk = (k + 1) % kRingX;
#pragma unroll
      for (int jj = 0; jj < kJobs; ++jj) {
        stage(pi + 1, w + WAVES * jj, ring[jj][nk]);
        fetch(pi + 1 + kRingX, w + WAVES * jj, ring[jj][nk]);
      }
    }
    if (!masked || tile * 16 <= wave_lim) {
      // ---- scores of the wave's 16 rows (past the last pair every score is
      // masked: the softmax state does not change)
      f32x4_t S[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4_t kc = s_k[par][s][lane];
        const int ksc = (int)s_ks[par][s][lane];
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (CONV) {
          // K codes with their scale to bf16 (exact); k-step j takes this
          // lane's converted channels 8 j .. 8 j + 7; q hi and lo accumulate
          // into the same scores
          const uint32_t kw[4] = {kc[0], kc[1], kc[2], kc[3]};
          uint32_t kb[16];
          dequant_group<KVQ_FMT_FP4_E2M1>(kw, scale_operand((uint32_t)ksc), kb);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8_t A = __builtin_bit_cast(bf16x8_t, u32x4_t{kb[4 * j], kb[4 * j + 1], kb[4 * j + 2], kb[4 * j + 3]});
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qv[0][j], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qv[1][j], acc, 0, 0, 0);
          }
        } else {
          const i32x8_t A = {(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
#pragma unroll
          for (int t = 0; t < kTX; ++t)
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, qb[t], acc, 4, 2, 0, ksc, 0, qs[t]);
        }
        S[s] = acc;
      }
      float sc[8];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[4 * s + i] = S[s][i];
      if (masked) {
        // score (s, i) is token tile * 16 + 16 s + 4 quad + i: visible while
        // 16 s + i <= rel
        const int rel = row_lim - tile * 16 - 4 * quad;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[4 * s + i] = (16 * s + i <= rel) ? sc[4 * s + i] : -INFINITY;
      }
      float mloc = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                         fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
      mloc = quad_max(mloc);
      // lazy reference maximum: a row's reference moves only when its
      // running maximum passes it by more than kLazyLog2, so most pairs
      // skip the rescale; weights stay below 2^kLazyLog2
      const float m_old = m_run;
      const float m_tgt = fmaxf(m_old, mloc);
      const bool grow = m_tgt > m_old + kLazyLog2;
      const float m_new = grow ? m_tgt : m_old;
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      m_run = m_new;
      float psum = 0.0f;
      // P of this lane's row as bf16 hi (A1) and lo (A2): the wave's 16 rows
      // are the MFMA rows of both, accumulated into the same O
      uint32_t a1[4], a2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(sc[2 * e] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(sc[2 * e + 1] - m_use);
        psum += p0 + p1;
        const uint32_t u0 = as_u32(p0), u1 = as_u32(p1);
        a1[e] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
        a2[e] = pack_bf16x2(p0 - as_f32(u0 & 0xFFFF0000u), p1 - as_f32(u1 & 0xFFFF0000u));
      }
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {
        // a row max moved: rescale.  Lane (quad, c) of O holds rows 4 quad + i;
        // lane c holds the factor of row c (in every quad)
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_use);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * quad + i, 64);
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            O[n][i] *= al;
          }
        }
      }
      l_run += psum;
      const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, u32x4_t{a1[0], a1[1], a1[2], a1[3]});
      const bf16x8_t A2 = __builtin_bit_cast(bf16x8_t, u32x4_t{a2[0], a2[1], a2[2], a2[3]});

      // ---- PV: B operands read transposed from the LDS V tiles
      const int rr = col >> 2;
      const int c4 = (col & 3) * 4;
      typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
      auto read_b = [&](int n) {
        lds_bf16x4* p0 = (lds_bf16x4*)((__attribute__((address_space(3))) uint8_t*)&s_v[par][0][4 * quad + rr][2 * (16 * n + c4)]);
        lds_bf16x4* p1 = (lds_bf16x4*)((__attribute__((address_space(3))) uint8_t*)&s_v[par][1][4 * quad + rr][2 * (16 * n + c4)]);
        const u32x2_t w0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p0));
        const u32x2_t w1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p1));
        return __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
      };
      bf16x8_t B0 = read_b(0);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const bf16x8_t C0 = (n + 1 < 8) ? read_b(n + 1) : B0;
        O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B0, O[n], 0, 0, 0);
        O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, B0, O[n], 0, 0, 0);
        B0 = C0;
      }
    }
    __syncthreads();
  };

  // one loop with a uniform mask flag: two loops (masked, unmasked) made
  // the compiler rotate the accumulators through copies
#pragma unroll 1
  for (int it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int k = 0; k < kRingX; ++k) pair_step(it, k, it >= n_int_iter);
  }
  // ---- partials: O = hi part + lo part (lane (quad, c) holds rows 4 quad + i
  // of the wave, channel 16 n + c), row sums; rows past p.rows are padding
  const float lrow = quad_sum(l_run);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long long d = part_row(r0 + 4 * quad + i);
    if (d >= 0) {
#pragma unroll
      for (int n = 0; n < 8; ++n) p.ws_o[d * kDX + 16 * n + col] = O[n][i];
    }
  }
  if (lane < 16) {
    const long long d = part_row(r0 + lane);
    if (d >= 0) {
      p.ws_ml[d * 2 + 0] = m_run;
      p.ws_ml[d * 2 + 1] = lrow;
    }
  }
}

constexpr int kMinTilesPerSplitX = 8;
constexpr int kMaxTilesPerSplitX = 512;
constexpr int kNarrowTilesPerSplitX = 256;
constexpr int kDefaultSlotsX = 256;  // wide blocks: one per CU (MI355X); narrow: six
constexpr int kMaxDevicesX = 64;
constexpr int kMaxRowsX = 1 << 16;

template <int WAVES, bool CONV = false>
int resident_blocks_x() {
  static std::atomic<int> cache[kMaxDevicesX];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < kMaxDevicesX) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0, blocks = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, extend_kernel<false, WAVES, CONV>, 64 * WAVES, 0) !=
          hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int v = cus * blocks;
  if (dev < kMaxDevicesX) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

int plan_extend(const CacheGeom& c, int batch, int hq, int n_q, int max_context_len, uint32_t flags,
                DecodePlan* plan) {
  return plan_extend_rows(c, batch, (long long)(hq / c.hkv) * n_q, max_context_len, flags, plan);
}

int plan_extend_rows(const CacheGeom& c, int batch, long long rows, int max_context_len, uint32_t flags,
                     DecodePlan* plan, int block_rows) {
  if (c.d != kDX || c.fmt != KVQ_FMT_FP4_E2M1) return KVQ_ERR_UNSUPPORTED;
  if (rows < 1 || rows > kMaxRowsX) return KVQ_ERR_UNSUPPORTED;
  const bool conv = (flags & KVQ_QK_CONVERT) != 0;
  if (block_rows == 0) block_rows = rows <= kNarrowMaxRows ? 16 * kNarrowX : 16 * kWideX;
  if (block_rows != 16 * kNarrowX && block_rows != 16 * kWideX) return KVQ_ERR_UNSUPPORTED;
  const int kRowsX = block_rows;
  const int row_blocks = (int)((rows + kRowsX - 1) / kRowsX);
  const int n_tiles = (int)(((long long)max_context_len + 15) / 16);
  int splits = (int)((flags & KVQ_SPLITS_MASK) >> KVQ_SPLITS_SHIFT);
  if (splits <= 0) {
    // one round of blocks over the device, at least kMinTilesPerSplitX tiles
    // and at most a cap per split (below)
    int slots = block_rows == 16 * kNarrowX ? (conv ? resident_blocks_x<kNarrowX, true>() : resident_blocks_x<kNarrowX>())
                                             : (conv ? resident_blocks_x<kWideX, true>() : resident_blocks_x<kWideX>());
    if (slots <= 0) slots = block_rows == 16 * kNarrowX ? 6 * kDefaultSlotsX : kDefaultSlotsX;
    const long long work = (long long)batch * c.hkv * row_blocks;
    long long want = work >= slots ? 1 : slots / work;
    const long long by_len = n_tiles / kMinTilesPerSplitX;
    if (want > by_len) want = by_len;
    // Only the longest context is known here.  A cap above one round's
    // split count is rounded up to whole rounds (a partial last round would
    // leave most of the device idle on a batch of equal contexts).  Narrow
    // blocks (decode-like rows, where batches are ragged) also take a smaller
    // cap when it asks for at least two rounds: the longest sequences of a
    // ragged batch then spread over more blocks.
    const long long per_round = work >= slots ? 1 : slots / work;
    auto whole_rounds = [&](long long n) { return (n + per_round - 1) / per_round * per_round; };
    const long long by_cap = (n_tiles + kMaxTilesPerSplitX - 1) / kMaxTilesPerSplitX;
    if (want < by_cap) want = whole_rounds(by_cap);
    if (block_rows == 16 * kNarrowX) {
      const long long by_narrow = (n_tiles + kNarrowTilesPerSplitX - 1) / kNarrowTilesPerSplitX;
      if (by_narrow >= 2 * per_round && want < by_narrow) want = whole_rounds(by_narrow);
    }
    splits = (int)(want < 1 ? 1 : want);
  }
  if (splits > kMaxSplits) splits = kMaxSplits;
  int per = (n_tiles + splits - 1) / splits;
  per = (per + 1) & ~1;
  if (per < 2) per = 2;
  splits = (n_tiles + per - 1) / per;
  if (splits < 1) splits = 1;
  const size_t rows_pad = (size_t)row_blocks * kRowsX;
  plan->rows = (int)rows;
  plan->row_tiles = row_blocks;
  plan->block_rows = block_rows;
  plan->splits = splits;
  plan->tiles_per_split = per;
  plan->qk_convert = conv ? 1 : 0;
  // query operands per 16-row group: kTX FP6 terms of 8 dwords per lane, or
  // (conversion route) bf16 hi and lo of 4 k-steps of 4 dwords: the same size
  plan->qops_bytes = (size_t)batch * c.hkv * (rows_pad / 16) * kTX * 64 * 8 * sizeof(uint32_t);
  plan->workspace = plan->qops_bytes + (size_t)batch * c.hkv * splits * rows_pad * (kDX + 2) * sizeof(float);
  return KVQ_OK;
}

template <bool GRP, int WAVES, bool CONV>
void launch_x(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  if (p.flat)
    hipLaunchKernelGGL((extend_kernel<GRP, WAVES, CONV, true>), grid, dim3(64 * WAVES), 0, stream, p);
  else
    hipLaunchKernelGGL((extend_kernel<GRP, WAVES, CONV, false>), grid, dim3(64 * WAVES), 0, stream, p);
}

hipError_t launch_extend(const DecodeArgs& a, hipStream_t stream) {
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
  p.batch = a.batch;
  p.q = a.q;
  p.hq = a.hq;
  p.n_q = a.n_q;
  p.group = a.group;
  p.rows = a.plan.rows;
  p.rows_pad = a.plan.row_tiles * a.plan.block_rows;
  p.block_tables = a.block_tables;
  p.max_pages = a.max_pages;
  p.context_lens = a.context_lens;
  p.qscale = a.qscale;
  p.norm = fwht_norm(kDX);
  p.rotate_q = a.rotate_q;
  p.rotate_out = a.rotate_out;
  p.splits = a.plan.splits;
  p.tiles_per_split = a.plan.tiles_per_split;
  p.out = a.out;
  p.tok_start = a.tok_start;
  p.grp_ptr = a.grp_ptr;
  p.grp_seq = a.grp_seq;
  p.shared_lens = a.shared_lens;
  p.rows_seq = a.rows_seq;
  p.keep_partials = a.keep_partials;
  const bool grp = a.grp_ptr != nullptr;
  const size_t units = (size_t)a.batch * a.c.hkv;
  // partial rows: per unit and padded, or (prefix level) per member sequence
  const size_t part_rows = grp ? (size_t)a.grp_seqs * a.c.hkv * a.rows_seq : units * p.rows_pad;
  const size_t n_o = part_rows * a.plan.splits * kDX;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.workspace);
  p.qops = reinterpret_cast<uint32_t*>(ws);
  p.ws_o = reinterpret_cast<float*>(ws + a.plan.qops_bytes);
  p.ws_ml = p.ws_o + n_o;
  const unsigned qblocks = (unsigned)(units * p.rows_pad / 4);
  const bool conv = a.plan.qk_convert != 0 && !grp;  // the prefix level keeps the native route
  if (conv)
    hipLaunchKernelGGL(qprep_ext_kernel<true>, dim3(qblocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(qprep_ext_kernel<false>, dim3(qblocks), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((size_t)p.splits * units * a.plan.row_tiles));
  const bool narrow = a.plan.block_rows == 16 * kNarrowX;
  if (conv && narrow)
    launch_x<false, kNarrowX, true>(p, grid, stream);
  else if (conv)
    launch_x<false, kWideX, true>(p, grid, stream);
  else if (grp && narrow)
    launch_x<true, kNarrowX, false>(p, grid, stream);
  else if (grp)
    launch_x<true, kWideX, false>(p, grid, stream);
  else if (narrow)
    launch_x<false, kNarrowX, false>(p, grid, stream);
  else
    launch_x<false, kWideX, false>(p, grid, stream);
  e = hipGetLastError();
  if (e != hipSuccess || a.keep_partials) return e;
  hipLaunchKernelGGL((merge_kernel<0, 2>), dim3(qblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq

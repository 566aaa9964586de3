// Shared-prefix (cascade) decode over the FP4 cache, head_dim 128.
//
// Method: ROCm blog "UltraQuant on AMD Instinct", section "Agentic serving:
// workload and setup" (agent traffic: long prefixes shared across requests,
// a high prefix-cache hit rate) and section "Why UltraQuant beats 8-bit KV"
// (every decode step re-reads the cache).  The attention each query row
// computes is unchanged; only the order of the reads is: the pages of a
// prefix that several sequences share are scanned once for all their rows.
//
//  1. prefix level: the many-row kernel with one unit per (prefix group, KV
//     head); the rows of all members are gathered, member s sees prefix
//     tokens 0 .. shared_lens[s] - 1 (and the causal rule of its verify
//     positions); partials are stored per member sequence;
//  2. suffix level: the ordinary decode kernel of the row count (up to 24
//     rows: one wave per unit; more: the many-row kernel) over each
//     sequence's tokens shared_lens[b] .. context_lens[b] - 1;
//  3. merge: per query row, the log-sum-exp combination of both levels'
//     split partials (base 2), normalise, rotate back, store.
#include "kvq_decode_common.h"

namespace kvq {
namespace {

constexpr int kDS = 128;
constexpr int kMaxLevelSplits = kMaxSplits / 2;  // both levels share one wave's lanes in the merge
// Tiles per split unless the caller forces the split count.  Prefix lengths
// and suffix lengths are ragged, and only their maxima are known here: short
// splits keep the longest ones from setting the time of the call (a split
// with no tile of its sequence leaves at once).
constexpr int kPrefixTilesPerSplit = 256;
constexpr int kSuffixTilesPerSplit = 32;

struct MergeParams {
  const float* o1;   // prefix partials [B][hkv][s1][rows_seq][D]
  const float* ml1;  // (m, l) of each
  const float* o2;   // suffix partials [B][hkv][s2][rows2][D]
  const float* ml2;
  const int32_t* shared_lens;
  float* out;
  int s1, s2, rows2;
  int batch, hkv, hq, n_q, group, rows_seq;
  int rotate_out;
  float norm;
};

// One wave per (sequence, KV head, row); lane s < s1 holds prefix split s's
// (m, l), lane s1 + s suffix split s's; lane l accumulates channels 2l, 2l+1.
__global__ __launch_bounds__(256) void shared_merge_kernel(const MergeParams m) {
  constexpr int C = 2;
  const int lane = threadIdx.x & 63;
  const long long gr = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r = (int)(gr % m.rows_seq);
  const long long bh = gr / m.rows_seq;
  if (bh >= (long long)m.batch * m.hkv) return;  // grid padding: the whole wave leaves
  const int kvh = (int)(bh % m.hkv);
  const int b = (int)(bh / m.hkv);
  // a sequence with no shared tokens has no prefix partial
  const int S1 = m.shared_lens[b] > 0 ? m.s1 : 0;
  const int S = S1 + m.s2;
  const float* ml = nullptr;
  if (lane < S1)
    ml = m.ml1 + ((bh * m.s1 + lane) * m.rows_seq + r) * 2;
  else if (lane < S)
    ml = m.ml2 + ((bh * m.s2 + (lane - S1)) * m.rows2 + r) * 2;
  float ms = -INFINITY, ls = 0.0f;
  if (ml) {
    ms = ml[0];
    ls = ml[1];
  }
  float lsum = 0.0f;
  float acc[C] = {0.0f, 0.0f};
  const float* p1 = m.o1 + ((size_t)bh * m.s1 * m.rows_seq + r) * kDS + C * lane;
  const float* p2 = m.o2 + ((size_t)bh * m.s2 * m.rows2 + r) * kDS + C * lane;
  // S >= 1: the suffix level has at least one split
  merge_splits<C>(
      acc, S,
      [&](int sp) { return sp < S1 ? p1 + (size_t)sp * m.rows_seq * kDS : p2 + (size_t)(sp - S1) * m.rows2 * kDS; },
      [&] {
        float M = ms;
        M = wave_max(M, lane);
        const float ws = (M != -INFINITY) ? __builtin_amdgcn_exp2f(ms - M) : 0.0f;
        lsum = ws * ls;
        lsum = wave_sum(lsum, lane);
        return ws;
      });
  const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
  acc[0] *= inv;
  acc[1] *= inv;
  if (m.rotate_out) wave_fwht<C>(acc, lane, m.norm);
  const int j = r / m.group;
  const int hh = r - j * m.group;
  float* dst = m.out + (((size_t)b * m.n_q + j) * m.hq + (size_t)kvh * m.group + hh) * kDS + C * lane;
  *reinterpret_cast<f32x2_t*>(dst) = f32x2_t{acc[0], acc[1]};
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Plan one level of n_tiles tiles at most: the caller's split count if it
// forces one, else the kernel's own plan refined to at most max_per tiles per
// split; never more splits than the merge holds.
template <typename F>
int plan_level(F plan_fn, uint32_t flags, int n_tiles, int max_per, DecodePlan* plan) {
  const uint32_t base = flags & ~KVQ_SPLITS_MASK;
  const int forced = (int)((flags & KVQ_SPLITS_MASK) >> KVQ_SPLITS_SHIFT);
  if (forced > 0) return plan_fn(base | KVQ_SPLITS(forced < kMaxLevelSplits ? forced : kMaxLevelSplits), plan);
  int st = plan_fn(base, plan);
  if (st != KVQ_OK) return st;
  int want = plan->splits;
  if (plan->tiles_per_split > max_per) want = (n_tiles + max_per - 1) / max_per;
  if (want > kMaxLevelSplits) want = kMaxLevelSplits;
  if (want == plan->splits) return KVQ_OK;
  return plan_fn(base | KVQ_SPLITS(want), plan);
}

}  // namespace

int plan_shared(const CacheGeom& c, int batch, int hq, int n_q, const kvq_prefix_groups& g, uint32_t flags,
                SharedPlan* plan) {
  if (c.d != kDS || c.fmt != KVQ_FMT_FP4_E2M1) return KVQ_ERR_UNSUPPORTED;
  const long long rows_seq = (long long)(hq / c.hkv) * n_q;
  const long long pre_rows = rows_seq * g.max_group_size;
  const int prefix_len = g.max_prefix_pages * c.p;
  int st = plan_level(
      // 32-row blocks: a block holds about one member's rows, so it scans
      // little beyond that member's shared length (members of one group may
      // share prefixes of very different lengths)
      [&](uint32_t f, DecodePlan* p) { return plan_extend_rows(c, g.num_groups, pre_rows, prefix_len, f, p, 32); },
      flags, (int)(((long long)prefix_len + 15) / 16), kPrefixTilesPerSplit, &plan->prefix);
  if (st != KVQ_OK) return st;
  plan->prefix.kind = kDecodeMany;
  // prefix partials are stored per member sequence, not per padded unit
  plan->prefix.workspace =
      plan->prefix.qops_bytes + (size_t)batch * c.hkv * plan->prefix.splits * rows_seq * (kDS + 2) * sizeof(float);
  const int suffix_len = g.max_suffix_len > 0 ? g.max_suffix_len : 1;
  st = plan_level([&](uint32_t f, DecodePlan* p) { return plan_decode(c, batch, hq, n_q, suffix_len, f, p); },
                  flags, (int)(((long long)suffix_len + 15) / 16), kSuffixTilesPerSplit, &plan->suffix);
  if (st != KVQ_OK) return st;
  plan->suffix_offset = align256(plan->prefix.workspace);
  plan->workspace = plan->suffix_offset + plan->suffix.workspace;
  return KVQ_OK;
}

hipError_t launch_shared(const SharedArgs& a, hipStream_t stream) {
  const SharedPlan& sp = a.plan;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.base.workspace);
  const int rows_seq = a.base.group * a.base.n_q;

  // 1. prefix level
  DecodeArgs pre = a.base;
  pre.plan = sp.prefix;
  pre.batch = a.groups.num_groups;
  pre.block_tables = a.groups.prefix_tables;
  pre.max_pages = a.groups.max_prefix_pages;
  pre.grp_ptr = a.groups.indptr;
  pre.grp_seq = a.groups.members;
  pre.shared_lens = a.groups.shared_lens;
  pre.rows_seq = rows_seq;
  pre.grp_seqs = a.base.batch;
  pre.keep_partials = 1;
  pre.workspace = reinterpret_cast<float*>(ws);
  hipError_t e = launch_extend(pre, stream);
  if (e != hipSuccess) return e;

  // 2. suffix level
  DecodeArgs suf = a.base;
  suf.plan = sp.suffix;
  suf.tok_start = a.groups.shared_lens;
  suf.keep_partials = 1;
  suf.workspace = reinterpret_cast<float*>(ws + sp.suffix_offset);
  e = launch_decode(suf, stream);
  if (e != hipSuccess) return e;

  // 3. merge both levels
  MergeParams m{};
  const size_t n_o1 = (size_t)a.base.batch * a.base.c.hkv * sp.prefix.splits * rows_seq * kDS;
  m.o1 = reinterpret_cast<const float*>(ws + sp.prefix.qops_bytes);
  m.ml1 = m.o1 + n_o1;
  const int rows2 = sp.suffix.kind == kDecodeMany ? sp.suffix.row_tiles * sp.suffix.block_rows : 8 * sp.suffix.row_tiles;
  const size_t n_o2 = (size_t)a.base.batch * a.base.c.hkv * sp.suffix.splits * rows2 * kDS;
  m.o2 = reinterpret_cast<const float*>(ws + sp.suffix_offset + sp.suffix.qops_bytes);
  m.ml2 = m.o2 + n_o2;
  m.shared_lens = a.groups.shared_lens;
  m.out = a.base.out;
  m.s1 = sp.prefix.splits;
  m.s2 = sp.suffix.splits;
  m.rows2 = rows2;
  m.batch = a.base.batch;
  m.hkv = a.base.c.hkv;
  m.hq = a.base.hq;
  m.n_q = a.base.n_q;
  m.group = a.base.group;
  m.rows_seq = rows_seq;
  m.rotate_out = a.base.rotate_out;
  m.norm = fwht_norm(kDS);
  const size_t waves = (size_t)a.base.batch * a.base.c.hkv * rows_seq;
  hipLaunchKernelGGL(shared_merge_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace kvq

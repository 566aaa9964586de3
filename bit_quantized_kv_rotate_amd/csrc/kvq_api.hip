// C entry points of libkvq: argument checks on the host, then kernel
// launches on the caller's stream.  Nothing here allocates device memory or
// synchronises.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <mutex>

#include "kvq_internal.h"

// Scratch of kvq_decode_attn_fp4_scratch: one copy per device, resident while
// the code object is loaded.  Host code must not pass `scratch` itself to a
// kernel (on the host the name is a stand-in, not a device address): it uses
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[KVQ_SCRATCH_BYTES];

namespace kvq {

float fwht_norm(int d) { return (float)(1.0 / std::sqrt((double)d)); }

namespace {

thread_local hipError_t g_last_hip = hipSuccess;
thread_local char g_msg[256];

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Largest host-side token bound a call takes (max_context_len, max_selected,
// a prefix's tokens): tile and token counts derived from it stay far from
// int32 overflow on the host and on the device.
constexpr int64_t kMaxTokens = (int64_t)1 << 30;

// Validate a description; fills geometry.  Pointers are checked by callers
// that use them.
int check_desc(const kvq_cache_desc* d, CacheGeom* g) {
  if (!d) return KVQ_ERR_NULL;
  if (d->format != KVQ_FMT_FP4_E2M1 && d->format != KVQ_FMT_FP8_E4M3) return KVQ_ERR_FORMAT;
  if (d->num_kv_heads <= 0 || d->num_pages <= 0 || d->head_dim <= 0 || d->page_size <= 0)
    return KVQ_ERR_SHAPE;
  if (!pow2(d->head_dim) || d->head_dim < 32 || d->head_dim > 1024) return KVQ_ERR_SHAPE;
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64) return KVQ_ERR_UNSUPPORTED;
  if (d->rotate != 0 && d->rotate != 1) return KVQ_ERR_SHAPE;
  if (d->kv_shared != 0 && d->kv_shared != 1) return KVQ_ERR_SHAPE;
  g->fmt = d->format;
  g->rotate = d->rotate;
  g->kv_shared = d->kv_shared;
  g->hkv = d->num_kv_heads;
  g->d = d->head_dim;
  g->g = d->head_dim / 32;
  g->p = d->page_size;
  g->num_pages = d->num_pages;
  g->cb = (d->format == KVQ_FMT_FP4_E2M1) ? 16 : 32;
  g->c_head = (int64_t)g->g * g->p * g->cb;
  g->c_page = (int64_t)g->hkv * g->c_head;
  g->s_head = (int64_t)g->g * g->p;
  g->s_page = (int64_t)g->hkv * g->s_head;
  g->kc = (const uint8_t*)d->k_codes;
  g->ks = (const uint8_t*)d->k_scales;
  g->vc = (const uint8_t*)d->v_codes;
  g->vs = (const uint8_t*)d->v_scales;
  return KVQ_OK;
}

int check_cache_ptrs(const kvq_cache_desc* d) {
  if (!d->k_codes || !d->k_scales) return KVQ_ERR_NULL;
  if (!d->kv_shared && (!d->v_codes || !d->v_scales)) return KVQ_ERR_NULL;
  // code arrays are read and written in 16-byte (token, group) units
  if ((uintptr_t)d->k_codes & 15u) return KVQ_ERR_SHAPE;
  if (!d->kv_shared && ((uintptr_t)d->v_codes & 15u)) return KVQ_ERR_SHAPE;
  return KVQ_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KVQ_OK;
  g_last_hip = e;
  return KVQ_ERR_HIP;
}

// Device address of the current device's `scratch` array, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
constexpr int kScratchDevices = 64;

void* scratch_address() {
  static std::atomic<void*> addr[kScratchDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !q) {
      g_last_hip = e != hipSuccess ? e : hipErrorInvalidSymbol;
      (void)hipGetLastError();
      return nullptr;
    }
    p = q;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

int decode_common(int want_fmt, const kvq_cache_desc* desc, const void* q, int32_t batch,
                  int32_t num_q_heads, int32_t n_q, const int32_t* block_tables,
                  int32_t max_pages_per_seq, const int32_t* context_lens, int32_t max_context_len,
                  float sm_scale, uint32_t flags, float* out, void* workspace,
                  size_t workspace_bytes, kvq_stream_t stream, const AppendArgs* append = nullptr,
                  bool use_scratch = false) {
  CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != KVQ_OK) return st;
  if (g.fmt != want_fmt) return KVQ_ERR_FORMAT;
  st = check_cache_ptrs(desc);
  if (st != KVQ_OK) return st;
  if (!q || !block_tables || !context_lens || !out) return KVQ_ERR_NULL;
  if (batch < 0 || num_q_heads <= 0 || n_q < 1 || max_pages_per_seq <= 0 || max_context_len < 0)
    return KVQ_ERR_SHAPE;
  if (max_context_len > kMaxTokens) return KVQ_ERR_SHAPE;
  if (num_q_heads % g.hkv != 0) return KVQ_ERR_SHAPE;
  if ((int64_t)max_pages_per_seq * g.p < (int64_t)max_context_len) return KVQ_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_SHAPE;
  if (flags & ~(KVQ_Q_PREROTATED | KVQ_OUT_ROTATED | KVQ_QK_CONVERT | KVQ_SPLITS_MASK)) return KVQ_ERR_SHAPE;
  if (batch == 0) {
    // nothing to attend to; an append still runs
    if (append && append->n_tokens > 0)
      return hip_status(launch_append(g, append->kc, append->ks, append->vc, append->vs, append->k_new,
                                      append->v_new, append->slots, append->n_tokens, (hipStream_t)stream));
    return KVQ_OK;
  }
  DecodePlan plan;
  st = plan_decode(g, batch, num_q_heads, n_q, max_context_len > 0 ? max_context_len : 1, flags, &plan);
  if (st != KVQ_OK) return st;
  if (use_scratch) {
    // the allocation-free entry point: the static array instead of a workspace
    if (plan.workspace > KVQ_SCRATCH_BYTES) return KVQ_ERR_SCRATCH;
    workspace = scratch_address();
    if (!workspace) return KVQ_ERR_HIP;
    workspace_bytes = KVQ_SCRATCH_BYTES;
  }
  if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace)) return KVQ_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 15u) return KVQ_ERR_WORKSPACE;
  DecodeArgs a;
  a.c = g;
  a.plan = plan;
  a.q = (const uint16_t*)q;
  a.batch = batch;
  a.hq = num_q_heads;
  a.n_q = n_q;
  a.group = num_q_heads / g.hkv;
  a.block_tables = block_tables;
  a.max_pages = max_pages_per_seq;
  a.context_lens = context_lens;
  a.qscale = (float)((double)sm_scale * 1.4426950408889634);  // log2(e)
  a.rotate_q = g.rotate && !(flags & KVQ_Q_PREROTATED);
  a.rotate_out = g.rotate && !(flags & KVQ_OUT_ROTATED);
  a.out = out;
  a.workspace = (float*)workspace;
  a.append = append;
  return hip_status(launch_decode(a, (hipStream_t)stream));
}

// Host-side fields of a shared-prefix call's groups, and its plan.
int plan_shared_call(const CacheGeom& g, int32_t batch, int32_t num_q_heads, int32_t n_q,
                     const kvq_prefix_groups* groups, uint32_t flags, SharedPlan* plan) {
  if (!groups) return KVQ_ERR_NULL;
  if (batch <= 0 || num_q_heads <= 0 || n_q < 1 || num_q_heads % g.hkv != 0) return KVQ_ERR_SHAPE;
  if (groups->num_groups < 1 || groups->max_group_size < 1 || groups->max_prefix_pages < 1 ||
      groups->max_suffix_len < 0)
    return KVQ_ERR_SHAPE;
  if (flags & ~(KVQ_Q_PREROTATED | KVQ_OUT_ROTATED | KVQ_SPLITS_MASK)) return KVQ_ERR_SHAPE;
  if ((int64_t)groups->max_prefix_pages * g.p > kMaxTokens || groups->max_suffix_len > kMaxTokens)
    return KVQ_ERR_SHAPE;
  if (g.d != 128) return KVQ_ERR_UNSUPPORTED;
  const int64_t rows_seq = (int64_t)(num_q_heads / g.hkv) * n_q;
  if (rows_seq > 65536 || rows_seq * groups->max_group_size > 65536) return KVQ_ERR_UNSUPPORTED;
  return plan_shared(g, batch, num_q_heads, n_q, *groups, flags, plan);
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" {

size_t kvq_cache_code_bytes(const kvq_cache_desc* desc) {
  CacheGeom g;
  if (check_desc(desc, &g) != KVQ_OK) return 0;
  return (size_t)g.c_page * (size_t)g.num_pages;
}

size_t kvq_cache_scale_bytes(const kvq_cache_desc* desc) {
  CacheGeom g;
  if (check_desc(desc, &g) != KVQ_OK) return 0;
  return (size_t)g.s_page * (size_t)g.num_pages;
}

int kvq_rotate_quantize_append(const kvq_cache_desc* desc, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, int32_t n_tokens, kvq_stream_t stream) {
  CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != KVQ_OK) return st;
  st = check_cache_ptrs(desc);
  if (st != KVQ_OK) return st;
  if (n_tokens < 0) return KVQ_ERR_SHAPE;
  if (n_tokens == 0) return KVQ_OK;
  if (!k_new || !slot_mapping) return KVQ_ERR_NULL;
  if (!g.kv_shared && !v_new) return KVQ_ERR_NULL;
  return hip_status(launch_append(g, (uint8_t*)desc->k_codes, (uint8_t*)desc->k_scales,
                                  (uint8_t*)desc->v_codes, (uint8_t*)desc->v_scales,
                                  (const uint16_t*)k_new, (const uint16_t*)v_new, slot_mapping,
                                  n_tokens, (hipStream_t)stream));
}

size_t kvq_decode_workspace_bytes(const kvq_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                                  int32_t n_q, int32_t max_context_len, uint32_t flags) {
  CacheGeom g;
  if (check_desc(desc, &g) != KVQ_OK) return 0;
  if (batch <= 0 || num_q_heads <= 0 || n_q < 1 || max_context_len < 0 || max_context_len > kMaxTokens) return 0;
  if (num_q_heads % g.hkv != 0) return 0;
  DecodePlan plan;
  // the decode call plans a context of at least one token, as here
  if (plan_decode(g, batch, num_q_heads, n_q, max_context_len > 0 ? max_context_len : 1, flags, &plan) != KVQ_OK)
    return 0;
  return plan.workspace;
}

size_t kvq_decode_shared_workspace_bytes(const kvq_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                                         int32_t n_q, const kvq_prefix_groups* groups, uint32_t flags) {
  CacheGeom g;
  if (check_desc(desc, &g) != KVQ_OK || g.fmt != KVQ_FMT_FP4_E2M1) return 0;
  SharedPlan plan;
  if (plan_shared_call(g, batch, num_q_heads, n_q, groups, flags, &plan) != KVQ_OK) return 0;
  return plan.workspace;
}

int kvq_decode_attn_fp4_shared(const kvq_cache_desc* desc, const void* q, int32_t batch,
                               int32_t num_q_heads, int32_t n_q, const int32_t* block_tables,
                               int32_t max_pages_per_seq, const int32_t* context_lens, int32_t max_context_len,
                               const kvq_prefix_groups* groups, float sm_scale, uint32_t flags, float* out,
                               void* workspace, size_t workspace_bytes, kvq_stream_t stream) {
  CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != KVQ_OK) return st;
  if (g.fmt != KVQ_FMT_FP4_E2M1) return KVQ_ERR_FORMAT;
  st = check_cache_ptrs(desc);
  if (st != KVQ_OK) return st;
  if (!q || !block_tables || !context_lens || !out || !groups) return KVQ_ERR_NULL;
  if (!groups->indptr || !groups->members || !groups->prefix_tables || !groups->shared_lens)
    return KVQ_ERR_NULL;
  if (batch < 0 || max_pages_per_seq <= 0 || max_context_len < 0 || max_context_len > kMaxTokens)
    return KVQ_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_SHAPE;
  if (batch == 0) return KVQ_OK;
  SharedPlan plan;
  st = plan_shared_call(g, batch, num_q_heads, n_q, groups, flags, &plan);
  if (st != KVQ_OK) return st;
  // the suffix scan indexes block_tables[b] by token position up to
  // context_lens[b] - 1, so a row must cover the longest context
  if ((int64_t)max_pages_per_seq * g.p < (int64_t)max_context_len) return KVQ_ERR_SHAPE;
  if (groups->max_suffix_len > max_context_len) return KVQ_ERR_SHAPE;
  if (!workspace || workspace_bytes < plan.workspace) return KVQ_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 15u) return KVQ_ERR_WORKSPACE;
  SharedArgs a;
  a.base.c = g;
  a.base.q = (const uint16_t*)q;
  a.base.batch = batch;
  a.base.hq = num_q_heads;
  a.base.n_q = n_q;
  a.base.group = num_q_heads / g.hkv;
  a.base.block_tables = block_tables;
  a.base.max_pages = max_pages_per_seq;
  a.base.context_lens = context_lens;
  a.base.qscale = (float)((double)sm_scale * 1.4426950408889634);  // log2(e)
  a.base.rotate_q = g.rotate && !(flags & KVQ_Q_PREROTATED);
  a.base.rotate_out = g.rotate && !(flags & KVQ_OUT_ROTATED);
  a.base.out = out;
  a.base.workspace = (float*)workspace;
  a.plan = plan;
  a.groups = *groups;
  return hip_status(launch_shared(a, (hipStream_t)stream));
}

size_t kvq_decode_selected_workspace_bytes(const kvq_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                                           int32_t max_selected, uint32_t flags) {
  CacheGeom g;
  if (check_desc(desc, &g) != KVQ_OK || g.fmt != KVQ_FMT_FP4_E2M1 || g.d != 512) return 0;
  if (batch <= 0 || num_q_heads <= 0 || max_selected < 0 || max_selected > kMaxTokens ||
      num_q_heads % g.hkv != 0)
    return 0;
  DecodePlan plan;
  if (plan_decode(g, batch, num_q_heads, 1, max_selected > 0 ? max_selected : 1, flags, &plan) != KVQ_OK) return 0;
  return plan.workspace;
}

int kvq_decode_attn_fp4_selected(const kvq_cache_desc* desc, const void* q, int32_t batch, int32_t num_q_heads,
                                 const int32_t* block_tables, int32_t max_pages_per_seq, const int32_t* sel,
                                 const int32_t* sel_lens, int32_t max_selected, float sm_scale, uint32_t flags,
                                 float* out, void* workspace, size_t workspace_bytes, kvq_stream_t stream) {
  CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != KVQ_OK) return st;
  if (g.fmt != KVQ_FMT_FP4_E2M1) return KVQ_ERR_FORMAT;
  st = check_cache_ptrs(desc);
  if (st != KVQ_OK) return st;
  if (!q || !block_tables || !sel || !sel_lens || !out) return KVQ_ERR_NULL;
  if (batch < 0 || num_q_heads <= 0 || max_pages_per_seq <= 0 || max_selected < 0 || max_selected > kMaxTokens)
    return KVQ_ERR_SHAPE;
  if (num_q_heads % g.hkv != 0) return KVQ_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_SHAPE;
  if (flags & ~(KVQ_Q_PREROTATED | KVQ_OUT_ROTATED | KVQ_SPLITS_MASK)) return KVQ_ERR_SHAPE;
  if (g.d != 512) return KVQ_ERR_UNSUPPORTED;
  if (batch == 0) return KVQ_OK;
  DecodePlan plan;
  st = plan_decode(g, batch, num_q_heads, 1, max_selected > 0 ? max_selected : 1, flags, &plan);
  if (st != KVQ_OK) return st;
  if (!workspace || workspace_bytes < plan.workspace) return KVQ_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 15u) return KVQ_ERR_WORKSPACE;
  DecodeArgs a;
  a.c = g;
  a.plan = plan;
  a.q = (const uint16_t*)q;
  a.batch = batch;
  a.hq = num_q_heads;
  a.n_q = 1;
  a.group = num_q_heads / g.hkv;
  a.block_tables = block_tables;
  a.max_pages = max_pages_per_seq;
  a.context_lens = sel_lens;  // the scan runs over each sequence's list
  a.qscale = (float)((double)sm_scale * 1.4426950408889634);  // log2(e)
  a.rotate_q = g.rotate && !(flags & KVQ_Q_PREROTATED);
  a.rotate_out = g.rotate && !(flags & KVQ_OUT_ROTATED);
  a.out = out;
  a.workspace = (float*)workspace;
  a.sel = sel;
  a.sel_stride = max_selected > 0 ? max_selected : 1;
  return hip_status(launch_decode(a, (hipStream_t)stream));
}

int kvq_append_decode_attn_fp4(const kvq_cache_desc* desc, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, int32_t n_tokens, const void* q, int32_t batch,
                               int32_t num_q_heads, int32_t n_q, const int32_t* block_tables,
                               int32_t max_pages_per_seq, const int32_t* context_lens, int32_t max_context_len,
                               float sm_scale, uint32_t flags, float* out, void* workspace,
                               size_t workspace_bytes, kvq_stream_t stream) {
  CacheGeom g;
  const int st = check_desc(desc, &g);
  if (st != KVQ_OK) return st;
  if (n_tokens < 0) return KVQ_ERR_SHAPE;
  if (n_tokens > 0) {
    if (!k_new || !slot_mapping) return KVQ_ERR_NULL;
    if (!g.kv_shared && !v_new) return KVQ_ERR_NULL;
  }
  const AppendArgs ap{(uint8_t*)desc->k_codes, (uint8_t*)desc->k_scales, (uint8_t*)desc->v_codes,
                      (uint8_t*)desc->v_scales, (const uint16_t*)k_new, (const uint16_t*)v_new, slot_mapping,
                      n_tokens};
  return decode_common(KVQ_FMT_FP4_E2M1, desc, q, batch, num_q_heads, n_q, block_tables, max_pages_per_seq,
                       context_lens, max_context_len, sm_scale, flags, out, workspace, workspace_bytes, stream,
                       &ap);
}

int kvq_decode_attn_fp4(const kvq_cache_desc* desc, const void* q, int32_t batch,
                        int32_t num_q_heads, int32_t n_q, const int32_t* block_tables,
                        int32_t max_pages_per_seq, const int32_t* context_lens,
                        int32_t max_context_len, float sm_scale, uint32_t flags, float* out,
                        void* workspace, size_t workspace_bytes, kvq_stream_t stream) {
  return decode_common(KVQ_FMT_FP4_E2M1, desc, q, batch, num_q_heads, n_q, block_tables,
                       max_pages_per_seq, context_lens, max_context_len, sm_scale, flags, out,
                       workspace, workspace_bytes, stream);
}

int kvq_decode_attn_fp4_scratch(const kvq_cache_desc* desc, const void* q, int32_t batch,
                                int32_t num_q_heads, int32_t n_q, const int32_t* block_tables,
                                int32_t max_pages_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float sm_scale, uint32_t flags, float* out,
                                kvq_stream_t stream) {
  return decode_common(KVQ_FMT_FP4_E2M1, desc, q, batch, num_q_heads, n_q, block_tables,
                       max_pages_per_seq, context_lens, max_context_len, sm_scale, flags, out,
                       nullptr, 0, stream, nullptr, /*use_scratch=*/true);
}

int kvq_decode_attn_fp8(const kvq_cache_desc* desc, const void* q, int32_t batch,
                        int32_t num_q_heads, int32_t n_q, const int32_t* block_tables,
                        int32_t max_pages_per_seq, const int32_t* context_lens,
                        int32_t max_context_len, float sm_scale, uint32_t flags, float* out,
                        void* workspace, size_t workspace_bytes, kvq_stream_t stream) {
  return decode_common(KVQ_FMT_FP8_E4M3, desc, q, batch, num_q_heads, n_q, block_tables,
                       max_pages_per_seq, context_lens, max_context_len, sm_scale, flags, out,
                       workspace, workspace_bytes, stream);
}

int kvq_dequant(const kvq_cache_desc* desc, const int32_t* slots, int32_t n, float* k_out,
                float* v_out, kvq_stream_t stream) {
  CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != KVQ_OK) return st;
  st = check_cache_ptrs(desc);
  if (st != KVQ_OK) return st;
  if (n < 0) return KVQ_ERR_SHAPE;
  if (n == 0) return KVQ_OK;
  if (!slots || !k_out) return KVQ_ERR_NULL;
  if (!g.kv_shared && !v_out) return KVQ_ERR_NULL;
  return hip_status(launch_dequant(g, slots, n, k_out, v_out, (hipStream_t)stream));
}

const char* kvq_strerror(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "a size is non-positive or inconsistent";
    case KVQ_ERR_FORMAT: return "cache format does not match the call";
    case KVQ_ERR_UNSUPPORTED: return "no kernel is built for this shape";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_SCRATCH: return "the call needs more than the library's static scratch (KVQ_SCRATCH_BYTES)";
    case KVQ_ERR_HIP:
      snprintf(g_msg, sizeof g_msg, "HIP error: %s", hipGetErrorString(g_last_hip));
      return g_msg;
    default: return "unknown status";
  }
}

int kvq_version(void) { return KVQ_VERSION; }

}  // extern "C"

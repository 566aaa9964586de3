// Internal declarations shared by the translation units of libkvq.
// Host-side launchers take already-validated arguments.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kvq.h"

namespace kvq {

// Geometry of one paged cache, derived from kvq_cache_desc (byte strides).
struct CacheGeom {
  const uint8_t* kc;
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  int fmt;          // KVQ_FMT_*
  int rotate;
  int kv_shared;
  int hkv;
  int d;            // head_dim
  int g;            // head_dim / 32
  int p;            // page_size
  int num_pages;
  int cb;           // code bytes per (token, group): 16 (FP4) or 32 (FP8)
  int64_t c_head;   // code bytes per (page, head)  = g * p * cb
  int64_t c_page;   // code bytes per page          = hkv * c_head
  int64_t s_head;   // scale bytes per (page, head) = g * p
  int64_t s_page;   // scale bytes per page         = hkv * s_head
};

// fp32 rounding of 1/sqrt(d): the single multiply after the butterfly.
float fwht_norm(int d);

// New tokens to append (rotate, quantise, store) before a decode reads the
// cache: kvq_rotate_quantize_append's arguments.
struct AppendArgs {
  uint8_t* kc;
  uint8_t* ks;
  uint8_t* vc;
  uint8_t* vs;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* slots;
  int n_tokens;
};

hipError_t launch_append(const CacheGeom& c, uint8_t* kc, uint8_t* ks,
                         uint8_t* vc, uint8_t* vs, const uint16_t* k_new,
                         const uint16_t* v_new, const int32_t* slots,
                         int n_tokens, hipStream_t stream);

hipError_t launch_dequant(const CacheGeom& c, const int32_t* slots, int n,
                          float* k_out, float* v_out, hipStream_t stream);

struct DecodePlan {
  int kind;              // kDecodeFew, kDecodeMany or kDecodeLatent
  int rows;              // query rows per KV head = n_q * group
  int row_tiles;         // 8-row tiles (few), 128-row blocks (many), 16-row groups (latent)
  int splits;            // context splits per (sequence, KV head)
  int tiles_per_split;   // 16-token tiles per split (even)
  size_t qops_bytes;     // query operands (first part of the workspace)
  size_t workspace;      // bytes
  int block_rows = 0;    // many-row kernel: rows per block (16 per wave)
  int qk_convert = 0;    // FP4 scores through bf16 conversion of the codes (KVQ_QK_CONVERT)
};

// Decide split count and workspace size; returns KVQ_OK or an error code.
int plan_decode(const CacheGeom& c, int batch, int hq, int n_q,
                int max_context_len, uint32_t flags, DecodePlan* plan);

struct DecodeArgs {
  CacheGeom c;
  DecodePlan plan;
  const uint16_t* q;
  int batch, hq, n_q, group;
  const int32_t* block_tables;
  int max_pages;
  const int32_t* context_lens;
  float qscale;      // sm_scale * log2(e)
  int rotate_q;      // rotate the query inside the kernel
  int rotate_out;    // rotate the output back inside the kernel
  float* out;
  float* workspace;
  // shared-prefix decode (kvq_shared.hip); null / zero in a plain call
  const int32_t* tok_start = nullptr;    // suffix level: first token scanned per sequence
  const int32_t* grp_ptr = nullptr;      // prefix level: units are prefix groups
  const int32_t* grp_seq = nullptr;
  const int32_t* shared_lens = nullptr;
  int rows_seq = 0;                      // prefix level: rows per member sequence
  int grp_seqs = 0;                      // prefix level: sequences (partials are stored per sequence)
  int keep_partials = 0;                 // leave split partials, launch no merge
  // selected-position decode (latent kernel): context_lens then holds the
  // list lengths
  const int32_t* sel = nullptr;          // [batch][sel_stride] token positions
  int sel_stride = 0;
  // tokens to append before the scan reads the cache (null: none); the
  // one-wave FP4 path appends inside its query prologue launch
  const AppendArgs* append = nullptr;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// which decode kernel family a plan uses
constexpr int kDecodeFew = 0;     // head_dim 128, up to 16 rows per KV head (FP8: 24) (kvq_decode.hip)
constexpr int kDecodeMany = 1;    // head_dim 128, more rows (kvq_extend.hip)
constexpr int kDecodeLatent = 2;  // head_dim 512 (kvq_decode512.hip)

// many rows per KV head (extend / prefill chunks): kvq_extend.hip
int plan_extend(const CacheGeom& c, int batch, int hq, int n_q, int max_context_len, uint32_t flags,
                DecodePlan* plan);
// the same plan for `units` (sequence or prefix group) x num_kv_heads units of
// `rows` rows each, in blocks of `block_rows` rows (32 or 128; 0: by the row
// count)
int plan_extend_rows(const CacheGeom& c, int units, long long rows, int max_context_len, uint32_t flags,
                     DecodePlan* plan, int block_rows = 0);
hipError_t launch_extend(const DecodeArgs& a, hipStream_t stream);
constexpr int kExtendRowBlock = 128;   // rows per wide many-row block

// shared-prefix decode, head_dim 128 FP4: kvq_shared.hip
struct SharedPlan {
  DecodePlan prefix;     // many-row kernel over the prefix groups
  DecodePlan suffix;     // the row count's decode kernel over each sequence's suffix
  size_t suffix_offset;  // workspace bytes before the suffix level's part
  size_t workspace;      // bytes
};
int plan_shared(const CacheGeom& c, int batch, int hq, int n_q, const kvq_prefix_groups& g, uint32_t flags,
                SharedPlan* plan);
struct SharedArgs {
  DecodeArgs base;  // the call's arguments (plan unused)
  SharedPlan plan;
  kvq_prefix_groups groups;
};
hipError_t launch_shared(const SharedArgs& a, hipStream_t stream);

// head_dim 512 (latent width): planned and launched by kvq_decode512.hip
int plan_decode512(const CacheGeom& c, int batch, int hq, int n_q, int max_context_len, uint32_t flags,
                   DecodePlan* plan);
hipError_t launch_decode512(const DecodeArgs& a, hipStream_t stream);

}  // namespace kvq

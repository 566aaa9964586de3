/*
 * kvq.h -- C interface of libkvq: a paged, Walsh-Hadamard-rotated 4-bit KV
 * cache and decode attention over it, for AMD Instinct MI355X (gfx950).
 *
 * The method is the one the AMD ROCm blog post "UltraQuant on AMD Instinct"
 * describes:
 *   - section "What is UltraQuant?": every key/value head vector is rotated by
 *     a Walsh-Hadamard transform that spreads outlier channels, then stored on
 *     the FP4 (E2M1) grid, each 32-channel group sharing one power-of-two
 *     scale; a group costs 17 bytes against 32 for an 8-bit cache;
 *   - section "Why UltraQuant beats 8-bit KV": scales are UE8M0 bytes, the
 *     decode kernel consumes codes and scales without a lookup table, and
 *     each decode step re-reads the whole cache, so fewer bytes per value is
 *     a faster step (the page reports 2.25x over 8-bit at 32K context);
 *   - section "Throughput vs latency trade-off": MTP verify steps carry
 *     several query positions per sequence over one paged cache.
 * The pages give no interface; the calls below are this library's own.
 *
 * Conventions shared by every call
 *   - Every pointer argument that names tensor data is a DEVICE pointer owned
 *     by the caller.  The library allocates nothing, keeps no state between
 *     calls beyond a cache of device properties (compute units, kernel
 *     occupancy) and the static scratch array of
 *     kvq_decode_attn_fp4_scratch, never synchronises, and enqueues its
 *     kernels on `stream`.
 *   - Arguments are checked on the host before any HIP call; on a failed
 *     check nothing is enqueued and the call returns a negative KVQ_ERR_*.
 *   - Contract violations that can only be seen on the device (a block-table
 *     entry >= num_pages, a slot out of range, context_lens[b] above
 *     max_context_len, non-finite inputs) are undefined behaviour.
 *   - bf16 inputs are IEEE bfloat16 bit patterns (uint16), row-major.
 *
 * Cache layout (per tensor K and V; P = page_size, G = head_dim / 32):
 *   FP4 codes  : uint8 [num_pages][num_kv_heads][G][P][16]
 *                16 bytes hold the 32 E2M1 codes of one (token, group):
 *                channel 32g + 2i in the low nibble of byte i, channel
 *                32g + 2i + 1 in the high nibble; code bit 3 is the sign.
 *   FP8 codes  : uint8 [num_pages][num_kv_heads][G][P][32]  (E4M3FN bytes)
 *   scales     : uint8 [num_pages][num_kv_heads][G][P]
 *                UE8M0: byte e stands for 2^(e - 127).
 *   A token's slot is page * P + offset; its group g lives at
 *   ((page * num_kv_heads + head) * G + g) * P + offset (in units of 16 or 32
 *   code bytes, or of 1 scale byte).  One FP4 (token, group) is 16 + 1 = 17
 *   bytes, as on the page; the FP8 comparator is 32 + 1 = 33 bytes.
 *
 * Quantisation rule (identical for every call that writes the cache)
 *   y = rotate ? fp32 Walsh-Hadamard(x) : x, with radix-2 stages h = 1..d/2
 *   in order (x[j] + x[j+h], x[j] - x[j+h]) and one final multiply by
 *   fp32(1/sqrt(head_dim)); per group amax = max |y|; scale exponent
 *   e_s = max(floor(log2 amax) - emax, -127) (emax = 2 for E2M1, 8 for E4M3;
 *   amax = 0 gives -127); code = round-to-nearest-even of y * 2^-e_s onto the
 *   element grid, saturating at its largest value (6 or 448), sign bit copied
 *   from y.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_VERSION 1

/* ---- status codes ---------------------------------------------------- */
#define KVQ_OK 0
#define KVQ_ERR_NULL (-1)        /* a required pointer is NULL */
#define KVQ_ERR_SHAPE (-2)       /* a size is non-positive or inconsistent */
#define KVQ_ERR_FORMAT (-3)      /* cache format does not match the call */
#define KVQ_ERR_UNSUPPORTED (-4) /* valid, but no kernel is built for it */
#define KVQ_ERR_WORKSPACE (-5)   /* workspace missing or too small */
#define KVQ_ERR_HIP (-6)         /* a HIP runtime call failed */
#define KVQ_ERR_SCRATCH (-7)     /* needs more than KVQ_SCRATCH_BYTES of scratch */

/* ---- cache formats ---------------------------------------------------- */
#define KVQ_FMT_FP4_E2M1 1 /* 16 code bytes + 1 scale byte per 32 values */
#define KVQ_FMT_FP8_E4M3 2 /* 32 code bytes + 1 scale byte per 32 values */

/* ---- decode flags ----------------------------------------------------- */
/* q is already in the rotated basis (the caller folded H into its weights) */
#define KVQ_Q_PREROTATED 0x1u
/* leave `out` in the rotated basis (the caller folds H into what follows) */
#define KVQ_OUT_ROTATED 0x2u
/* FP4 cache: compute the scores by converting the K codes with their scales
 * to bf16 and multiplying against a bf16 hi + lo query on bf16 MFMAs,
 * instead of feeding the codes to the scaled FP4 MFMA against FP6 query
 * terms.  The two routes give the same attention within the acceptance
 * bound; the flag exists to compare them (the native route is the faster,
 * and the default).  Decode calls only; ignored for an FP8 cache. */
#define KVQ_QK_CONVERT 0x4u
/* bits 16..27 force the number of context splits (0: chosen by the library);
 * the result does not depend on it beyond fp32 rounding. */
#define KVQ_SPLITS_SHIFT 16
#define KVQ_SPLITS_MASK 0x0FFF0000u
#define KVQ_SPLITS(n) (((uint32_t)(n) << KVQ_SPLITS_SHIFT) & KVQ_SPLITS_MASK)

/* A hipStream_t, passed as an opaque handle; NULL is the null stream. */
typedef void *kvq_stream_t;

/* Description of one paged cache.  The code and scale arrays are caller-owned
 * device memory of kvq_cache_code_bytes / kvq_cache_scale_bytes bytes each;
 * code arrays must be 16-byte aligned (KVQ_ERR_SHAPE otherwise).
 *   format       KVQ_FMT_FP4_E2M1 or KVQ_FMT_FP8_E4M3
 *   rotate       1: vectors are Walsh-Hadamard rotated before quantisation
 *   kv_shared    1: values are the keys (latent cache); v_* are ignored
 *   head_dim     power of two, 32 <= head_dim <= 1024
 *   page_size    16, 32 or 64 tokens */
typedef struct kvq_cache_desc {
  int32_t format;
  int32_t rotate;
  int32_t kv_shared;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_pages;
  void *k_codes;
  void *k_scales;
  void *v_codes;
  void *v_scales;
} kvq_cache_desc;

/* Bytes of one tensor's code array / scale array for `desc` (0 when the
 * description's sizes are invalid).  Host-only; no HIP call. */
size_t kvq_cache_code_bytes(const kvq_cache_desc *desc);
size_t kvq_cache_scale_bytes(const kvq_cache_desc *desc);

/* Append: rotate (if desc->rotate), quantise and store n_tokens new key and
 * value vectors ("What is UltraQuant?": the rotation as the preparation step
 * before the 4-bit grid).
 *   k_new, v_new   bf16 [n_tokens][num_kv_heads][head_dim], contiguous;
 *                  v_new is ignored (may be NULL) when kv_shared
 *   slot_mapping   int32 [n_tokens]; token i goes to slot slot_mapping[i]
 *                  (page * page_size + offset); a negative slot skips it
 * Writes the codes and scales of those slots only.  Two tokens with the same
 * slot in one call race; across calls the later call wins.
 * Returns KVQ_OK, or KVQ_ERR_NULL / SHAPE / UNSUPPORTED / HIP. */
int kvq_rotate_quantize_append(const kvq_cache_desc *desc, const void *k_new,
                               const void *v_new, const int32_t *slot_mapping,
                               int32_t n_tokens, kvq_stream_t stream);

/* Workspace bytes a decode call with these sizes needs (0 when the sizes are
 * invalid): the rotated, pre-scaled query operands, prepared once per
 * (sequence, KV head), and the partial results of the context splits.  The
 * caller passes at least this much device memory, 16-byte aligned, to the
 * decode call; its contents need no initialisation.  Calls that overlap in
 * time must not share a workspace.  Unless KVQ_SPLITS(n) fixes the split
 * count, the count (and so the size) is planned for the current HIP device:
 * query with the device current that the decode call will run on.  No
 * device work is enqueued. */
size_t kvq_decode_workspace_bytes(const kvq_cache_desc *desc, int32_t batch,
                                  int32_t num_q_heads, int32_t n_q,
                                  int32_t max_context_len, uint32_t flags);

/* Decode attention over an FP4 cache ("Why UltraQuant beats 8-bit KV": the
 * decode step that reads codes and scales natively, no lookup table).
 *   q               bf16 [batch][n_q][num_q_heads][head_dim]
 *   num_q_heads     multiple of num_kv_heads; query head h reads KV head
 *                   h / (num_q_heads / num_kv_heads).  Rows per KV head =
 *                   n_q * num_q_heads / num_kv_heads: up to 65536 at
 *                   head_dim 128 (more than 16 rows run the many-row kernel
 *                   also meant for prefill / extend chunks), up to 64 at
 *                   head_dim 512; other head_dims: KVQ_ERR_UNSUPPORTED
 *   n_q             query positions per sequence (MTP verify: > 1); the last
 *                   n_q cached tokens are the verify tokens and position j
 *                   sees tokens 0 .. context_lens[b] - n_q + j
 *   block_tables    int32 [batch][max_pages_per_seq] physical page ids
 *   context_lens    int32 [batch] (device) tokens in each sequence's cache
 *   max_context_len host-side upper bound of context_lens (sizes the grid),
 *                   at most 2^30; max_pages_per_seq * page_size >= it
 *   sm_scale        softmax scale (usually 1/sqrt(head_dim))
 *   flags           KVQ_Q_PREROTATED, KVQ_OUT_ROTATED, KVQ_SPLITS(n)
 *   out             fp32 [batch][n_q][num_q_heads][head_dim]
 * Rotated caches: unless KVQ_Q_PREROTATED, q is rotated by the same fp32
 * transform; unless KVQ_OUT_ROTATED, the output is rotated back, so `out` is
 * softmax(sm_scale q K^T) V of the dequantised cache in the caller's basis.
 * A position that sees no token gets zeros.
 * Returns KVQ_OK, or KVQ_ERR_NULL / SHAPE / FORMAT (cache is not FP4) /
 * UNSUPPORTED / WORKSPACE / HIP. */
int kvq_decode_attn_fp4(const kvq_cache_desc *desc, const void *q,
                        int32_t batch, int32_t num_q_heads, int32_t n_q,
                        const int32_t *block_tables, int32_t max_pages_per_seq,
                        const int32_t *context_lens, int32_t max_context_len,
                        float sm_scale, uint32_t flags, float *out,
                        void *workspace, size_t workspace_bytes,
                        kvq_stream_t stream);

/* One decode step in one call: kvq_rotate_quantize_append(desc, k_new,
 * v_new, slot_mapping, n_tokens) followed by kvq_decode_attn_fp4(desc, q,
 * ...) on the same stream, with identical results (the cache bytes and the
 * output are the ones the two calls give).  Where the decode runs the
 * one-wave kernel (head_dim 128, at most 16 rows per KV head) the append
 * runs inside its first launch, beside the query prologue, which saves a
 * launch per step; elsewhere it runs first, as its own launch.  Arguments as
 * for the two calls; the appended tokens must belong to the sequences'
 * contexts as context_lens states them.  Returns KVQ_OK, or the errors of
 * either call. */
int kvq_append_decode_attn_fp4(const kvq_cache_desc *desc, const void *k_new,
                               const void *v_new, const int32_t *slot_mapping,
                               int32_t n_tokens, const void *q, int32_t batch,
                               int32_t num_q_heads, int32_t n_q,
                               const int32_t *block_tables,
                               int32_t max_pages_per_seq,
                               const int32_t *context_lens,
                               int32_t max_context_len, float sm_scale,
                               uint32_t flags, float *out, void *workspace,
                               size_t workspace_bytes, kvq_stream_t stream);
/* Bytes of the library's static device scratch array (32 MiB), the most a
 * kvq_decode_attn_fp4_scratch call may need (kvq_decode_workspace_bytes of
 * its sizes). */
#define KVQ_SCRATCH_BYTES ((size_t)32 << 20)

/* kvq_decode_attn_fp4 without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The query operands and split partials
 * go to a file-scope static device array of KVQ_SCRATCH_BYTES bytes that the
 * library holds on every device it runs on until the process ends; the call
 * itself allocates nothing.  Arguments, results and flags are those of
 * kvq_decode_attn_fp4 (the same kernels, the same plan, so the same output);
 * the scratch needs no initialisation.  All calls on one device share that
 * device's array: calls that overlap in time on one device (two streams, two
 * threads) race and give undefined results; calls ordered on one stream do
 * not.  Returns the errors of kvq_decode_attn_fp4, with KVQ_ERR_SCRATCH in
 * place of KVQ_ERR_WORKSPACE when the sizes need more than
 * KVQ_SCRATCH_BYTES. */
int kvq_decode_attn_fp4_scratch(const kvq_cache_desc *desc, const void *q,
                                int32_t batch, int32_t num_q_heads,
                                int32_t n_q, const int32_t *block_tables,
                                int32_t max_pages_per_seq,
                                const int32_t *context_lens,
                                int32_t max_context_len, float sm_scale,
                                uint32_t flags, float *out,
                                kvq_stream_t stream);

/* The same decode over an FP8 (E4M3, per-32 UE8M0 scale) cache: the 8-bit
 * comparator of "UltraQuant vs 8-bit KV".  Identical arguments; returns
 * KVQ_ERR_FORMAT unless desc->format == KVQ_FMT_FP8_E4M3, and
 * KVQ_ERR_UNSUPPORTED for head_dim != 128 or more than 24 rows per KV head. */
int kvq_decode_attn_fp8(const kvq_cache_desc *desc, const void *q,
                        int32_t batch, int32_t num_q_heads, int32_t n_q,
                        const int32_t *block_tables, int32_t max_pages_per_seq,
                        const int32_t *context_lens, int32_t max_context_len,
                        float sm_scale, uint32_t flags, float *out,
                        void *workspace, size_t workspace_bytes,
                        kvq_stream_t stream);

/* Prefix groups of a shared-prefix decode (kvq_decode_attn_fp4_shared).
 * Agent traffic re-sends long prefixes, so many sequences of a batch start
 * with the same cached pages ("Agentic serving: workload and setup": long
 * shared prefixes, a high prefix-cache hit rate).  A group names such a
 * prefix and the sequences that start with it:
 *   num_groups       G >= 1
 *   max_group_size   host-side bound: indptr[g + 1] - indptr[g] <= it for
 *                    every g (sizes the grid)
 *   indptr           int32 [G + 1] (device), non-decreasing, indptr[0] = 0
 *   members          int32 [indptr[G]] (device): group g's sequences are
 *                    members[indptr[g]] .. members[indptr[g + 1] - 1];
 *                    listing them by decreasing shared_lens is fastest
 *   prefix_tables    int32 [G][max_prefix_pages] (device): the physical pages
 *                    of each group's prefix, in token order
 *   max_prefix_pages row length of prefix_tables, >= 1, with
 *                    max_prefix_pages * page_size at most 2^30
 *   shared_lens      int32 [batch] (device): tokens 0 .. shared_lens[b] - 1
 *                    of sequence b are tokens 0 .. shared_lens[b] - 1 of its
 *                    group's prefix; a multiple of 16 (whole pages of any
 *                    page size are), at most context_lens[b] and at most
 *                    max_prefix_pages * page_size.  A sequence with
 *                    shared_lens[b] > 0 is a member of exactly one group; one
 *                    with 0 may be a member of none
 *   max_suffix_len   host-side bound: context_lens[b] - shared_lens[b] <=
 *                    it for every b (sizes the grid), >= 0
 * Violations that only the device can see are undefined behaviour, as for
 * the other contracts above. */
typedef struct kvq_prefix_groups {
  int32_t num_groups;
  int32_t max_group_size;
  const int32_t *indptr;
  const int32_t *members;
  const int32_t *prefix_tables;
  int32_t max_prefix_pages;
  const int32_t *shared_lens;
  int32_t max_suffix_len;
} kvq_prefix_groups;
/* Workspace bytes of a shared-prefix decode with these sizes (0 when they
 * are invalid or unsupported); the same rules as kvq_decode_workspace_bytes.
 * Only the host-side fields of `groups` are read. */
size_t kvq_decode_shared_workspace_bytes(const kvq_cache_desc *desc,
                                         int32_t batch, int32_t num_q_heads,
                                         int32_t n_q,
                                         const kvq_prefix_groups *groups,
                                         uint32_t flags);
/* Shared-prefix (cascade) decode over an FP4 cache, head_dim 128: the same
 * result as kvq_decode_attn_fp4 (up to fp32 rounding) when block_tables[b]
 * starts with the pages of its group's prefix, but each group's prefix pages
 * are read once for the query rows of all its members, and each sequence's
 * own pages (tokens shared_lens[b] .. context_lens[b] - 1) once for its rows.
 *   block_tables   int32 [batch][max_pages_per_seq]; row b covers the
 *                  ceil(context_lens[b] / page_size) pages of sequence b,
 *                  indexed by token position (entries of tokens below
 *                  shared_lens[b] are not read)
 *   max_context_len host-side upper bound of context_lens, at most 2^30,
 *                  with max_pages_per_seq * page_size >= max_context_len
 *                  and max_suffix_len <= max_context_len
 *   groups         see kvq_prefix_groups
 *   other arguments as for kvq_decode_attn_fp4; rows per KV head (n_q *
 *   num_q_heads / num_kv_heads) and rows per group (that times
 *   max_group_size) are at most 65536; KVQ_SPLITS(n) forces the split count
 *   of both levels (at most 32 each)
 * Returns KVQ_OK, or KVQ_ERR_NULL / SHAPE / FORMAT / UNSUPPORTED (head_dim
 * other than 128) / WORKSPACE / HIP. */
int kvq_decode_attn_fp4_shared(const kvq_cache_desc *desc, const void *q,
                               int32_t batch, int32_t num_q_heads, int32_t n_q,
                               const int32_t *block_tables,
                               int32_t max_pages_per_seq,
                               const int32_t *context_lens,
                               int32_t max_context_len,
                               const kvq_prefix_groups *groups, float sm_scale,
                               uint32_t flags, float *out, void *workspace,
                               size_t workspace_bytes, kvq_stream_t stream);
/* Decode attention over selected history positions of a latent-width FP4
 * cache.  The page "GLM-5.3-Flash in MXFP4: A Lighter, Faster Checkpoint for
 * AMD MI355X", section "How the serving path works" ("Sparse attention and
 * K-pool selection"), has a separate index choose the history each token
 * attends to (pooled four-token groups plus a few recent tokens, 2,051
 * positions at most); building that index is the caller's.  This call
 * attends over the chosen positions of the 512-wide latent cache only.
 *   q             bf16 [batch][1][num_q_heads][head_dim]: one query position
 *                 per sequence (its heads share the selection)
 *   block_tables  int32 [batch][max_pages_per_seq]
 *   sel           int32 [batch][max_selected] (device): sel[b][j] for
 *                 j < sel_lens[b] are token positions of sequence b, each a
 *                 written slot of its pages; any order; a position listed
 *                 twice counts twice
 *   sel_lens      int32 [batch] (device), 0 <= sel_lens[b] <= max_selected
 *   max_selected  host-side row length of sel (sizes the grid), 0 to 2^30
 *   out           fp32 [batch][1][num_q_heads][head_dim]; a sequence with no
 *                 selected position gets zeros
 *   other arguments as for kvq_decode_attn_fp4; rows per KV head
 *   (num_q_heads / num_kv_heads) at most 64
 * Returns KVQ_OK, or KVQ_ERR_NULL / SHAPE / FORMAT (cache is not FP4) /
 * UNSUPPORTED (head_dim other than 512, more than 64 rows) / WORKSPACE / HIP. */
int kvq_decode_attn_fp4_selected(const kvq_cache_desc *desc, const void *q,
                                 int32_t batch, int32_t num_q_heads,
                                 const int32_t *block_tables,
                                 int32_t max_pages_per_seq,
                                 const int32_t *sel, const int32_t *sel_lens,
                                 int32_t max_selected, float sm_scale,
                                 uint32_t flags, float *out, void *workspace,
                                 size_t workspace_bytes, kvq_stream_t stream);
/* Workspace bytes of a selected-position decode with these sizes (0 when
 * they are invalid or unsupported); the rules of kvq_decode_workspace_bytes. */
size_t kvq_decode_selected_workspace_bytes(const kvq_cache_desc *desc,
                                           int32_t batch, int32_t num_q_heads,
                                           int32_t max_selected,
                                           uint32_t flags);
/* Dequantise n slots (for tests and export): fp32 [n][num_kv_heads][head_dim]
 * of code value * 2^(scale - 127), in the stored (rotated) basis.  v_out is
 * ignored (may be NULL) when kv_shared.  Slots must be in range.
 * Returns KVQ_OK, or KVQ_ERR_NULL / SHAPE / UNSUPPORTED / HIP. */
int kvq_dequant(const kvq_cache_desc *desc, const int32_t *slots, int32_t n,
                float *k_out, float *v_out, kvq_stream_t stream);

/* Text for a status code; for KVQ_ERR_HIP it names the last HIP error seen
 * by this thread.  The string is static or thread-local; do not free it. */
const char *kvq_strerror(int status);

/* KVQ_VERSION of the built library. */
int kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */

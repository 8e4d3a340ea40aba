/*
 * paged_decode.h - C ABI of the MI355X (gfx950) paged split-KV decode library.
 *
 * Two attention operations over a paged KV cache addressed through a
 * per-request block table, a static split-count helper and the split merge:
 *
 *   paged_decode_gqa   one query token per request, grouped-query heads,
 *                      optional per-head sinks and a sliding window;
 *   paged_verify_gqa   the same with qlen causal verify tokens per request
 *                      (paged_verify_gqa_varlen: a query length per request);
 *   paged_kv_append    writes the newest tokens' K/V into the paged cache
 *                      (paged_verify_gqa_append: fused with the GQA call);
 *   paged_verify_mla   qlen causal "verify" tokens per request over one shared
 *                      latent cache, V read as K[..., :Lv], bf16 or FP8 cache;
 *   *_partials         the split partials of a call, without the merge;
 *   num_kv_splits_cap  static split cap from static sizes (graph-capture safe;
 *                      pd_gqa_split_cap / pd_mla_split_cap / pd_split_rule);
 *   merge_splits       merges fp32 split partials into O and a natural-log LSE.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless marked [host].  The caller allocates
 *   and owns every buffer (inputs, outputs, workspace); the library keeps no
 *   per-call state and never allocates, frees or synchronises.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *   null stream).  The launch shape depends only on the integer arguments,
 *   never on device data, so a call can be captured in a HIP graph.
 * - Strides are in ELEMENTS of the tensor they describe; the innermost
 *   dimension is always contiguous (stride 1).
 * - Every argument check happens on the host before any HIP call; a failed
 *   check returns a negative pd_status and enqueues nothing.  Device data
 *   (lengths, block-table entries) is never read on the host.  On the device,
 *   a length below 0 counts as 0, a length beyond the block-table row's
 *   capacity (max_blocks * page_size) is clamped to it, and an attended
 *   block-table entry outside [0, num_pages) is never dereferenced: the
 *   affected (request, head) outputs are written as NaN instead.
 * - sm_scale must be finite and > 0 (the GQA kernel keeps its softmax
 *   reference, a running maximum, in unscaled scores, which orders them only
 *   for a positive scale); any other value returns PD_ERR_INVALID.
 * - bf16 values are IEEE binary32 truncated to their upper 16 bits (round to
 *   nearest even on output); FP8 is OCP E4M3FN.
 *
 * Numerics (module docstring of "vllm.models.flint.ops.decode_attention"):
 * scores are bf16 x bf16 products accumulated in fp32; softmax runs in fp32 as
 * exp2(s * c - m * c) with c = sm_scale * log2(e) and a reference m of the
 * unscaled scores (GQA: the running max, moved only when a score passes it
 * by more than 8 / c, so p <= 2^8; MLA: a row's first tile max);
 * probabilities are rounded to bf16 for the P.V product
 * (fp32 accumulation); split partials stay fp32.
 */
#ifndef PAGED_DECODE_H_
#define PAGED_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define PD_API __attribute__((visibility("default")))
#else
#define PD_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  0 is success; every error is negative. */
typedef enum {
  PD_OK = 0,
  PD_ERR_INVALID = -1,     /* null pointer, negative size or inconsistent sizes */
  PD_ERR_ALIGN = -2,       /* pointer not 16-byte aligned / stride not 16-byte multiple */
  PD_ERR_UNSUPPORTED = -3, /* a size this build has no kernel for */
  PD_ERR_WORKSPACE = -4,   /* workspace missing or smaller than pd_workspace_bytes() */
  PD_ERR_HIP = -5          /* a HIP runtime call failed (launch, device query) */
} pd_status;

/* Cache element type of the MLA latent cache. */
typedef enum { PD_KV_BF16 = 0, PD_KV_FP8_E4M3FN = 1 } pd_kv_dtype;

/* [host] Static text for a pd_status value (never NULL). */
PD_API const char* pd_status_string(int status);

/*
 * num_kv_splits_cap - [host] the static split cap this library's kernels
 * are tuned for, from static sizes only (graph-capture safe).
 *
 * head_dim_k == 576 with num_kv_heads == 1 selects the MLA verify kernel
 * (a program is one (request, 128-row block) pair); head_dim_k == 128 the
 * GQA kernel (a program is one (request, kv head) pair, whatever qlen: the
 * verify tokens of a kv head share its key stream).  The cap is
 * pd_split_rule with that kernel's policy:
 *   GQA: block_h 1, occupancy 1, min_work_per_split 256, max_splits 64,
 *        balance_chunk 1024;
 *   MLA: block_h 128, occupancy 1, min_work_per_split 128, max_splits 16,
 *        balance_chunk 2048;
 * num_cus = the compute units of `device` (< 0: the current device).
 * max_splits > 0 lowers the policy's max_splits to it; <= 0 keeps it.
 * For a GQA call with a sliding window use pd_gqa_split_cap, which bounds
 * the keys by the window.  Returns the cap (>= 1), PD_ERR_INVALID for
 * negative sizes or num_q_heads % num_kv_heads != 0, PD_ERR_UNSUPPORTED for
 * another head_dim_k, PD_ERR_HIP if the device query fails.
 */
PD_API int32_t num_kv_splits_cap(int32_t max_seq_len, int32_t batch, int32_t qlen,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_k,
                          int32_t max_splits, int32_t device);

/*
 * [host] The GQA policy of num_kv_splits_cap with a window: the keys of a
 * (request, kv head) are min(max_seq_len, window) for window > 0, else
 * max_seq_len.  The cap paged_decode_gqa / paged_verify_gqa(_varlen) are
 * tuned for.  num_cus <= 0 queries the current device.  Same return values.
 */
PD_API int32_t pd_gqa_split_cap(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                int32_t window, int32_t num_cus);

/*
 * [host] The MLA policy of num_kv_splits_cap: the cap paged_verify_mla is
 * tuned for.  num_cus <= 0 queries the current device.  Same return values.
 */
PD_API int32_t pd_mla_split_cap(int32_t batch, int32_t qlen, int32_t num_heads,
                                int32_t max_seq_len, int32_t num_cus);

/*
 * pd_split_rule - [host] the split rule itself, with every knob exposed.
 *
 * Restates "vllm.v1.attention.ops.triton_decode_attention",
 * verify_num_kv_splits: a program is one (request, row block) pair, with
 * ceil(qlen * num_heads / block_h) row blocks per request; the ideal split
 * count is ceil(max_seq_len / min_work_per_split); with
 * slots = floor(occupancy * num_cus) resident programs, if one split of every
 * request fits in one dispatch round the cap fills that round
 * (slots / programs), otherwise it is the n <= min(ideal, max_splits) that
 * minimises ceil(n * programs / slots) / n, preferring the smallest n within
 * 5% of the best; the result is clamped to [1, min(ideal, 2 * num_cus)].
 *
 * Skew extension (balance_chunk > 0): that rule assumes every request has
 * max_seq_len keys.  With skewed lengths one long request would leave a few
 * programs running long after the rest, so the cap is raised to at least
 * min(max_splits, ideal, ceil(max_seq_len / balance_chunk)), which bounds the
 * keys any one split of the longest request can hold.  balance_chunk <= 0
 * gives the unmodified rule.
 *
 * num_cus <= 0 queries the current device.  Reads no device data.  Returns
 * the cap (>= 1), or a negative pd_status for negative sizes, block_h < 1,
 * occupancy <= 0, max_splits < 1, or a failed device query.
 */
PD_API int32_t pd_split_rule(int32_t max_seq_len, int32_t batch, int32_t qlen,
                             int32_t num_heads, int32_t block_h, int32_t num_cus,
                             float occupancy, int32_t min_work_per_split,
                             int32_t max_splits, int32_t balance_chunk);

/*
 * [host] Bytes of fp32 workspace a call with `num_splits` > 1 needs:
 * rows * num_heads * num_splits * (head_dim_v + 1) * 4, laid out
 * [rows][num_heads][num_splits][head_dim_v + 1] ("vllm.v1.attention.ops.
 * triton_decode_attention", decode_attention_fwd_verify, parameter
 * attn_logits).  Slot [..., s, 0:Dv] holds split s's normalised output
 * O_s = sum_j e^{x_j} V_j / sum_j e^{x_j}; slot [..., s, Dv] holds its
 * natural-log lse_s (-inf when the split saw no key, O_s then unspecified).
 * Returns 0 when num_splits <= 1 (no workspace is used).
 */
PD_API size_t pd_workspace_bytes(int32_t rows, int32_t num_heads, int32_t num_splits,
                          int32_t head_dim_v);

/*
 * paged_decode_gqa - paged GQA decode, one query token per request.
 *
 * Defined by "vllm.models.flint.ops.decode_attention", flint_decode_attention
 * and its kernel: query head h of request b attends the keys at positions
 * [lo, L) of its kv head h / (Hq / Hkv), with L = seq_lens[b] (the KV length
 * including the current token) and lo = max(L - window, 0) for window > 0
 * (the last `window` positions), else lo = 0.  Position j is slot j % P of
 * physical page block_table[b][j / P] ("Atención paginada", decode path:
 * the block table maps a request's logical blocks to cache blocks; -1 marks
 * unallocated blocks, which are never read).
 *
 *   O[b,h]   = sum_j e^{x_j} V_j / (sum_j e^{x_j} + e^{sinks[h]}),
 *   x_j      = sm_scale * q[b,h] . K_j,
 *   LSE[b,h] = ln sum_j e^{x_j}           (sink excluded; -inf with no key),
 *   O = 0 for a request with no attended key (e.g. seq_lens[b] == 0).
 *
 * q            [B, Hq, D] bf16, strides (q_stride_b, q_stride_h, 1).
 * kv           HND cache [num_pages, Hkv, P, 2D] bf16: K in [..., 0:D], V in
 *              [..., D:2D], token stride 2D, strides (kv_stride_page,
 *              kv_stride_head, 2D, 1); 8 KB per page per kv head at D=128, P=16.
 * block_table  [B, max_blocks] int32, row stride bt_stride_b.
 * seq_lens     [B] int32.
 * sinks        [Hq] fp32 sink logits, or NULL for none.
 * window       <= 0 for full attention.
 * num_kv_splits static split cap S >= 1 (see num_kv_splits_cap); each request
 *              uses only as many splits as its own length needs.  S == 1
 *              writes O / LSE directly; S > 1 writes fp32 partials to
 *              `workspace` (>= pd_workspace_bytes(B, Hq, S, D) bytes) and
 *              merges them with the same kernel as merge_splits.
 * out          [B, Hq, D] bf16, strides (o_stride_b, o_stride_h, 1).
 * lse          [B, Hq] fp32 with row stride lse_stride_b, or NULL.
 *
 * Supported: D = 128; any page size P from 1 to 65536 tokens (the verify
 * module of "vllm.v1.attention.ops.triton_decode_attention" takes any page
 * size of at least one token; P < 1 gives PD_ERR_INVALID, P > 65536
 * PD_ERR_UNSUPPORTED); Hq = G * Hkv with 1 <= G <= 64.
 * q, kv, out, workspace 16-byte aligned; q/kv/out strides multiples of 8.
 * A workspace must not be shared by calls in flight on different streams.
 */
PD_API int paged_decode_gqa(const void* q, int64_t q_stride_b, int64_t q_stride_h,
                     const void* kv, int64_t kv_stride_page, int64_t kv_stride_head,
                     int32_t num_pages,
                     const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
                     const int32_t* seq_lens, const float* sinks, int32_t window,
                     float sm_scale, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t num_kv_splits, float* workspace, size_t workspace_bytes,
                     void* out, int64_t o_stride_b, int64_t o_stride_h,
                     float* lse, int64_t lse_stride_b, void* stream);

/*
 * paged_verify_gqa - paged GQA causal verify, qlen query tokens per request.
 *
 * The verify form of paged_decode_gqa.  Rows and limits follow
 * "vllm.v1.attention.ops.triton_decode_attention",
 * decode_attention_fwd_verify: the qlen verify tokens of request b are rows
 * b*qlen + t (t = 0..qlen-1) of q, out and lse, and row t attends key
 * positions [lo_t, hi_t) with
 *   hi_t = max(min(L - qlen + 1 + t, L_real), 0),  L = seq_lens[b],
 *   L_real = real_seq_lens[b] (or L when real_seq_lens is NULL),
 *   lo_t = max(hi_t - window, 0) for window > 0 (its own last `window`
 *   keys), else 0.
 * The cache, the block table, the head grouping, the sinks and O / LSE are
 * as for paged_decode_gqa (per row instead of per request); the block table
 * has one row per request shared by its qlen rows.  A row with no key gets
 * O = 0 and LSE = -inf.  qlen = 1 with real_seq_lens NULL is
 * paged_decode_gqa.
 *
 * q            [B*qlen, Hq, D] bf16, strides (q_stride_row, q_stride_h, 1).
 * kv_dtype     PD_KV_BF16, or PD_KV_FP8_E4M3FN: the cache holds E4M3FN codes
 *              (1 byte each) and K_j = code * k_scale, V_j = code * v_scale,
 *              as the scalar k_scale dequantises an FP8 cache in
 *              decode_attention_fwd_verify; K and V are separate tensors, so
 *              each has its own scale.
 * k_scale,     device fp32: one value (scale_per_head = 0) or [Hkv]
 * v_scale      (scale_per_head = 1); NULL means 1.  Ignored for bf16.  Each
 *              scale must be finite and > 0 (the softmax reference, a
 *              running maximum, is kept in unscaled scores).
 * real_seq_lens [B] int32 or NULL.
 * out          [B*qlen, Hq, D] bf16, strides (o_stride_row, o_stride_h, 1).
 * lse          [B*qlen, Hq] fp32 with row stride lse_stride_row, or NULL.
 * workspace    >= pd_workspace_bytes(B*qlen, Hq, S, D) bytes when S > 1.
 * Other arguments as for paged_decode_gqa.
 *
 * Supported: as paged_decode_gqa, any qlen >= 1.  Up to 64 (token, head)
 * pairs, qlen * G <= 64, the verify tokens of a kv head's query heads share
 * the score tiles (groups of 16 columns), so a cache tile is read once for
 * all of them.  Longer verify rows run as ceil(qlen * G / 64) launches of
 * consecutive tokens (slice sizes differ by at most one), each reading the
 * cache again; the split merge, if any, follows the last.  Also
 * ((qlen-1)*q_stride_row + (G-1)*q_stride_h + D) * 2 < 2^31.  FP8 cache
 * strides must be multiples of 16.
 */
PD_API int paged_verify_gqa(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                     const void* kv, int32_t kv_dtype, const float* k_scale,
                     const float* v_scale, int32_t scale_per_head,
                     int64_t kv_stride_page, int64_t kv_stride_head,
                     int32_t num_pages, const int32_t* block_table, int64_t bt_stride_b,
                     int32_t max_blocks, const int32_t* seq_lens,
                     const int32_t* real_seq_lens, int32_t qlen, const float* sinks,
                     int32_t window, float sm_scale, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t num_kv_splits, float* workspace, size_t workspace_bytes,
                     void* out, int64_t o_stride_row, int64_t o_stride_h,
                     float* lse, int64_t lse_stride_row, void* stream);

/*
 * paged_verify_gqa_append - paged_kv_append of the newest qlen tokens and
 * paged_verify_gqa over the cache that holds them, in one launch.
 *
 * "vllm.models.flint.ops.decode_attention" (module description) notes that
 * of all the pages a decode call reads, only the one holding the current
 * token depends on the kernel before it, the one writing that token's K/V;
 * "Atención paginada" (Ruta de decodificación) has the decode kernel update
 * the paged cache in place through the block table.  Here the attention
 * kernel does both: the rows of the newest qlen tokens of request b
 * (positions seq_lens[b] - qlen + t, t = 0..qlen-1) are read from k_new /
 * v_new, never from the cache, and the same launch writes them into the
 * cache.  Results (out, lse and the cache bytes) are bit for bit those of
 * paged_kv_append(k_new, v_new) followed by paged_verify_gqa on the same
 * stream; qlen = 1 with real_seq_lens NULL is decode.
 *
 * k_new, v_new [B*qlen, Hkv, D] in the cache's element type (bf16, or FP8
 *              E4M3FN codes already scaled like the cache), strides
 *              (*_stride_row, *_stride_h, 1) in elements (multiples of 16
 *              bytes, at most INT32_MAX, else PD_ERR_ALIGN / PD_ERR_UNSUPPORTED),
 *              16-byte aligned; row b*qlen + t is token t of request b.
 * kv           written: the new tokens' rows, as paged_kv_append writes
 *              them (a token at a negative position, past the block-table
 *              row or behind an entry outside [0, num_pages) is skipped).
 * Other arguments, supported sizes and errors as for paged_verify_gqa.
 * The new tokens' pages must not be read or written by another call in
 * flight, nor shared with another request.
 */
PD_API int paged_verify_gqa_append(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                     void* kv, int32_t kv_dtype, const float* k_scale,
                     const float* v_scale, int32_t scale_per_head,
                     int64_t kv_stride_page, int64_t kv_stride_head,
                     int32_t num_pages, const int32_t* block_table, int64_t bt_stride_b,
                     int32_t max_blocks, const int32_t* seq_lens,
                     const int32_t* real_seq_lens, int32_t qlen,
                     const void* k_new, int64_t k_new_stride_row, int64_t k_new_stride_h,
                     const void* v_new, int64_t v_new_stride_row, int64_t v_new_stride_h,
                     const float* sinks, int32_t window, float sm_scale, int32_t batch,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t num_kv_splits, float* workspace,
                     size_t workspace_bytes, void* out, int64_t o_stride_row,
                     int64_t o_stride_h, float* lse, int64_t lse_stride_row, void* stream);

/*
 * paged_verify_gqa_noalloc - paged_verify_gqa for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  No workspace argument.
 *
 * Same operation, arguments (minus workspace / workspace_bytes), kernels and
 * results as paged_verify_gqa (bit for bit).  With num_kv_splits > 1 the
 * split partials go to a scratch array the library holds in device memory,
 * one per GPU it runs on, 64 MiB each (67108864 bytes), kept until the
 * process ends.  A call whose partials would not fit,
 * B*qlen * Hq * S * (D + 1) * 4 > 67108864, returns PD_ERR_WORKSPACE and
 * enqueues nothing (use a smaller num_kv_splits or paged_verify_gqa).  The
 * call allocates nothing; it never needs the scratch cleared (every slot the
 * merge reads is written by the same call).  Every call on one GPU shares
 * that GPU's array: calls in flight at the same time on different streams of
 * one GPU race and give wrong results; calls on one stream are safe.  The
 * first call on a device looks up the array's device address (a HIP call,
 * made after every argument check); it fails with PD_ERR_HIP if that lookup
 * does.
 */
PD_API int paged_verify_gqa_noalloc(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                     const void* kv, int32_t kv_dtype, const float* k_scale,
                     const float* v_scale, int32_t scale_per_head,
                     int64_t kv_stride_page, int64_t kv_stride_head,
                     int32_t num_pages, const int32_t* block_table, int64_t bt_stride_b,
                     int32_t max_blocks, const int32_t* seq_lens,
                     const int32_t* real_seq_lens, int32_t qlen, const float* sinks,
                     int32_t window, float sm_scale, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t num_kv_splits, void* out, int64_t o_stride_row,
                     int64_t o_stride_h, float* lse, int64_t lse_stride_row, void* stream);

/*
 * paged_verify_gqa_varlen - paged GQA causal verify with a query length per
 * request.
 *
 * Defined by "Atención paginada", section Ruta Varlen (cumulative query
 * lengths map each query token to its sequence; a sequence may have none)
 * with the verify rule of paged_verify_gqa applied per request: request b
 * has qlen_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] query tokens in rows
 * cu_seqlens_q[b] + t, and row t attends the keys below
 * hi = max(min(L - qlen_b + 1 + t, L_real), 0), the last `window` of them.
 *
 * cu_seqlens_q [B+1] int32 on the device: cu[0] = 0, non-decreasing,
 *              cu[B] = total_rows.
 * max_qlen     host int >= every qlen_b; max_qlen * (Hq / Hkv) <= 64 (the
 *              score tiles hold a kv head's rows).  A request with more
 *              query rows than max_qlen breaks this contract: all its rows
 *              get NaN O and LSE (partials: NaN in every split slot), as
 *              for an invalid block-table entry.
 * total_rows   host int: rows of q, out and lse; 0 is a no-op.
 * q, out, lse  [total_rows, Hq, D] / [total_rows, Hq]; workspace
 *              >= pd_workspace_bytes(total_rows, Hq, S, D) bytes when S > 1.
 * Other arguments as for paged_verify_gqa.  cu_seqlens_q is read on the
 * device only, so the call stays graph-capture safe.  Returns
 * PD_ERR_INVALID for a NULL cu_seqlens_q (B > 0) or total_rows < 0.
 */
PD_API int paged_verify_gqa_varlen(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                     const void* kv, int32_t kv_dtype, const float* k_scale,
                     const float* v_scale, int32_t scale_per_head,
                     int64_t kv_stride_page, int64_t kv_stride_head,
                     int32_t num_pages, const int32_t* block_table, int64_t bt_stride_b,
                     int32_t max_blocks, const int32_t* seq_lens,
                     const int32_t* real_seq_lens, const int32_t* cu_seqlens_q,
                     int32_t max_qlen, int32_t total_rows, const float* sinks,
                     int32_t window, float sm_scale, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t num_kv_splits, float* workspace, size_t workspace_bytes,
                     void* out, int64_t o_stride_row, int64_t o_stride_h,
                     float* lse, int64_t lse_stride_row, void* stream);

/*
 * paged_decode_gqa_partials - the split partials of paged_decode_gqa only.
 *
 * Same arguments and key ranges as paged_decode_gqa (no sinks, no outputs):
 * writes every (request, query head, split) slot of `workspace`, laid out as
 * in pd_workspace_bytes(B, Hq, max(S, 2), D) but with S slots per head, for
 * S = num_kv_splits >= 1, and launches no merge.  A split slot a request does
 * not use gets lse = -inf.  merge_splits over that workspace (with the sinks)
 * gives exactly paged_decode_gqa's result.  This is the per-shard half of
 * split-KV ("vllm.models.flint.ops.decode_attention", module docstring:
 * per-split fp32 partials merged afterwards): a caller that holds a
 * request's keys in several places (another stream, another device) merges
 * the partials once they are gathered.  Workspace bytes >=
 * B * Hq * S * (D + 1) * 4.
 */
PD_API int paged_decode_gqa_partials(const void* q, int64_t q_stride_b, int64_t q_stride_h,
                              const void* kv, int64_t kv_stride_page, int64_t kv_stride_head,
                              int32_t num_pages, const int32_t* block_table,
                              int64_t bt_stride_b, int32_t max_blocks, const int32_t* seq_lens,
                              int32_t window, float sm_scale, int32_t batch,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t num_kv_splits, float* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * paged_verify_gqa_partials - the split partials of paged_verify_gqa (or,
 * with cu_seqlens_q, of paged_verify_gqa_varlen) only.
 *
 * Same key ranges, scales and argument meanings as those two calls, with no
 * sinks and no outputs.  cu_seqlens_q NULL: rows are b*qlen + t and
 * total_rows is ignored; cu_seqlens_q non-NULL: qlen is max_qlen and the
 * rows are the varlen ones (total_rows of them; total_rows = 0 with B > 0
 * returns PD_OK at once).  Writes every (row, query head, split) slot of
 * `workspace` ([rows, Hq, S, D + 1] fp32, S = num_kv_splits >= 1; for an
 * FP8 cache O is already multiplied by v_scale) and launches no merge; a
 * slot a row does not use gets lse = -inf.
 * merge_splits over that workspace, with the sinks, gives exactly the full
 * call's result.  The per-shard half of split-KV for verify, as
 * paged_decode_gqa_partials is for decode.  Workspace bytes >=
 * rows * Hq * S * (D + 1) * 4.
 */
PD_API int paged_verify_gqa_partials(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                              const void* kv, int32_t kv_dtype, const float* k_scale,
                              const float* v_scale, int32_t scale_per_head,
                              int64_t kv_stride_page, int64_t kv_stride_head, int32_t num_pages,
                              const int32_t* block_table, int64_t bt_stride_b,
                              int32_t max_blocks, const int32_t* seq_lens,
                              const int32_t* real_seq_lens, const int32_t* cu_seqlens_q,
                              int32_t qlen, int32_t total_rows, int32_t window, float sm_scale,
                              int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t num_kv_splits,
                              float* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_append - write the qlen newest tokens of every request into the
 * paged cache, through the block table (the cache write before a decode or
 * verify call).
 *
 * Defined by "Atención paginada", section "Ruta de decodificación" (the
 * decode kernel updates the paged cache in place through the block table:
 * position j of request b is slot j % P of page block_table[b][j / P]), with
 * the length convention of "vllm.models.flint.ops.decode_attention"
 * (seq_lens counts the current token): token t of request b, row b*qlen + t
 * of the sources, goes to position seq_lens[b] - qlen + t.  A byte copy,
 * bit-exact for any element type.
 *
 * src0         [B*qlen, H, src0_elems], strides (src0_stride_tok,
 *              src0_stride_h, 1): copied to elements [0, src0_elems) of the
 *              token's cache row (GQA: K; MLA: the latent row).
 * src1         [B*qlen, H, src1_elems] or NULL (then src1_elems = 0): copied
 *              to elements [src0_elems, src0_elems + src1_elems) (GQA: V).
 * elem_bytes   1 (FP8 codes) or 2 (bf16); every stride and element count is
 *              in these elements.
 * cache        page p, head h, slot s at p*cache_stride_page +
 *              h*cache_stride_head + s*cache_stride_tok: the GQA HND cache
 *              [num_pages, Hkv, P, 2D] or the MLA latent cache
 *              [num_pages, P, 1, Lk] (H = 1).
 * block_table  [B, max_blocks] int32; seq_lens [B] int32 (after the append).
 *
 * A token at a negative position (seq_lens[b] < qlen), past the block-table
 * row, or behind an entry outside [0, num_pages) is not written: nothing is
 * ever written outside the cache.  Pointers, strides and row sizes must be
 * 16-byte multiples (PD_ERR_ALIGN), src0_elems + src1_elems <=
 * cache_stride_tok.  Two appends in flight must not target the same slots.
 */
PD_API int paged_kv_append(const void* src0, int64_t src0_stride_tok, int64_t src0_stride_h,
                    int32_t src0_elems, const void* src1, int64_t src1_stride_tok,
                    int64_t src1_stride_h, int32_t src1_elems, int32_t elem_bytes,
                    void* cache, int64_t cache_stride_page, int64_t cache_stride_head,
                    int64_t cache_stride_tok, int32_t num_pages, const int32_t* block_table,
                    int64_t bt_stride_b, int32_t max_blocks, const int32_t* seq_lens,
                    int32_t qlen, int32_t batch, int32_t num_heads, int32_t page_size,
                    void* stream);

/*
 * paged_verify_mla - causal MLA verify over a per-request block table.
 *
 * Defined by "vllm.v1.attention.ops.triton_decode_attention",
 * decode_attention_fwd_verify: the qlen verify rows of request b are rows
 * b*qlen + t (t = 0..qlen-1) of q; row t attends key positions [0, hi) with
 *   hi = max(min(L - qlen + 1 + t, L_real), 0),  L = seq_lens[b],
 *   L_real = real_seq_lens[b] (or L when real_seq_lens is NULL);
 * K_j is latent row j (all Lk dims) and V_j = K_j[0:Lv]; the block table has
 * one row per request shared by its qlen rows.  O and LSE as for GQA without
 * sinks; rows with hi = 0 get O = 0 and LSE = -inf.
 *
 * q            [B*qlen, H, Lk] bf16, strides (q_stride_row, q_stride_h, 1).
 * kv           latent cache [num_pages, P, 1, Lk] (a [num_pages*P, 1, Lk]
 *              view is the same memory), element type kv_dtype, strides
 *              (kv_stride_page, kv_stride_tok, -, 1); each of the two strides
 *              spans under 4 GiB (PD_ERR_UNSUPPORTED otherwise).
 * k_scale      device fp32 scalar dequantising an FP8 cache (value = code *
 *              k_scale, for K and V alike), or NULL for 1; ignored for bf16.
 * block_table  [B, max_blocks] int32; seq_lens, real_seq_lens [B] int32
 *              (real_seq_lens may be NULL).
 * num_kv_splits, workspace: as for GQA with rows = B*qlen, Dv = Lv.
 * out          [B*qlen, H, Lv] bf16, strides (o_stride_row, o_stride_h, 1).
 * lse          [B*qlen, H] fp32 with row stride lse_stride_row, or NULL.
 *
 * Supported: Lk = 576, Lv = 512 (512 + 64 rope dims); any page size P from
 * 1 to 65536 tokens (the module states support for page size >= 1); any
 * qlen * H >= 1 (rows are processed in blocks of 128: fewer rows leave part
 * of a block idle); pointers 16-byte aligned; strides multiples of 16 bytes.
 */
PD_API int paged_verify_mla(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                     const void* kv, int32_t kv_dtype, int64_t kv_stride_page,
                     int64_t kv_stride_tok, int32_t num_pages, const float* k_scale,
                     const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
                     const int32_t* seq_lens, const int32_t* real_seq_lens,
                     int32_t qlen, float sm_scale, int32_t batch, int32_t num_heads,
                     int32_t head_dim_k, int32_t head_dim_v, int32_t page_size,
                     int32_t num_kv_splits, float* workspace, size_t workspace_bytes,
                     void* out, int64_t o_stride_row, int64_t o_stride_h,
                     float* lse, int64_t lse_stride_row, void* stream);

/*
 * paged_verify_mla_partials - the split partials of paged_verify_mla only.
 *
 * Same arguments and row limits as paged_verify_mla, with no outputs: writes
 * every (row, head, split) slot of `workspace` ([B*qlen, H, S, Lv + 1]
 * fp32, S = num_kv_splits >= 1, O already multiplied by k_scale) and
 * launches no merge; a slot a row does not use gets lse = -inf.
 * merge_splits over that workspace (no sinks) gives exactly
 * paged_verify_mla's result: the per-shard half of split-KV for MLA verify.
 * Workspace bytes >= B * qlen * H * S * (Lv + 1) * 4.
 */
PD_API int paged_verify_mla_partials(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                              const void* kv, int32_t kv_dtype, int64_t kv_stride_page,
                              int64_t kv_stride_tok, int32_t num_pages, const float* k_scale,
                              const int32_t* block_table, int64_t bt_stride_b,
                              int32_t max_blocks, const int32_t* seq_lens,
                              const int32_t* real_seq_lens, int32_t qlen, float sm_scale,
                              int32_t batch, int32_t num_heads, int32_t head_dim_k,
                              int32_t head_dim_v, int32_t page_size, int32_t num_kv_splits,
                              float* workspace, size_t workspace_bytes, void* stream);

/*
 * merge_splits - merge fp32 split partials into O (bf16) and LSE (fp32).
 *
 * For each (row, head) with partials (O_s, lse_s) in the workspace layout of
 * pd_workspace_bytes():
 *   M = max_s lse_s,  w_s = e^{lse_s - M} (0 when lse_s = -inf),
 *   O = sum_s w_s O_s / (sum_s w_s + e^{sinks[h] - M}),  LSE = M + ln sum_s w_s,
 * and O = 0, LSE = -inf when every lse_s is -inf.  This is the split combine
 * of "vllm.models.flint.ops.decode_attention" (combine_splits: max over
 * splits, per-split weights, weighted l and O, sink in the final
 * denominator) restated for normalised partials and natural logs.  A split
 * whose lse_s is -inf is skipped, so its O_s may hold anything (even NaN).
 * An lse_s of +inf ends the (row, head)'s list: the sums above run over the
 * slots before it, and nothing after it is read.  (The library's decode and
 * verify calls that merge themselves end each list that way, one store in
 * place of an lse = -inf in every slot no split uses; the *_partials entry
 * points still write -inf into every unused slot.)  A NaN lse_s makes the
 * (row, head) NaN.
 *
 * workspace  fp32 [rows, num_heads, num_splits, head_dim_v + 1], contiguous.
 * sinks      [num_heads] fp32 or NULL.
 * out        [rows, num_heads, head_dim_v] bf16, strides (o_stride_row,
 *            o_stride_h, 1); lse [rows, num_heads] fp32 or NULL.
 * Supported: head_dim_v in {128, 256, 512, 1024}; num_splits >= 1.
 */
PD_API int merge_splits(const float* workspace, int32_t rows, int32_t num_heads,
                 int32_t num_splits, int32_t head_dim_v, const float* sinks,
                 void* out, int64_t o_stride_row, int64_t o_stride_h,
                 float* lse, int64_t lse_stride_row, void* stream);

/*
 * pd_stream_read_probe - measurement helper, not part of the attention path.
 *
 * Reads `bytes` (rounded down to 16) from `src` once with 16-byte
 * non-temporal loads spread over `workgroups` workgroups of 256 threads and
 * keeps nothing: its rate is the streaming-read ceiling of the machine, the
 * figure the HBM-bound kernels above are compared with.  `sink` holds
 * `workgroups` uint32 values the kernel may write (almost never does).
 * src 16-byte aligned.  Returns PD_ERR_INVALID / PD_ERR_ALIGN on bad
 * arguments, PD_ERR_HIP if the launch fails.
 */
PD_API int pd_stream_read_probe(const void* src, size_t bytes, uint32_t* sink,
                                int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_DECODE_H_ */

/*
 * mla.h -- C ABI of libmla.so: MLA (multi-head latent attention) decoding over a
 * paged latent KV cache on one AMD Instinct MI355X (gfx950).
 *
 * The operation.  The TileLang notes ("TileLang: bridging programmability and
 * performance in modern neural kernels", section "A complete example: two-stage
 * optimisation of FlashMLA") present MLA decoding as two chained GEMMs with a
 * softmax between them: S = Q . KV^T kept in registers, down-cast, then
 * O += S_cast . KV.  The pages do not write out the rest; this library fixes it
 * as follows (the plainest reading, and the one the tests hold it to):
 *
 *   For sequence b, query position t < q_len and head h (row r = t*H + h):
 *     L      = cache_seqlens[b]   (counts every cached token, the q_len new ones included)
 *     n      = L                          if !causal or q_len == 1
 *            = max(0, L - q_len + 1 + t)  if causal  (query t sees positions p <= L - q_len + t)
 *     k_p    = kv_cache[block_table[b][p / 64]][p % 64][0:576]   for p < n
 *     s_p    = scale * dot(q[b][t][h][0:576], k_p)
 *     lse    = ln(sum_p exp(s_p))                                 (natural log)
 *     out[d] = sum_p exp(s_p - lse) * k_p[d]        for d < 512   (V = first 512 dims)
 *   A row with n == 0 gets out = 0 and lse = -inf.
 *
 * Attention sinks (mla_decode_ex with variant->sinks != NULL).  The TileLang notes name
 * an attention-sink variant of attention a few lines away from the standard kernel (main
 * results table, and the programmability remarks after it) without writing it out.
 * This library reads it as one more softmax term per head: a logit sinks[h], in score
 * units (the scale does not multiply it), whose value row is zero:
 *     lse    = ln(exp(sinks[h]) + sum_p exp(s_p))
 *     out[d] = sum_p exp(s_p - lse) * k_p[d]
 *   A row with n == 0 then gets out = 0 and lse = sinks[h]; sinks[h] = -inf is the
 *   plain decode for head h, bit for bit.
 *
 * Sparse (top-k) decode (problem->topk > 0, variant->indices).  The DeepSeek-V4 TileLang
 * note mentions the dynamic sparse attention of DeepSeek models without its details.
 * This library reads it as: every (b, t) carries a list of topk token positions of
 * sequence b, shared by all heads, -1 marking an unused entry, and its rows attend to
 * exactly the listed tokens, once per entry, in place of the causal range:
 *     keys of row (b, t, h) = { k_p : p in indices[b][t][0:topk], p != -1 }
 *   Every other entry must lie in [0, cache_seqlens[b]); one that does not (or whose
 *   page is outside the pool) makes that (b, t)'s rows NaN and raises the plan's error
 *   flag.  A list with no used entry gives out = 0, lse = -inf (or the sink).  Each
 *   (b, t) is decoded as its own unit of num_heads rows, so q_len * num_heads may exceed
 *   128 (num_heads may not); bf16 only, causal must be 0, and a plan is required (its
 *   workspace holds the lists turned into pool rows).
 *
 * Sizes fixed by the library: 576-wide cache rows (512 latent + 64 rope), 512-wide
 * values, 64-token pages.  q_len * num_heads (rows per sequence) must be <= 128.
 *
 * Layouts (all C-contiguous, row-major):
 *   q            [batch, q_len, num_heads, 576]     dtype
 *   kv_cache     [num_pages, 64, 576]               dtype
 *   block_table  [batch, block_table_stride] int32; only the first ceil(L/64)
 *                entries of row b are read
 *   cache_seqlens[batch] int32
 *   out          [batch, q_len, num_heads, 512]     dtype (bf16 out is rounded
 *                to nearest even from the fp32 result)
 *   lse          [batch, q_len, num_heads] float32
 *
 * Memory.  Every pointer argument except `problem`, `options`, `plan` and `num_cus` is
 * DEVICE memory; the caller owns every buffer (the library allocates nothing and
 * keeps no per-call state).  Device pointers must be 16-byte aligned (int32 arrays:
 * 4-byte).  `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *
 * Asynchrony.  mla_get_metadata and mla_decode only enqueue work on `stream`;
 * they never synchronise it, never copy to the host and never allocate, so they
 * can be captured in a HIP graph.  A plan (metadata) is valid only for the
 * cache_seqlens contents it was computed from and the problem it was made for.
 *
 * Errors.  Every call returns an mla_status_t.  Argument faults the host can see
 * are reported before anything is enqueued.  Faults only the device can see
 * (a block_table entry outside [0, num_pages), or L > 64 * max_blocks_per_seq)
 * never cause an out-of-bounds access: the affected sequence's out and lse are
 * written as NaN and a flag is raised in the plan's metadata, which
 * mla_plan_error() reads back (that call synchronises the stream).  A decode called
 * without a plan (plan == NULL) has nowhere to raise the flag: its NaN rows are then
 * the only report.  Float32 problems take a plan for this purpose alone.
 * No call throws across the ABI; the library is reentrant and thread-safe.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_PAGE 64
#define MLA_MAX_ROWS 128

typedef enum {
  MLA_DTYPE_F32 = 0,
  MLA_DTYPE_BF16 = 1,
} mla_dtype_t;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,         /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,        /* a size (or the scale) is out of range */
  MLA_ERR_DTYPE = 3,        /* unknown dtype */
  MLA_ERR_ALIGN = 4,        /* a pointer is not aligned as required */
  MLA_ERR_WORKSPACE = 5,    /* metadata or workspace buffer too small */
  MLA_ERR_UNSUPPORTED = 6,  /* valid request this build does not serve */
  MLA_ERR_LAUNCH = 7,       /* the HIP runtime refused a launch */
  MLA_ERR_DEVICE = 8,       /* device query failed */
  MLA_ERR_BAD_INPUT = 9,    /* device-side data fault flagged (see mla_plan_error) */
} mla_status_t;

/* Host-side description of one decode problem. */
typedef struct {
  int32_t batch;               /* B >= 0 (0 = nothing to do) */
  int32_t q_len;               /* T >= 1 new tokens per sequence */
  int32_t num_heads;           /* H >= 1, with T * H <= 128 */
  int32_t causal;              /* 0 or 1: mask within the T new tokens (only used when T > 1) */
  int32_t num_pages;           /* pages in kv_cache (>= 1) */
  int32_t block_table_stride;  /* int32 elements between block_table rows (>= max_blocks_per_seq) */
  int32_t max_blocks_per_seq;  /* entries of a block_table row the library may read (>= 1) */
  int32_t dtype;               /* mla_dtype_t of q, kv_cache and out */
  int32_t topk;                /* sparse decode: list entries per (b, t) (0 = dense) */
} mla_problem_t;

/* Optional knobs of the split planner (NULL = defaults).  Zero fields take defaults. */
typedef struct {
  int32_t num_workgroups;      /* decode workgroups to spread the work over (default: one per CU) */
  int32_t min_blocks_per_wg;   /* smallest share of 64-token blocks per workgroup (default 4) */
  int32_t row_split;           /* split each sequence's rows over this many workgroups: 1, 2 or 4 (default 1) */
  int32_t fixed_split_blocks;  /* > 0: batch-invariant plan (below); 0: balanced shares (default) */
  int32_t split_rule;          /* 0: the cost model picks (default); 1: equal block shares;
                                  2: cost-balanced shares (see mla_get_metadata) */
  int32_t segment_cost;        /* cost model's per-segment overhead in quarter blocks
                                  (0: from the traffic of a segment's rows, see below) */
  int32_t plan_in_decode;      /* 1: every decode launch re-plans from the lengths it is given
                                  (see mla_get_metadata); 0: the plan is made once (default) */
} mla_plan_options_t;

/* Variants of the operation.  NULL (or every field NULL) = plain MLA decode. */
typedef struct {
  const float* sinks;          /* DEVICE float32 [num_heads] attention-sink logits, or NULL */
  const int32_t* indices;      /* DEVICE int32 [batch, q_len, topk] sparse token lists (topk > 0) */
} mla_variant_t;

/* Human-readable name of a status code (static string). */
MLA_API const char* mla_status_string(int32_t status);

/* Compute units of the current HIP device (host call, no GPU work). */
MLA_API int32_t mla_device_num_cus(int32_t* num_cus);

/*
 * Size in bytes of the metadata buffer mla_get_metadata needs for `problem`
 * with `options` (NULL = defaults) on a device with `num_cus` CUs (<= 0: query
 * the current device).  Host-only arithmetic; returns 0 for an invalid problem.
 */
MLA_API size_t mla_metadata_bytes(const mla_problem_t* problem, const mla_plan_options_t* options,
                          int32_t num_cus);

/*
 * Size in bytes of the workspace mla_decode needs with a plan made for the same
 * problem/options/num_cus: room for the split partials, and for a sparse problem the
 * lists turned into pool rows (4 bytes per entry, padded to 64 per (b, t), plus a
 * count).  Host-only arithmetic.
 * A split partial row (one row of one split) takes 2056 bytes, and each partial slot
 * 64 more: the row's float32 output before normalisation, u = o / f (f = 1 / the row's
 * sum of exponentials over the split), as a compensated pair of bf16 halves,
 * hi = bf16(u) and lo = bf16(u - hi) (2 x 1024 B), its float32 natural-log LSE and f, and
 * per slot 4 flag bits per row.  The decode always writes hi, and writes lo only for a
 * quarter of a row (128 values) whose largest normalised |o| exceeds 1, setting that
 * quarter's bit; the merge scales by f, so a partial enters it within 2^-8 (hi alone,
 * |o| <= 1) or 2^-16 |o| (hi + lo) of its float32 value, however much a row's partials
 * cancel.
 */
MLA_API size_t mla_workspace_bytes(const mla_problem_t* problem, const mla_plan_options_t* options,
                           int32_t num_cus);

/*
 * A split plan: the caller-owned device buffer the planner writes, plus the launch
 * shape the host side needs (filled in by mla_get_metadata on the host, so
 * mla_decode never reads device memory to launch).
 */
typedef struct {
  void* metadata;              /* device buffer, >= mla_metadata_bytes (caller sets) */
  size_t metadata_bytes;       /* its size (caller sets) */
  int32_t grid_wg;             /* decode workgroups to launch (filled) */
  int32_t row_split;           /* workgroups per sequence's rows (filled) */
  int32_t rows_per_wg;         /* rows per workgroup (filled) */
  int32_t max_partials;        /* partial slots the workspace must hold (filled) */
  int32_t batch;               /* problem the plan was made for (filled) */
  int32_t rows;                /* q_len * num_heads of that problem (filled) */
  int32_t plan_in_decode;      /* decode launches re-plan (filled; options->plan_in_decode) */
  int32_t min_blocks, fixed_blocks, split_rule, segment_cost, topk;   /* the plan's settings (filled) */
} mla_plan_t;

/*
 * Plan the split-KV work.  Reads cache_seqlens on the device, writes the plan
 * into plan->metadata: every sequence's 64-token blocks (times row_split) are
 * laid end to end and cut into num_workgroups contiguous ranges; a sequence cut across
 * k > 1 workgroups gets k partial results that mla_decode merges by log-sum-exp.
 * Two cuts are ranked by a cost model (the TileLang notes' tile recommender ranks
 * candidate configurations by traffic over bandwidth, "Key design 2: tile
 * recommendation"): equal block shares, and equal shares of cost where every segment a
 * workgroup decodes (a sequence's rows, or its slice of them) adds the traffic of its
 * Q and output rows and its fixed costs, segment_cost quarter blocks (default: from a
 * step-time model in roofline form fitted on MI355X, 11 for 128 rows per workgroup, 13
 * for 64 or fewer).  The plan keeps the cut whose busiest workgroup costs less,
 * equal block shares on a tie; split_rule forces either.
 * With options->fixed_split_blocks = C > 0 the plan is batch-invariant instead: every
 * sequence (row slice) is cut into chunks of C blocks from its own start, one chunk per
 * workgroup, so where a sequence is split -- and so every bit of its output -- does
 * not depend on the other sequences of the batch or on the CU count.  grid_wg is then
 * batch * row_split * ceil(max_blocks_per_seq / C) (workgroups beyond the chunks exit;
 * num_workgroups and min_blocks_per_wg are ignored).
 * A sparse problem is planned as batch * q_len units of ceil(topk / 64) blocks each
 * (cache_seqlens is not read and may be NULL).
 * One single-workgroup kernel launch on `stream`; fills the host fields of *plan.
 * With options->plan_in_decode = 1 (bf16 problems of at most 4095 sequences, or sparse
 * units), the plan depends on the lengths only through the decode: every mla_decode /
 * mla_decode_splits launch made with it recomputes the same cut from the cache_seqlens
 * it is given, inside the decode kernel (each workgroup takes its own share, one writes
 * the metadata the combine reads), so one mla_get_metadata serves every later step of
 * the same problem shape and no planner launch runs per step.  The fault flag is then
 * only ever raised by the decode; mla_plan_error reads and clears it.
 */
MLA_API int32_t mla_get_metadata(const mla_problem_t* problem, const int32_t* cache_seqlens,
                         const mla_plan_options_t* options, int32_t num_cus,
                         mla_plan_t* plan, void* stream);

/*
 * Decode.  Argument order follows the problem statement
 * (q, kv_cache, block_table, cache_seqlens, scale, out, lse, ..., stream).
 *   scale      multiplies every q . k (e.g. 192^-0.5); must be positive and finite
 *              (MLA_ERR_SHAPE otherwise)
 *   plan       from mla_get_metadata for the same problem and cache_seqlens, or
 *              NULL: one workgroup per sequence, no splits, no workspace needed
 *   workspace  device buffer of >= mla_workspace_bytes (unused when plan is NULL)
 * bf16 problems run the MFMA kernel (split-KV decode, then the LSE combine when
 * the plan splits anything); float32 problems run a plain float32 kernel that does not
 * split, and use a plan (NULL allowed) only to raise the device-side fault flag.
 */
MLA_API int32_t mla_decode(const mla_problem_t* problem,
                   const void* q, const void* kv_cache,
                   const int32_t* block_table, const int32_t* cache_seqlens,
                   float scale, void* out, float* lse,
                   const mla_plan_t* plan, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * mla_decode with a variant of the operation (see the top of this file): identical
 * arguments, plus `variant` (NULL = mla_decode).  sinks and indices must be 4-byte
 * aligned (MLA_ERR_ALIGN) and are read on the device only; a sparse problem needs
 * indices (MLA_ERR_NULL) and a plan (MLA_ERR_UNSUPPORTED), and runs one more launch
 * first (its lists into pool rows).  The sink enters each row once, where
 * its final result is formed: in the decode kernel for an unsplit sequence, in the
 * combine for a split one (partials never include it), so split and unsplit plans
 * agree to rounding.
 */
MLA_API int32_t mla_decode_ex(const mla_problem_t* problem, const mla_variant_t* variant,
                              const void* q, const void* kv_cache,
                              const int32_t* block_table, const int32_t* cache_seqlens,
                              float scale, void* out, float* lse,
                              const mla_plan_t* plan, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The two launches of mla_decode_ex, for callers (and benchmarks) that want them apart.
 * mla_decode_splits: the split-KV decode kernel alone -- writes out/lse of every
 *   sequence the plan did not split, and the partials of the split ones into
 *   `workspace` (per split: the normalised output as a compensated bf16 pair, see
 *   mla_workspace_bytes, and its natural-log LSE in float32).
 * mla_combine: merges those partials by log-sum-exp into out/lse (sequences with no
 *   cached tokens get out = 0, lse = -inf).  Same plan and workspace as the decode.
 * Both require a plan and a bf16 problem, and take the same `variant` (NULL = plain);
 * mla_decode_ex(plan != NULL) == splits + combine.
 */
MLA_API int32_t mla_decode_splits(const mla_problem_t* problem, const mla_variant_t* variant,
                                  const void* q, const void* kv_cache,
                                  const int32_t* block_table, const int32_t* cache_seqlens,
                                  float scale, void* out, float* lse,
                                  const mla_plan_t* plan, void* workspace, size_t workspace_bytes,
                                  void* stream);
/*
 * mla_decode_splits_timed: mla_decode_splits whose decode kernel launch also records
 * two caller-created HIP events (hipEvent_t, timing enabled) bound to that kernel's own
 * start and end, so hipEventElapsedTime(start, stop) is the kernel's duration.  The
 * events add no packet of their own between launches (a sparse problem's list kernel
 * runs before `start`).  For measurement; both events NULL is mla_decode_splits, one
 * NULL is MLA_ERR_NULL.
 */
MLA_API int32_t mla_decode_splits_timed(const mla_problem_t* problem, const mla_variant_t* variant,
                                        const void* q, const void* kv_cache,
                                        const int32_t* block_table, const int32_t* cache_seqlens,
                                        float scale, void* out, float* lse,
                                        const mla_plan_t* plan, void* workspace, size_t workspace_bytes,
                                        void* stream, void* start_event, void* stop_event);
MLA_API int32_t mla_combine(const mla_problem_t* problem, const mla_variant_t* variant,
                            void* out, float* lse,
                            const mla_plan_t* plan, const void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  mla_get_metadata + mla_decode_ex in one
 * call, with the default plan (one workgroup per CU of the stream's device) and the split
 * partials kept in device memory the library owns: a static array of
 * MLA_NOALLOC_SCRATCH_BYTES (137 MiB: 1 MiB of plan metadata, 136 MiB of workspace) that
 * every device the library runs on holds until the process ends.  The caller passes the
 * inputs and outputs only; the call allocates nothing and never synchronises.
 *   - A problem whose default plan needs more metadata or workspace than that (for
 *     128-row problems, more than 541 partial slots, i.e. far more sequences than CUs)
 *     returns MLA_ERR_WORKSPACE before anything is enqueued; a sparse problem
 *     (topk > 0) returns MLA_ERR_UNSUPPORTED (its row lists need a caller workspace).
 *   - Every call on a device shares that device's scratch, which keeps the last call's
 *     contents: two calls that overlap on one device (different streams, or different
 *     host threads) race and may corrupt each other's results.  Serialise them.
 *   - Device-side input faults make the affected rows NaN, as in mla_decode; the flag
 *     they raise stays in the scratch and is not reported (use mla_decode with a plan to
 *     read it).
 * Results are bit-identical to mla_get_metadata (default options, the device's CU count)
 * followed by mla_decode_ex with that plan.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)137 << 20)
MLA_API int32_t mla_decode_noalloc(const mla_problem_t* problem, const mla_variant_t* variant,
                                   const void* q, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* cache_seqlens,
                                   float scale, void* out, float* lse, void* stream);

/*
 * Read back the device-side error flag of a plan after mla_decode ran with it:
 * synchronises `stream`, returns MLA_OK or MLA_ERR_BAD_INPUT, and clears the flag.
 */
MLA_API int32_t mla_plan_error(const mla_plan_t* plan, void* stream);

/*
 * HBM streaming-read probe, a measurement aid outside the decode path: the read
 * bandwidth the device delivers to a plain stream, the ceiling the decode's bytes per
 * second are read against (the TileLang notes rank candidate kernels by traffic over
 * bandwidth, "Key design 2: tile recommendation"; this measures the bandwidth term).
 *
 * Reads `bytes` of DEVICE memory at `src` (16-byte aligned) exactly once, split into
 * equal contiguous chunks over `num_workgroups` workgroups of 256 threads (<= 0: 4 per
 * CU for mode 0, 1 per CU for mode 1), either
 *   mode 0: with 16-byte vector loads into registers, or
 *   mode 1: with the decode's wave-wide global->LDS copies (1 KB each) into an LDS ring.
 * `sink` (DEVICE uint32 [num_workgroups], 4-byte aligned) keeps the loads live; its
 * contents are unspecified.  Each chunk (bytes / workgroups) must be a positive multiple
 * of 16 KiB below 4 GiB (MLA_ERR_SHAPE otherwise); NULL pointers give MLA_ERR_NULL, a
 * mode other than 0 or 1 MLA_ERR_UNSUPPORTED, misalignment MLA_ERR_ALIGN, all before
 * anything is enqueued.  Enqueues one kernel on `stream`; time it with events there.
 */
MLA_API int32_t mla_hbm_read_probe(const void* src, size_t bytes, int32_t mode, int32_t num_workgroups,
                                   uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */

// Host side of libmla.so: argument checks, sizing, plan bookkeeping and launches.
// Validation happens here in C++ before anything is enqueued (the DeepSeek-V4
// TileLang note, section "Points from the V4 report", on moving launch and tensor
// checks out of Python into compiled host code).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mla.h"
#include "mla_args.h"
#include "mla_device.h"
#include "mla_plan_core.h"

namespace {

constexpr int kDefaultMinBlocks = 4;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Split partials, over prow = slots * rows partial rows: the unnormalised output's bf16
// high halves [prow, 512]; the fp32 (LSE, normalising factor) pairs [prow, 2], padded to
// 16 bytes; the low-half flags [slots, kLoMaskWords]; the low halves [prow, 512].  The
// combine reads the first three.
size_t lse_bytes(size_t prow) { return (prow * 2 * sizeof(float) + 15) / 16 * 16; }
size_t partial_bytes(int64_t slots, int64_t rows_per_wg) {
  const size_t prow = (size_t)slots * rows_per_wg;
  return 2 * prow * mla::kDv * sizeof(uint16_t) + lse_bytes(prow) + (size_t)slots * mla::kLoMaskWords * sizeof(uint32_t);
}

int32_t check_problem(const mla_problem_t* p) {
  if (!p) return MLA_ERR_NULL;
  if (p->dtype != MLA_DTYPE_F32 && p->dtype != MLA_DTYPE_BF16) return MLA_ERR_DTYPE;
  if (p->batch < 0 || p->q_len < 1 || p->num_heads < 1 || p->topk < 0) return MLA_ERR_SHAPE;
  // a sparse problem decodes every (b, t) as its own unit of num_heads rows
  const int64_t rows = p->topk > 0 ? p->num_heads : (int64_t)p->q_len * p->num_heads;
  if (rows > MLA_MAX_ROWS) return MLA_ERR_SHAPE;
  if (p->topk > 0) {
    if (p->topk > (1 << 24) || (int64_t)p->batch * p->q_len > INT32_MAX / 2) return MLA_ERR_SHAPE;
    if ((int64_t)p->batch * p->q_len * ((p->topk + 63) / 64) * 4 > INT32_MAX) return MLA_ERR_SHAPE;
    if (p->causal != 0 || p->dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  }
  if (p->causal != 0 && p->causal != 1) return MLA_ERR_SHAPE;
  if (p->num_pages < 1 || p->max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  if (p->block_table_stride < p->max_blocks_per_seq) return MLA_ERR_SHAPE;
  // global block positions, page offsets and partial indices stay in int32 range
  if ((int64_t)p->batch * p->max_blocks_per_seq > INT32_MAX / 4) return MLA_ERR_SHAPE;
  if ((int64_t)p->batch * p->block_table_stride > INT32_MAX) return MLA_ERR_SHAPE;
  return MLA_OK;
}

// The problem the planner and the decode kernel see.  A sparse problem becomes
// batch * q_len sequences of one query token and num_heads rows, each holding topk keys
// (blocks of 64 list entries).  A dense problem is unchanged.
mla_problem_t effective_problem(const mla_problem_t& p) {
  if (p.topk <= 0) return p;
  mla_problem_t e = p;
  e.batch = p.batch * p.q_len;
  e.q_len = 1;
  e.causal = 0;
  e.max_blocks_per_seq = (p.topk + mla::kPage - 1) / mla::kPage;
  e.block_table_stride = e.max_blocks_per_seq;
  e.topk = 0;
  return e;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Sparse scratch after the partials: pool rows [units, 64 * blocks] and kept counts [units].
size_t sparse_rows_bytes(const mla_problem_t& p) {
  if (p.topk <= 0) return 0;
  const size_t units = (size_t)p.batch * p.q_len;
  return align256(units * ((p.topk + mla::kPage - 1) / mla::kPage) * mla::kPage * sizeof(int32_t));
}
size_t sparse_bytes(const mla_problem_t& p) {
  return p.topk <= 0 ? 0 : sparse_rows_bytes(p) + align256((size_t)p.batch * p.q_len * sizeof(int32_t));
}

std::atomic<int32_t> g_cus_cache{0};

int32_t resolve_cus(int32_t num_cus, int32_t* out) {
  if (num_cus > 0) { *out = num_cus; return MLA_OK; }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MLA_ERR_DEVICE;
  *out = cus;
  return MLA_OK;
}

struct PlanShape {
  int grid_wg, row_split, rows_per_wg, min_blocks, max_partials, fixed_blocks, split_rule, seg_cost, in_decode;
};

// Cost-model overhead of one segment (a unit's rows decoded by one workgroup) besides
// its KV blocks, in quarter blocks: the step-time model's per-segment time over its time
// per block at this row count, the larger of a block's HBM time and its MFMA time (the
// TileLang notes' tile recommender in its roofline form, "Key design 2: tile
// recommendation").  The three times, in hundredths of a microsecond, were measured by
// fitting the model to plan sweeps on MI355X (mla_decode_03_amd.tune fit): 7.61 us per
// segment, 2.31 us per block from HBM, 2.86 us per block of MFMA work at 128 rows.
// 128 rows give 11 quarters, 64 or fewer 13.
constexpr int64_t kSegHundredthsUs = 761, kBlkMemHundredthsUs = 231, kBlkMfma128HundredthsUs = 286;
int segment_cost_quarters(int rows_per_wg) {
  const int64_t blk = std::max<int64_t>(kBlkMemHundredthsUs * 128, kBlkMfma128HundredthsUs * (int64_t)rows_per_wg);
  return (int)((4 * kSegHundredthsUs * 128 + blk / 2) / blk);
}

int32_t plan_shape(const mla_problem_t* problem, const mla_plan_options_t* o, int32_t num_cus, PlanShape* s) {
  int32_t rc = check_problem(problem);
  if (rc != MLA_OK) return rc;
  const mla_problem_t e = effective_problem(*problem);
  const mla_problem_t* p = &e;
  int32_t cus = 0;
  rc = resolve_cus(num_cus, &cus);
  if (rc != MLA_OK) return rc;
  const int rows = p->q_len * p->num_heads;
  int grid = (o && o->num_workgroups > 0) ? o->num_workgroups : cus;
  int minb = (o && o->min_blocks_per_wg > 0) ? o->min_blocks_per_wg : kDefaultMinBlocks;
  int rsplit = (o && o->row_split > 0) ? o->row_split : 1;
  if (rsplit != 1 && rsplit != 2 && rsplit != 4) return MLA_ERR_UNSUPPORTED;
  if (rows % rsplit != 0) return MLA_ERR_UNSUPPORTED;
  const int fixed = (o && o->fixed_split_blocks > 0) ? o->fixed_split_blocks : 0;
  const int64_t units = (int64_t)p->batch * rsplit;
  if (fixed > 0) {
    // one workgroup per chunk of `fixed` blocks, at most ceil(max_blocks / fixed) per unit
    const int64_t g = units * (((int64_t)p->max_blocks_per_seq + fixed - 1) / fixed);
    if (g > 65536) return MLA_ERR_SHAPE;
    grid = (int)(g > 0 ? g : 1);
  }
  if (grid > 65536) return MLA_ERR_SHAPE;
  s->grid_wg = grid;
  s->row_split = rsplit;
  s->rows_per_wg = rows / rsplit;
  s->min_blocks = minb;
  s->fixed_blocks = fixed;
  s->split_rule = o ? o->split_rule : 0;
  if (s->split_rule < 0 || s->split_rule > 2) return MLA_ERR_UNSUPPORTED;
  s->seg_cost = (o && o->segment_cost > 0) ? o->segment_cost : segment_cost_quarters(s->rows_per_wg);
  if (s->seg_cost > (1 << 20)) return MLA_ERR_SHAPE;
  // each workgroup range holds at most one partial segment at each end (fixed chunks: one)
  s->max_partials = fixed > 0 ? grid : (int)(grid + (units < grid ? units : grid));
  // re-planning inside the decode keeps the lengths' prefix sums in LDS
  s->in_decode = (o && o->plan_in_decode) ? 1 : 0;
  if (o && (o->plan_in_decode < 0 || o->plan_in_decode > 1)) return MLA_ERR_UNSUPPORTED;
  if (s->in_decode && (p->batch > mla::kPlanLdsBatch || p->dtype != MLA_DTYPE_BF16)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer";
    case MLA_ERR_SHAPE: return "size out of range";
    case MLA_ERR_DTYPE: return "unknown dtype";
    case MLA_ERR_ALIGN: return "misaligned pointer";
    case MLA_ERR_WORKSPACE: return "metadata or workspace too small";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_DEVICE: return "device query failed";
    case MLA_ERR_BAD_INPUT: return "device-side input fault (bad block_table entry or sequence length)";
    default: return "unknown status";
  }
}

int32_t mla_device_num_cus(int32_t* num_cus) {
  if (!num_cus) return MLA_ERR_NULL;
  int32_t c = g_cus_cache.load(std::memory_order_relaxed);
  if (c <= 0) {
    int32_t rc = resolve_cus(0, &c);
    if (rc != MLA_OK) return rc;
    g_cus_cache.store(c, std::memory_order_relaxed);
  }
  *num_cus = c;
  return MLA_OK;
}

size_t mla_metadata_bytes(const mla_problem_t* problem, const mla_plan_options_t* options, int32_t num_cus) {
  PlanShape s;
  if (plan_shape(problem, options, num_cus, &s) != MLA_OK) return 0;
  return mla::meta_words(effective_problem(*problem).batch, s.row_split, s.grid_wg) * sizeof(int32_t);
}

size_t mla_workspace_bytes(const mla_problem_t* problem, const mla_plan_options_t* options, int32_t num_cus) {
  PlanShape s;
  if (plan_shape(problem, options, num_cus, &s) != MLA_OK) return 0;
  return align256(partial_bytes(s.max_partials, s.rows_per_wg)) + sparse_bytes(*problem);
}

int32_t mla_get_metadata(const mla_problem_t* problem, const int32_t* cache_seqlens,
                         const mla_plan_options_t* options, int32_t num_cus, mla_plan_t* plan,
                         void* stream) {
  if (!problem || !plan) return MLA_ERR_NULL;
  PlanShape s;
  int32_t rc = plan_shape(problem, options, num_cus, &s);
  if (rc != MLA_OK) return rc;
  const int topk = problem->topk;          // sparse: every unit holds topk keys, lengths unread
  const bool sparse = topk > 0;
  const mla_problem_t e = effective_problem(*problem);
  problem = &e;
  if (!plan->metadata || (problem->batch > 0 && !sparse && !cache_seqlens)) return MLA_ERR_NULL;
  if (!aligned(plan->metadata, 16) || !aligned(cache_seqlens, 4)) return MLA_ERR_ALIGN;
  const size_t need = mla::meta_words(problem->batch, s.row_split, s.grid_wg) * sizeof(int32_t);
  if (plan->metadata_bytes < need) return MLA_ERR_WORKSPACE;
  plan->grid_wg = s.grid_wg;
  plan->row_split = s.row_split;
  plan->rows_per_wg = s.rows_per_wg;
  plan->max_partials = s.max_partials;
  plan->batch = problem->batch;
  plan->rows = problem->q_len * problem->num_heads;
  plan->plan_in_decode = s.in_decode;
  plan->min_blocks = s.min_blocks;
  plan->fixed_blocks = s.fixed_blocks;
  plan->split_rule = s.split_rule;
  plan->segment_cost = s.seg_cost;
  plan->topk = topk;
  if (mla_launch_plan(cache_seqlens, static_cast<int32_t*>(plan->metadata), problem->batch,
                      plan->rows, s.row_split, s.grid_wg, s.min_blocks, problem->max_blocks_per_seq,
                      s.max_partials, s.fixed_blocks, s.split_rule, s.seg_cost,
                      topk,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_LAUNCH;
  return MLA_OK;
}

namespace {

// Checks shared by every decode entry; fills the kernel argument block for the problem
// the kernels see (effective_problem).
int32_t prepare_decode(const mla_problem_t* problem, const void* q, const void* kv_cache,
                       const int32_t* block_table, const int32_t* cache_seqlens, float scale,
                       void* out, float* lse, mla::DecodeArgs* a) {
  int32_t rc = check_problem(problem);
  if (rc != MLA_OK) return rc;
  const mla_problem_t p = effective_problem(*problem);
  if (!q || !kv_cache || !block_table || !cache_seqlens || !out || !lse) return MLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
      !aligned(block_table, 4) || !aligned(cache_seqlens, 4))
    return MLA_ERR_ALIGN;
  a->q = static_cast<const uint8_t*>(q);
  a->kv = static_cast<const uint8_t*>(kv_cache);
  a->block_table = block_table;
  a->seqlens = cache_seqlens;
  a->out = static_cast<uint16_t*>(out);
  a->lse = lse;
  a->scale_log2 = scale * mla::kLog2e;
  // the kernels take the row max on unscaled scores: the scale must be positive
  if (!(scale > 0.f) || !(a->scale_log2 <= 3.0e38f)) return MLA_ERR_SHAPE;
  a->batch = p.batch;
  a->rows = p.q_len * p.num_heads;
  a->q_len = p.q_len;
  a->heads = p.num_heads;
  a->causal = p.causal;
  a->num_pages = p.num_pages;
  a->bt_stride = p.block_table_stride;
  a->max_blocks = p.max_blocks_per_seq;
  a->meta = nullptr;
  a->ws_hi = nullptr;
  a->ws_lo = nullptr;
  a->ws_lse = nullptr;
  a->ws_lo_mask = nullptr;
  a->rows_per_wg = a->rows;
  a->row_split = 1;
  a->plan_in_decode = 0;
  a->plan_min_blocks = a->plan_max_partials = a->plan_fixed_blocks = 0;
  a->plan_split_rule = a->plan_seg_cost = a->plan_uniform_len = 0;
  a->sinks = nullptr;
  a->sparse_rows = nullptr;
  a->sparse_stride = 0;
  return MLA_OK;
}

// Reads the variant into *a (NULL = the plain operation).  A sparse problem's decode
// needs the index lists (need_indices); its combine does not.
int32_t attach_variant(const mla_problem_t& p, const mla_variant_t* variant, bool need_indices,
                       mla::DecodeArgs* a, const int32_t** indices) {
  const int32_t* idx = variant ? variant->indices : nullptr;
  if (p.topk > 0 && need_indices && !idx) return MLA_ERR_NULL;
  if (idx && !aligned(idx, 4)) return MLA_ERR_ALIGN;
  if (variant && variant->sinks && !aligned(variant->sinks, 4)) return MLA_ERR_ALIGN;
  a->sinks = variant ? variant->sinks : nullptr;
  if (indices) *indices = idx;
  return MLA_OK;
}

// Bytes of the workspace's partials region: bf16 outputs, then fp32 LSEs (a sparse
// problem's row lists follow it, 256-byte aligned).
size_t partials_region(const mla_problem_t& p, int64_t slots, int64_t rows_per_wg) {
  const size_t b = partial_bytes(slots, rows_per_wg);
  return p.topk > 0 ? align256(b) : b;
}

// Checks a plan and workspace against the problem; sets the plan fields of *a (and, for
// a sparse problem, the row lists and kept counts the first launch writes).
int32_t attach_plan(const mla_problem_t& orig, const mla_plan_t* plan, const void* workspace,
                    size_t workspace_bytes, mla::DecodeArgs* a) {
  if (!plan || !plan->metadata) return MLA_ERR_NULL;
  const mla_problem_t p = effective_problem(orig);
  const int rows = p.q_len * p.num_heads;
  if (plan->batch != p.batch || plan->rows != rows || plan->grid_wg < 1 || plan->row_split < 1 ||
      plan->rows_per_wg * plan->row_split != rows || plan->max_partials < 0)
    return MLA_ERR_SHAPE;
  if (!aligned(plan->metadata, 16)) return MLA_ERR_ALIGN;
  const size_t part = partials_region(orig, plan->max_partials, plan->rows_per_wg);
  const size_t ws_need = part + sparse_bytes(orig);
  if (ws_need > 0 && !workspace) return MLA_ERR_NULL;
  if (workspace_bytes < ws_need) return MLA_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 16)) return MLA_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(const_cast<void*>(workspace));
  a->meta = static_cast<int32_t*>(plan->metadata);
  const size_t prow = (size_t)plan->max_partials * plan->rows_per_wg;   // partial rows
  uint8_t* p_lse = ws + prow * mla::kDv * sizeof(uint16_t);
  uint8_t* p_mask = p_lse + lse_bytes(prow);
  a->ws_hi = reinterpret_cast<uint16_t*>(ws);
  a->ws_lse = reinterpret_cast<float*>(p_lse);
  a->ws_lo_mask = reinterpret_cast<uint32_t*>(p_mask);
  a->ws_lo = reinterpret_cast<uint16_t*>(p_mask + (size_t)plan->max_partials * mla::kLoMaskWords * sizeof(uint32_t));
  a->rows_per_wg = plan->rows_per_wg;
  a->row_split = plan->row_split;
  a->plan_in_decode = plan->plan_in_decode;
  a->plan_min_blocks = plan->min_blocks;
  a->plan_max_partials = plan->max_partials;
  a->plan_fixed_blocks = plan->fixed_blocks;
  a->plan_split_rule = plan->split_rule;
  a->plan_seg_cost = plan->segment_cost;
  a->plan_uniform_len = plan->topk;
  if (plan->plan_in_decode && (p.batch > mla::kPlanLdsBatch || p.dtype != MLA_DTYPE_BF16)) return MLA_ERR_UNSUPPORTED;
  if (orig.topk > 0) {
    a->sparse_rows = reinterpret_cast<const int32_t*>(ws + part);
    a->sparse_stride = p.max_blocks_per_seq * mla::kPage;
    a->seqlens = reinterpret_cast<const int32_t*>(ws + part + sparse_rows_bytes(orig));   // kept counts
  }
  return MLA_OK;
}

// Sparse problems: turn the (b, t) index lists into pool rows and kept counts (the
// buffers attach_plan pointed *a at).
int32_t launch_sparse_rows(const mla_problem_t& orig, const int32_t* indices, const int32_t* block_table,
                           const int32_t* cache_seqlens, const mla::DecodeArgs& a, hipStream_t st) {
  mla::SparseArgs sp;
  sp.indices = indices;
  sp.seqlens = cache_seqlens;
  sp.block_table = block_table;
  sp.rows = const_cast<int32_t*>(a.sparse_rows);
  sp.lens = const_cast<int32_t*>(a.seqlens);
  sp.units = orig.batch * orig.q_len;
  sp.q_len = orig.q_len;
  sp.topk = orig.topk;
  sp.row_stride = a.sparse_stride;
  sp.bt_stride = orig.block_table_stride;
  sp.max_blocks = orig.max_blocks_per_seq;
  sp.num_pages = orig.num_pages;
  return mla_launch_sparse_rows(&sp, st) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

// The merge of a plan's partials.  The grouped form (4 thread groups per row) where the
// plan's units average 8 or more partials (grid_wg >= 8 units); chosen from the plan's
// shape, never from the lengths, and never for fixed chunks, whose results must not depend
// on the batch around a sequence.
int32_t launch_combine(const mla::DecodeArgs& a, int grid_wg, hipStream_t st) {
  mla::CombineArgs c;
  c.grouped = a.plan_fixed_blocks == 0 && grid_wg >= 8 * a.batch * a.row_split;
  c.meta = a.meta;
  c.ws_hi = a.ws_hi;
  c.ws_lo = a.ws_lo;
  c.ws_lse = a.ws_lse;
  c.ws_lo_mask = a.ws_lo_mask;
  c.out = a.out;
  c.lse = a.lse;
  c.batch = a.batch;
  c.rows = a.rows;
  c.rows_per_wg = a.rows_per_wg;
  c.row_split = a.row_split;
  c.heads = a.heads;
  c.sinks = a.sinks;
  return mla_launch_combine(&c, st) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

// The bf16 decode launches of a planned problem: row lists (sparse), then the split-KV
// kernel.
int32_t launch_planned_decode(const mla_problem_t& orig, const int32_t* indices, const int32_t* block_table,
                              const int32_t* cache_seqlens, const mla::DecodeArgs& a, int grid, hipStream_t st,
                              hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
  if (orig.topk > 0) {
    const int32_t rc = launch_sparse_rows(orig, indices, block_table, cache_seqlens, a, st);
    if (rc != MLA_OK) return rc;
  }
  return mla_launch_decode_bf16(&a, grid, st, start, stop) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // namespace

int32_t mla_decode(const mla_problem_t* problem, const void* q, const void* kv_cache,
                   const int32_t* block_table, const int32_t* cache_seqlens, float scale, void* out,
                   float* lse, const mla_plan_t* plan, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return mla_decode_ex(problem, nullptr, q, kv_cache, block_table, cache_seqlens, scale, out, lse, plan,
                       workspace, workspace_bytes, stream);
}

int32_t mla_decode_ex(const mla_problem_t* problem, const mla_variant_t* variant, const void* q,
                      const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
                      float scale, void* out, float* lse, const mla_plan_t* plan, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int32_t rc = check_problem(problem);
  if (rc != MLA_OK) return rc;
  if (problem->batch == 0) return MLA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  mla::DecodeArgs a;
  rc = prepare_decode(problem, q, kv_cache, block_table, cache_seqlens, scale, out, lse, &a);
  if (rc != MLA_OK) return rc;
  const int32_t* indices = nullptr;
  rc = attach_variant(*problem, variant, true, &a, &indices);
  if (rc != MLA_OK) return rc;
  if (problem->dtype == MLA_DTYPE_F32) {
    mla::F32Args f;
    f.q = static_cast<const float*>(q);
    f.kv = static_cast<const float*>(kv_cache);
    f.block_table = block_table;
    f.seqlens = cache_seqlens;
    f.out = static_cast<float*>(out);
    f.lse = lse;
    f.sinks = a.sinks;
    f.scale = scale;
    f.batch = a.batch;
    f.rows = a.rows;
    f.q_len = a.q_len;
    f.heads = a.heads;
    f.causal = a.causal;
    f.num_pages = a.num_pages;
    f.bt_stride = a.bt_stride;
    f.max_blocks = a.max_blocks;
    // float32 problems are not split; a plan, if given, only receives the fault flag
    f.err = nullptr;
    if (plan) {
      if (!plan->metadata) return MLA_ERR_NULL;
      if (plan->batch != a.batch || plan->rows != a.rows) return MLA_ERR_SHAPE;
      if (!aligned(plan->metadata, 16)) return MLA_ERR_ALIGN;
      f.err = static_cast<int32_t*>(plan->metadata) + mla::kHdrError;
    }
    return mla_launch_decode_f32(&f, st) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
  }
  if (!plan) {
    if (problem->topk > 0) return MLA_ERR_UNSUPPORTED;   // the row lists live in the workspace
    return mla_launch_decode_bf16(&a, a.batch, st, nullptr, nullptr) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
  }
  rc = attach_plan(*problem, plan, workspace, workspace_bytes, &a);
  if (rc != MLA_OK) return rc;
  rc = launch_planned_decode(*problem, indices, block_table, cache_seqlens, a, plan->grid_wg, st);
  if (rc != MLA_OK) return rc;
  return launch_combine(a, plan->grid_wg, st);
}

int32_t mla_decode_splits(const mla_problem_t* problem, const mla_variant_t* variant, const void* q,
                          const void* kv_cache,
                          const int32_t* block_table, const int32_t* cache_seqlens, float scale,
                          void* out, float* lse, const mla_plan_t* plan, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return mla_decode_splits_timed(problem, variant, q, kv_cache, block_table, cache_seqlens, scale, out, lse, plan,
                                 workspace, workspace_bytes, stream, nullptr, nullptr);
}

int32_t mla_decode_splits_timed(const mla_problem_t* problem, const mla_variant_t* variant, const void* q,
                                const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
                                float scale, void* out, float* lse, const mla_plan_t* plan, void* workspace,
                                size_t workspace_bytes, void* stream, void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return MLA_ERR_NULL;
  int32_t rc = check_problem(problem);
  if (rc != MLA_OK) return rc;
  if (problem->dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (problem->batch == 0) return MLA_OK;
  mla::DecodeArgs a;
  rc = prepare_decode(problem, q, kv_cache, block_table, cache_seqlens, scale, out, lse, &a);
  if (rc != MLA_OK) return rc;
  const int32_t* indices = nullptr;
  rc = attach_variant(*problem, variant, true, &a, &indices);
  if (rc != MLA_OK) return rc;
  rc = attach_plan(*problem, plan, workspace, workspace_bytes, &a);
  if (rc != MLA_OK) return rc;
  return launch_planned_decode(*problem, indices, block_table, cache_seqlens, a, plan->grid_wg,
                               static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                               static_cast<hipEvent_t>(stop_event));
}

int32_t mla_combine(const mla_problem_t* problem, const mla_variant_t* variant, void* out, float* lse,
                    const mla_plan_t* plan, const void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc = check_problem(problem);
  if (rc != MLA_OK) return rc;
  if (problem->dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (problem->batch == 0) return MLA_OK;
  if (!out || !lse) return MLA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(lse, 4)) return MLA_ERR_ALIGN;
  const mla_problem_t e = effective_problem(*problem);
  mla::DecodeArgs a{};
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.batch = e.batch;
  a.rows = e.q_len * e.num_heads;
  a.heads = e.num_heads;
  rc = attach_variant(*problem, variant, false, &a, nullptr);
  if (rc != MLA_OK) return rc;
  rc = attach_plan(*problem, plan, workspace, workspace_bytes, &a);
  if (rc != MLA_OK) return rc;
  return launch_combine(a, plan->grid_wg, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- the entry point that allocates nothing --------------------------------------------
// mla_decode_noalloc keeps its plan and split partials in `scratch`, library-owned device
// memory: the first kScratchMetaBytes hold the plan's metadata, the rest the workspace.
namespace {
constexpr size_t kScratchMetaBytes = size_t(1) << 20;
constexpr size_t kScratchWorkspaceBytes = size_t(136) << 20;
constexpr size_t kScratchBytes = kScratchMetaBytes + kScratchWorkspaceBytes;
static_assert(kScratchBytes == MLA_NOALLOC_SCRATCH_BYTES, "mla.h states the scratch size");
}  // namespace

__device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];   // per device: the array's device address there

// Device address of `scratch` on device `dev`, looked up once per device with that device
// current (each device holds its own copy of the array at its own address).
int32_t scratch_on(int dev, uint8_t** out) {
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MLA_ERR_DEVICE;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MLA_ERR_DEVICE;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MLA_ERR_DEVICE;
    if (e != hipSuccess || !ptr) return MLA_ERR_DEVICE;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}
}  // namespace

extern "C" {

int32_t mla_decode_noalloc(const mla_problem_t* problem, const mla_variant_t* variant, const void* q,
                           const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
                           float scale, void* out, float* lse, void* stream) {
  int32_t rc = check_problem(problem);
  if (rc != MLA_OK) return rc;
  if (problem->topk > 0) return MLA_ERR_UNSUPPORTED;   // sparse row lists need a caller workspace
  if (problem->batch == 0) return MLA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MLA_ERR_DEVICE;
  // the default plan on that device must fit the scratch (checked before anything is enqueued)
  PlanShape s;
  rc = plan_shape(problem, nullptr, cus, &s);
  if (rc != MLA_OK) return rc;
  const size_t meta_need = mla::meta_words(problem->batch, s.row_split, s.grid_wg) * sizeof(int32_t);
  const size_t ws_need = problem->dtype == MLA_DTYPE_BF16 ? partial_bytes(s.max_partials, s.rows_per_wg) : 0;
  if (meta_need > kScratchMetaBytes || ws_need > kScratchWorkspaceBytes) return MLA_ERR_WORKSPACE;
  uint8_t* base = nullptr;
  rc = scratch_on(dev, &base);
  if (rc != MLA_OK) return rc;
  mla_plan_t plan;
  std::memset(&plan, 0, sizeof plan);
  plan.metadata = base;
  plan.metadata_bytes = kScratchMetaBytes;
  rc = mla_get_metadata(problem, cache_seqlens, nullptr, cus, &plan, stream);
  if (rc != MLA_OK) return rc;
  return mla_decode_ex(problem, variant, q, kv_cache, block_table, cache_seqlens, scale, out, lse, &plan,
                       base + kScratchMetaBytes, kScratchWorkspaceBytes, stream);
}

int32_t mla_plan_error(const mla_plan_t* plan, void* stream) {
  if (!plan || !plan->metadata) return MLA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t flag = 0;
  int32_t* dflag = static_cast<int32_t*>(plan->metadata) + mla::kHdrError;
  if (hipStreamSynchronize(st) != hipSuccess) return MLA_ERR_DEVICE;
  if (hipMemcpy(&flag, dflag, sizeof flag, hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_DEVICE;
  if (flag) {
    const int32_t zero = 0;
    if (hipMemcpy(dflag, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return MLA_ERR_DEVICE;
    return MLA_ERR_BAD_INPUT;
  }
  return MLA_OK;
}

// the probe's launcher (mla_probe.hip); declared here, the probe is no part of the decode
MLA_INTERNAL hipError_t mla_launch_probe(const void* src, size_t bytes, int mode, int num_wg, uint32_t* sink,
                                         hipStream_t stream);

int32_t mla_hbm_read_probe(const void* src, size_t bytes, int32_t mode, int32_t num_workgroups, uint32_t* sink,
                           void* stream) {
  if (!src || !sink) return MLA_ERR_NULL;
  if (mode != 0 && mode != 1) return MLA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return MLA_ERR_ALIGN;
  int32_t nwg = num_workgroups;
  if (nwg <= 0) {
    if (bytes == 0) return MLA_ERR_SHAPE;
    int32_t cus = 0;
    const int32_t rc = mla_device_num_cus(&cus);
    if (rc != MLA_OK) return rc;
    nwg = mode == 0 ? 4 * cus : cus;
  }
  // every workgroup reads an equal chunk, a multiple of 16 KiB below 4 GiB
  if (bytes == 0 || bytes % (size_t)nwg != 0) return MLA_ERR_SHAPE;
  const size_t chunk = bytes / (size_t)nwg;
  if (chunk % 16384 != 0 || chunk >= ((size_t)1 << 32)) return MLA_ERR_SHAPE;
  return mla_launch_probe(src, bytes, mode, nwg, sink, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_LAUNCH;
}

}  // extern "C"

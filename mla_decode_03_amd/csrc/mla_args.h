// Kernel argument blocks and launcher entry points shared by the host API and the
// kernel translation units of libmla.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Low-half flags of a partial slot: 4 bits per row (bit q: values 128q .. 128q+127 of the
// row have a low half), rows 8m .. 8m+7 in word m, so 16 words cover a slot's 128 rows.
constexpr int kLoMaskWords = 16;

struct DecodeArgs {
  const uint8_t* q;            // bf16 [B, R, 576]
  const uint8_t* kv;           // bf16 [num_pages, 64, 576]
  const int32_t* block_table;  // [B, bt_stride]
  const int32_t* seqlens;      // [B]
  uint16_t* out;               // bf16 [B, R, 512]
  float* lse;                  // [B, R]
  int32_t* meta;               // plan, or nullptr (one workgroup per sequence)
  uint16_t* ws_hi;             // split partials: normalised output rounded to bf16 [slots, rows_per_wg, 512]
  uint16_t* ws_lo;             // bf16(output - hi) [slots, rows_per_wg, 512], written for flagged quarters only
  float* ws_lse;               // partial (log-sum-exp, 1 / row sum) [slots, rows_per_wg, 2]
  uint32_t* ws_lo_mask;        // low-half flags [slots, kLoMaskWords]
  const float* sinks;          // attention-sink logits [heads], or nullptr
  const int32_t* sparse_rows;  // sparse: pool rows per unit [units, row_stride], or nullptr
  int sparse_stride;           // row_stride of sparse_rows (a multiple of 64)
  float scale_log2;            // scale * log2(e)
  int batch, rows, q_len, heads, causal, num_pages, bt_stride, max_blocks;
  int rows_per_wg, row_split;
  // plan_in_decode: every workgroup re-plans from seqlens with the plan's settings
  int plan_in_decode, plan_min_blocks, plan_max_partials, plan_fixed_blocks, plan_split_rule, plan_seg_cost,
      plan_uniform_len;
};

struct CombineArgs {
  const int32_t* meta;
  const uint16_t* ws_hi;       // partial outputs, high halves (bf16)
  const uint16_t* ws_lo;       // low halves, read where ws_lo_mask has the quarter's bit
  const float* ws_lse;
  const uint32_t* ws_lo_mask;
  uint16_t* out;    // bf16 [B, R, 512]
  float* lse;       // [B, R]
  const float* sinks;  // attention-sink logits [heads], or nullptr
  int batch, rows, rows_per_wg, row_split, heads;
  int grouped;         // 1: the grouped form (units of 8 or more partials)
};

// Sparse lists -> pool rows (one workgroup per (b, t) unit).
struct SparseArgs {
  const int32_t* indices;      // [units, topk] token positions, -1 = unused
  const int32_t* seqlens;      // [B] cached tokens per sequence
  const int32_t* block_table;  // [B, bt_stride]
  int32_t* rows;               // out: [units, row_stride] pool rows, kept entries first
  int32_t* lens;               // out: [units] kept entries, or -1 for a bad list
  int units, q_len, topk, row_stride, bt_stride, max_blocks, num_pages;
};

struct F32Args {
  const float* q;              // [B, R, 576]
  const float* kv;             // [num_pages, 64, 576]
  const int32_t* block_table;  // [B, bt_stride]
  const int32_t* seqlens;      // [B]
  float* out;                  // [B, R, 512]
  float* lse;                  // [B, R]
  const float* sinks;          // attention-sink logits [heads], or nullptr
  int32_t* err;                // a plan's device-side fault word, or nullptr
  float scale;
  int batch, rows, q_len, heads, causal, num_pages, bt_stride, max_blocks;
};

}  // namespace mla

// Internal launchers: not part of the exported ABI.
#define MLA_INTERNAL __attribute__((visibility("hidden")))

extern "C" MLA_INTERNAL hipError_t mla_launch_plan(const int32_t* seqlens, int32_t* meta, int batch, int rows,
                                      int row_split, int grid_wg, int min_blocks, int max_blocks,
                                      int max_partials, int fixed_blocks, int split_rule, int seg_cost,
                                      int uniform_len, hipStream_t stream);
// start/stop: events recorded at the kernel's own start and end (both null: a plain launch)
extern "C" MLA_INTERNAL hipError_t mla_launch_decode_bf16(const mla::DecodeArgs* args, int grid, hipStream_t stream,
                                                       hipEvent_t start, hipEvent_t stop);
extern "C" MLA_INTERNAL hipError_t mla_launch_combine(const mla::CombineArgs* args, hipStream_t stream);
extern "C" MLA_INTERNAL hipError_t mla_launch_decode_f32(const mla::F32Args* args, hipStream_t stream);
extern "C" MLA_INTERNAL hipError_t mla_launch_sparse_rows(const mla::SparseArgs* args, hipStream_t stream);

// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MLA_LDS __attribute__((address_space(3)))

namespace mla {

constexpr int kDqk = 576;                 // cache row: 512 latent + 64 rope
constexpr int kDv = 512;                  // value width (first 512 dims of a row)
constexpr int kPage = 64;                 // tokens per page = tokens per KV block
constexpr int kRowBytes = kDqk * 2;       // one bf16 cache row: 1152 B = 72 chunks of 16 B
constexpr int kChunksPerRow = kRowBytes / 16;
constexpr int kBlockBytes = kPage * kRowBytes;   // 73728 B per bf16 page
constexpr int kLoadsPerBlock = kBlockBytes / 1024;  // 72 wave-wide 16 B/lane loads
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---- plan (metadata) layout, int32 words --------------------------------------------
// header
constexpr int kMetaMagic = 0x4D4C4150;    // 'MLAP'
enum MetaHdr {
  kHdrMagic = 0,
  kHdrBatch = 1,
  kHdrRows = 2,          // rows per sequence R = q_len * heads
  kHdrRowSplit = 3,      // workgroups sharing one sequence's rows
  kHdrRowsPerWg = 4,
  kHdrNumWg = 5,         // workgroups that have work (device-computed)
  kHdrGridWg = 6,        // workgroups launched (host-known upper bound)
  kHdrTotal = 7,         // total 64-token blocks over all units
  kHdrNumPartials = 8,   // partial slots used
  kHdrError = 9,         // device-side input fault flag
  kHdrMaxPartials = 10,  // partial slot capacity of the workspace
  kHdrMaxBlocks = 11,    // max_blocks_per_seq the plan was made for
  kHdrRule = 12,         // partition rule used (PlanRule)
  kHdrCostPages = 13,    // busiest workgroup's cost under the pages rule (auto only)
  kHdrCostBalanced = 14, // ... under the cost rule (auto only)
  kHdrSegCost = 15,      // per-segment overhead of the cost model, quarter blocks
  kHdrWords = 16,
};
// Partition rules of the planner (the split_rule option; the header's kHdrRule).
enum PlanRule { kRuleAuto = 0, kRulePages = 1, kRuleCost = 2, kRuleFixed = 3 };
// arrays follow the header: cu_blocks[B+1], num_splits[U], first_wg[U], part_off[U],
// wg_begin[grid+1], wg_seq[grid], with U = B * row_split units (unit u = b * row_split + g).
// wg_seq[w] is the sequence holding workgroup w's first block (0 past the workgroups with
// work), so a decode workgroup finds its first segment without a search.
struct MetaView {
  int32_t* hdr;
  int32_t* cu_blocks;
  int32_t* num_splits;
  int32_t* first_wg;
  int32_t* part_off;
  int32_t* wg_begin;
};
__host__ __device__ inline size_t meta_words(int batch, int row_split, int grid_wg) {
  const size_t units = (size_t)batch * row_split;
  return kHdrWords + (size_t)(batch + 1) + 3 * units + 2 * (size_t)grid_wg + 1;
}
// wg_seq of a plan made for grid_wg workgroups (after wg_begin's grid_wg + 1 words)
__host__ __device__ inline int32_t* meta_wg_seq(const MetaView& v, int grid_wg) { return v.wg_begin + grid_wg + 1; }
__host__ __device__ inline MetaView meta_view(int32_t* base, int batch, int row_split) {
  MetaView v;
  const size_t units = (size_t)batch * row_split;
  v.hdr = base;
  v.cu_blocks = base + kHdrWords;
  v.num_splits = v.cu_blocks + batch + 1;
  v.first_wg = v.num_splits + units;
  v.part_off = v.first_wg + units;
  v.wg_begin = v.part_off + units;
  return v;
}

// ---- small device utilities ---------------------------------------------------------
// Read-only kernel inputs (block tables, sequence lengths, the plan) are read through the
// constant address space so uniform reads become scalar loads.
#define MLA_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, size_t i) {
  return ((const MLA_CONST T*)p)[i];
}
// Index of this wave in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ inline float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
// max of v over lanes l and l ^ 32, in VALU (gfx950's lane-half swap): no LDS access, so
// it adds nothing to the LDS wait counter.  After the swap of v with itself, the first
// result holds the low half's values in both halves and the second the high half's.
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Two floats -> a packed bf16 pair (lo in bits 0-15), round to nearest even, NaN kept
// NaN: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// Workgroup barrier for communication through LDS only: it orders LDS accesses and
// does not wait for global stores in flight (__syncthreads also waits for those).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block-wide exclusive scan of one value per thread (256 threads = 4 waves): a scan
// inside each wave, then the wave totals through LDS.  Returns the exclusive prefix and
// writes the block total to *total.
// Inclusive sum over a wave's 64 lanes with DPP moves (no LDS): shifts by 1, 2, 4 and 8
// inside each 16-lane row, then the last lane of row 0 into row 1 and of row 2 into row 3,
// then lane 31 into rows 2 and 3.  Lanes with no source add 0.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

__device__ inline int32_t block_exclusive_scan(int32_t v, int32_t* s, int32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int32_t x = wave_inclusive_sum(v);
  if (lane == 63) s[wv] = x;
  lds_barrier();
  int32_t base = 0;
  for (int k = 0; k < wv; ++k) base += s[k];
  *total = s[0] + s[1] + s[2] + s[3];
  lds_barrier();  // s is reused by the next scan
  return base + x - v;
}

// Attention sink folded into one row's softmax statistics: m = the row's shift, l = sum
// over its keys of exp(s - m) (0: no key), sink = the sink logit, all in the units of
// the exponential (base 2 or e, per Base2).  The sink is one more softmax term with a
// zero value row, so the denominator becomes l*exp(m) + exp(sink).  Returns the factor
// that maps the unnormalised output sum (taken with shift m) to the final output, and
// the log of the denominator.  Both terms are taken relative to max(m, sink), so
// neither overflows; sink = -inf gives exactly 1/l and m + log(l), as without a sink.
struct SinkFold {
  float scale_o, lse;
};
template <bool Base2>
__device__ inline SinkFold fold_sink(float m, float l, float sink) {
  if (l == 0.f) return {0.f, sink};                  // no key: out 0, lse = the sink
  const float mx = fmaxf(m, sink);                   // NaN sink: c below is NaN
  const float a = Base2 ? __builtin_amdgcn_exp2f(m - mx) : expf(m - mx);
  const float c = Base2 ? __builtin_amdgcn_exp2f(sink - mx) : expf(sink - mx);
  const float den = fmaf(l, a, c);
  return {a / den, mx + (Base2 ? __log2f(den) : logf(den))};
}

}  // namespace mla

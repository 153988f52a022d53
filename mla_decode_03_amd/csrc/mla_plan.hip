// Split planner for MLA decode (the kernel behind mla_get_metadata).
//
// Every sequence b contributes row_split "units" (one per slice of its rows), each
// holding nblk_b = ceil(L_b / 64) KV blocks.  Units are laid end to end (sequence-
// major) and the concatenated block range [0, total) is cut into num_wg contiguous
// workgroup ranges.  A unit cut across k > 1 workgroups gets k partial results,
// merged later by log-sum-exp; their slots are numbered unit by unit.
//
// Two ways to cut, ranked by a cost model in the spirit of the TileLang notes' tile
// recommender ("Key design 2: tile recommendation": time is traffic over bandwidth,
// and candidate configurations are ranked by it):
//   pages rule  equal block shares [floor(w*total/num_wg), floor((w+1)*total/num_wg));
//   cost rule   equal shares of a cost axis on which each non-empty unit first takes
//               `seg_cost` quarter-blocks (the traffic a segment adds besides its KV
//               blocks: its Q rows and its output or partial rows) and then 4 quarters
//               per block.  A cut in a unit's overhead moves to its first block, one
//               inside its blocks rounds down to a block.
// A workgroup's cost is 4 per block it streams plus seg_cost per unit it touches; the
// planner keeps the rule whose busiest workgroup costs less (the pages rule on a tie,
// so evenly sized batches keep their cut).  Deterministic, integer only.
#include "mla_plan_core.h"

namespace mla {

template <bool CU_IN_LDS>
__global__ __launch_bounds__(256) void mla_plan_kernel(const int32_t* __restrict__ seqlens,
                                                       int32_t* __restrict__ meta, int batch,
                                                       int rows, int row_split, int grid_wg,
                                                       int min_blocks, int max_blocks,
                                                       int max_partials, int fixed_blocks,
                                                       int split_rule, int seg_cost, int uniform_len) {
  __shared__ int32_t s_scan[256];
  __shared__ int32_t s_cu[kPlanLdsBatch + 1];   // cu_blocks, when the batch fits
  __shared__ int32_t s_ne[kPlanLdsBatch + 1];   // non-empty sequences before b, likewise
  __shared__ int64_t s_red[4];
  __shared__ int32_t s_bp[kPlanLdsWg + 1], s_bc[kPlanLdsWg + 1];   // the two rules' cuts
  __shared__ int32_t s_err, s_share[kShareWords];
  const PlanParams p{seqlens, batch, rows, row_split, grid_wg, min_blocks, max_blocks, max_partials, fixed_blocks,
                     split_rule, seg_cost, uniform_len};
  const PlanLds L{s_scan, s_cu, s_ne, s_red, s_bp, s_bc, &s_err, s_share};
  plan_core<CU_IN_LDS>(p, L, meta_view(meta, batch, row_split), true, -1);
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_plan(const int32_t* seqlens, int32_t* meta, int batch, int rows,
                                      int row_split, int grid_wg, int min_blocks, int max_blocks,
                                      int max_partials, int fixed_blocks, int split_rule, int seg_cost,
                                      int uniform_len, hipStream_t stream) {
  if (batch <= mla::kPlanLdsBatch)
    hipLaunchKernelGGL(mla::mla_plan_kernel<true>, dim3(1), dim3(256), 0, stream, seqlens, meta, batch,
                       rows, row_split, grid_wg, min_blocks, max_blocks, max_partials, fixed_blocks,
                       split_rule, seg_cost, uniform_len);
  else
    hipLaunchKernelGGL(mla::mla_plan_kernel<false>, dim3(1), dim3(256), 0, stream, seqlens, meta, batch,
                       rows, row_split, grid_wg, min_blocks, max_blocks, max_partials, fixed_blocks,
                       split_rule, seg_cost, uniform_len);
  return hipGetLastError();
}

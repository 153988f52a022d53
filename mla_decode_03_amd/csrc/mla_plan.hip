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
#include "mla_args.h"
#include "mla_device.h"

namespace mla {

constexpr int kPlanLdsBatch = 4095;   // batches up to this size keep cu_blocks in LDS
constexpr int kPlanLdsWg = 1024;      // plans up to this many workgroups keep both cuts in LDS

// Block-wide maximum of one int64 per thread (256 threads); every thread gets it.
__device__ inline int64_t block_max(int64_t x, int64_t* s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int64_t y = __shfl_xor(x, off, 64);
    x = x > y ? x : y;
  }
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  lds_barrier();
  const int64_t r = max(max(s[0], s[1]), max(s[2], s[3]));
  lds_barrier();  // s is reused by the next call
  return r;
}

// floor(n / d) for 0 <= n < 2^53, 0 < d < 2^31: a double quotient, corrected to the
// exact integer (the rounded quotient is off by at most one).
__device__ inline int64_t floor_div(int64_t n, int64_t d) {
  int64_t q = (int64_t)((double)n / (double)d);
  if (q * d > n) --q;
  else if ((q + 1) * d <= n) ++q;
  return q;
}

// Workgroup holding global block position x (0 <= x < total): the largest w < num_wg
// with floor(w*total/num_wg) <= x.
__device__ inline int32_t wg_of(int64_t x, int64_t total, int64_t num_wg) {
  return (int32_t)floor_div((x + 1) * num_wg - 1, total);
}

// CU_IN_LDS: the batch fits kPlanLdsBatch, so cu_blocks and the non-empty prefix are kept
// in LDS (a compile-time choice: selecting the array at run time made every read a generic
// load that waits on both LDS and global memory).
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
  const int t = threadIdx.x;
  constexpr bool cu_in_lds = CU_IN_LDS;
  MetaView v = meta_view(meta, batch, row_split);
  // Larger batches keep the non-empty prefix in first_wg (rewritten by the unit pass).
  int32_t* ne_glob = v.first_wg;
  // wg_seq[w]: the sequence holding workgroup w's first block (0 past the workgroups with work)
  int32_t* wg_seq = meta_wg_seq(v, grid_wg);
  int err = 0;

  // 1. blocks per sequence and their prefix sums; non-empty sequences before each; the
  // largest sequence
  int32_t carry = 0, ne_carry = 0;
  int64_t nb_max = 0;
  for (int base = 0; base < batch; base += 256) {
    const int b = base + t;
    int32_t nb = 0;
    if (b < batch) {
      int64_t L = uniform_len > 0 ? uniform_len : seqlens[b];   // sparse: every unit holds topk
      if (L < 0) { L = 0; err = 1; }
      int64_t n = (L + kPage - 1) / kPage;
      if (n > max_blocks) { n = max_blocks; err = 1; }
      nb = (int32_t)n;
      nb_max = max<int64_t>(nb_max, n);
    }
    int32_t tot, ntot;
    const int32_t excl = block_exclusive_scan(nb, s_scan, &tot);
    const int32_t nexcl = block_exclusive_scan(nb > 0 ? 1 : 0, s_scan, &ntot);
    if (b < batch) {
      v.cu_blocks[b] = carry + excl;
      if (cu_in_lds) {
        s_cu[b] = carry + excl;
        s_ne[b] = ne_carry + nexcl;
      } else {
        ne_glob[b] = ne_carry + nexcl;
      }
    }
    carry += tot;
    ne_carry += ntot;
  }
  if (t == 0) {
    v.cu_blocks[batch] = carry;
    if (cu_in_lds) {
      s_cu[batch] = carry;
      s_ne[batch] = ne_carry;
    }
  }
  // cu_blocks and the non-empty prefix visible to the whole workgroup.  Larger batches
  // read them back from global memory, so their stores must have landed; batches that fit
  // keep them in LDS, and the barrier need not wait for the stores.
  if constexpr (!cu_in_lds) {
    __threadfence_block();
    __syncthreads();
  } else {
    lds_barrier();
  }

  const int64_t total = (int64_t)row_split * carry;
  const int units = batch * row_split;
  int64_t num_wg = 0;
  int32_t pcarry = 0;
  bool use_cost = false;
  if (fixed_blocks > 0) {
    // Batch-invariant plan: every unit cut into chunks of fixed_blocks blocks from its own
    // start, one chunk per workgroup, in unit order.
    int32_t ccarry = 0;
    for (int base = 0; base < units; base += 256) {
      const int u = base + t;
      int32_t ns = 0;
      int64_t ustart = 0;
      if (u < units) {
        const int b = u / row_split, g = u % row_split;
        const int32_t cb0 = cu_in_lds ? s_cu[b] : v.cu_blocks[b];
        const int32_t cb1 = cu_in_lds ? s_cu[b + 1] : v.cu_blocks[b + 1];
        const int32_t nb = cb1 - cb0;
        ustart = (int64_t)row_split * cb0 + (int64_t)g * nb;
        ns = (nb + fixed_blocks - 1) / fixed_blocks;
      }
      int32_t ctot, ptot;
      const int32_t first = ccarry + block_exclusive_scan(ns, s_scan, &ctot);
      const int32_t poff = pcarry + block_exclusive_scan(ns > 1 ? ns : 0, s_scan, &ptot);
      if (u < units) {
        v.num_splits[u] = ns;
        v.first_wg[u] = ns > 0 ? first : -1;
        v.part_off[u] = poff;
        for (int k = 0; k < ns; ++k)
          if (first + k < grid_wg) {
            v.wg_begin[first + k] = (int32_t)(ustart + (int64_t)k * fixed_blocks);
            wg_seq[first + k] = u / row_split;
          }
      }
      ccarry += ctot;
      pcarry += ptot;
    }
    num_wg = ccarry;
    if (num_wg > grid_wg) err = 1;   // cannot happen when grid_wg covers max_blocks
    for (int w = (int)min<int64_t>(num_wg, grid_wg) + t; w <= grid_wg; w += 256) {
      v.wg_begin[w] = (int32_t)total;
      if (w < grid_wg) wg_seq[w] = 0;
    }
  } else {
    if (total > 0) {
      num_wg = (total + min_blocks - 1) / min_blocks;
      if (num_wg > grid_wg) num_wg = grid_wg;
      if (num_wg < 1) num_wg = 1;
    }
    const int rs = row_split;
    const int64_t c = seg_cost;
    const int64_t ctot = 4 * total + c * rs * (int64_t)ne_carry;   // length of the cost axis
    auto cu_at = [&](int b) -> int64_t { return cu_in_lds ? s_cu[b] : v.cu_blocks[b]; };
    auto ne_at = [&](int b) -> int64_t { return cu_in_lds ? s_ne[b] : (b < batch ? ne_glob[b] : ne_carry); };
    auto cost_at = [&](int b) -> int64_t { return 4 * rs * cu_at(b) + c * rs * ne_at(b); };
    // sequence holding block position p < total: the largest b with rs * cu[b] <= p
    auto seq_of_block = [&](int64_t p) -> int {
      int lo = 0, hi = batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rs * cu_at(mid) <= p) lo = mid; else hi = mid - 1;
      }
      return lo;
    };
    // sequence holding cost position x < ctot: the largest b with cost_at(b) <= x
    auto seq_of_cost = [&](int64_t x) -> int {
      int lo = 0, hi = batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cost_at(mid) <= x) lo = mid; else hi = mid - 1;
      }
      return lo;
    };
    // cost rule: block position of the cut at cost position x
    auto block_at = [&](int64_t x) -> int64_t {
      if (x >= ctot) return total;
      const int b = seq_of_cost(x);
      const int64_t nb = cu_at(b + 1) - cu_at(b);
      const int64_t ucost = c + 4 * nb;
      const int64_t g = rs == 1 ? 0 : floor_div(x - cost_at(b), ucost);
      const int64_t off = x - cost_at(b) - g * ucost;
      return rs * cu_at(b) + g * nb + (off < c ? 0 : (off - c) >> 2);
    };
    // rank of the unit holding block p among the non-empty units
    auto rank_of_block = [&](int64_t p) -> int64_t {
      const int b = seq_of_block(p);
      const int64_t nb = cu_at(b + 1) - cu_at(b);
      return rs * ne_at(b) + (rs == 1 ? 0 : floor_div(p - rs * cu_at(b), nb));
    };
    auto pages_begin = [&](int64_t w) -> int64_t { return floor_div(w * total, num_wg); };
    auto cost_begin = [&](int64_t w) -> int64_t { return block_at(floor_div(w * ctot, num_wg)); };
    auto range_cost = [&](int64_t lo, int64_t hi) -> int64_t {
      return hi > lo ? 4 * (hi - lo) + c * (rank_of_block(hi - 1) - rank_of_block(lo) + 1) : 0;
    };

    // 2. the busiest workgroup under each rule; keep the cheaper rule.  When every
    // non-empty unit holds the same nb blocks and the equal shares line up with the
    // units (share a multiple of nb, or nb of share), every workgroup of the pages rule
    // costs exactly the average, which no cut's busiest workgroup can beat: keep it
    // without evaluating.  Otherwise each cut is computed once (kept in LDS when the plan
    // fits).
    int64_t worst_p = 0, worst_c = 0;
    bool evaluate = split_rule == kRuleAuto && num_wg > 0;
    if (evaluate) {
      const int64_t nbm = block_max(nb_max, s_red);
      const int64_t share = total / num_wg;
      if ((int64_t)carry == nbm * ne_carry && share * num_wg == total && nbm > 0 &&
          (share % nbm == 0 || nbm % share == 0))
        evaluate = false;
    }
    const bool cuts_in_lds = evaluate && num_wg <= kPlanLdsWg;
    if (cuts_in_lds) {
      for (int w = t; w <= num_wg; w += 256) {
        s_bp[w] = (int32_t)pages_begin(w);
        s_bc[w] = (int32_t)cost_begin(w);
      }
      lds_barrier();
    }
    auto cut_p = [&](int64_t w) -> int64_t { return cuts_in_lds ? s_bp[w] : pages_begin(w); };
    auto cut_c = [&](int64_t w) -> int64_t { return cuts_in_lds ? s_bc[w] : cost_begin(w); };
    if (evaluate) {
      for (int64_t w = t; w < num_wg; w += 256) {
        worst_p = max(worst_p, range_cost(cut_p(w), cut_p(w + 1)));
        worst_c = max(worst_c, range_cost(cut_c(w), cut_c(w + 1)));
      }
      worst_p = block_max(worst_p, s_red);
      worst_c = block_max(worst_c, s_red);
    }
    use_cost = split_rule == kRuleCost || (split_rule == kRuleAuto && worst_c < worst_p);
    if (t == 0) {
      v.hdr[kHdrCostPages] = (int32_t)min<int64_t>(worst_p, INT32_MAX);
      v.hdr[kHdrCostBalanced] = (int32_t)min<int64_t>(worst_c, INT32_MAX);
    }

    // 3. workgroup ranges, and the sequence holding each one's first block
    for (int w = t; w <= grid_wg; w += 256) {
      const int64_t begin = (w <= num_wg && num_wg > 0) ? (use_cost ? cut_c(w) : cut_p(w)) : total;
      v.wg_begin[w] = (int32_t)begin;
      if (w < grid_wg) wg_seq[w] = (w < num_wg && begin < total) ? seq_of_block(begin) : 0;
    }
    // workgroup holding block p: the largest w < num_wg whose range starts at or before p.
    // Cost rule: a cut at cost x lands at or before p exactly when x < Y, Y = the cost
    // position just past block p, so the answer is the largest w with w*ctot < Y*num_wg.
    auto holder = [&](int64_t p) -> int32_t {
      if (!use_cost) return wg_of(p, total, num_wg);
      const int b = seq_of_block(p);
      const int64_t nb = cu_at(b + 1) - cu_at(b);
      const int64_t g = rs == 1 ? 0 : floor_div(p - rs * cu_at(b), nb);
      const int64_t y = cost_at(b) + g * (c + 4 * nb) + c + 4 * (p - rs * cu_at(b) - g * nb) + 4;
      return (int32_t)min<int64_t>(floor_div(y * num_wg - 1, ctot), num_wg - 1);
    };
    // 4. units: which workgroups cover each, and the partial slots of the split ones.
    auto unit_span = [&](int u, int32_t& first) -> int32_t {
      const int b = u / rs, g = u % rs;
      const int64_t nb = cu_at(b + 1) - cu_at(b);
      first = -1;
      if (nb == 0) return 0;
      const int64_t start = rs * cu_at(b) + g * nb;
      first = holder(start);
      return holder(start + nb - 1) - first + 1;
    };
    if (cu_in_lds) {
      for (int base = 0; base < units; base += 256) {
        const int u = base + t;
        int32_t ns = 0, first = -1;
        if (u < units) {
          ns = unit_span(u, first);
          v.num_splits[u] = ns;
          v.first_wg[u] = first;
        }
        int32_t tot;
        const int32_t excl = block_exclusive_scan(ns > 1 ? ns : 0, s_scan, &tot);
        if (u < units) v.part_off[u] = pcarry + excl;
        pcarry += tot;
      }
    } else {
      // first_wg still holds the non-empty prefix: first every unit's span (the first
      // workgroup waits in part_off) ...
      for (int u = t; u < units; u += 256) {
        int32_t first;
        v.num_splits[u] = unit_span(u, first);
        v.part_off[u] = first;
      }
      __threadfence_block();
      __syncthreads();
      // ... then, each unit by the thread that wrote it, the slots.
      for (int base = 0; base < units; base += 256) {
        const int u = base + t;
        int32_t ns = 0;
        if (u < units) {
          ns = v.num_splits[u];
          v.first_wg[u] = v.part_off[u];
        }
        int32_t tot;
        const int32_t excl = block_exclusive_scan(ns > 1 ? ns : 0, s_scan, &tot);
        if (u < units) v.part_off[u] = pcarry + excl;
        pcarry += tot;
      }
    }
  }

  // 4. header (the error flag is the OR over threads)
  __shared__ int32_t s_err;
  if (t == 0) s_err = 0;
  lds_barrier();
  if (err) atomicOr(&s_err, 1);
  lds_barrier();
  if (t == 0) {
    v.hdr[kHdrMagic] = kMetaMagic;
    v.hdr[kHdrBatch] = batch;
    v.hdr[kHdrRows] = rows;
    v.hdr[kHdrRowSplit] = row_split;
    v.hdr[kHdrRowsPerWg] = rows / row_split;
    v.hdr[kHdrNumWg] = (int32_t)num_wg;
    v.hdr[kHdrGridWg] = grid_wg;
    v.hdr[kHdrTotal] = (int32_t)total;
    v.hdr[kHdrNumPartials] = pcarry;
    v.hdr[kHdrError] = (s_err || pcarry > max_partials) ? 1 : 0;
    v.hdr[kHdrMaxPartials] = max_partials;
    v.hdr[kHdrMaxBlocks] = max_blocks;
    v.hdr[kHdrRule] = fixed_blocks > 0 ? kRuleFixed : (use_cost ? kRuleCost : kRulePages);
    v.hdr[kHdrSegCost] = fixed_blocks > 0 ? 0 : seg_cost;
    if (fixed_blocks > 0) {
      v.hdr[kHdrCostPages] = 0;
      v.hdr[kHdrCostBalanced] = 0;
    }
    if (pcarry > max_partials || num_wg > grid_wg) v.hdr[kHdrNumWg] = 0;  // refuse to run a plan that overflows
  }
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

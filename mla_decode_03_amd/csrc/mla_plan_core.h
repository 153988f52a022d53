// The split planner's computation, shared by the planner kernel and by decode launches
// that plan for themselves (every decode workgroup runs it on the current lengths, and
// takes its own share of the plan from LDS).
#pragma once
#include "mla_args.h"
#include "mla_device.h"

namespace mla {

constexpr int kPlanLdsBatch = 4095;   // batches up to this size keep cu_blocks in LDS
constexpr int kPlanLdsWg = 1024;      // plans up to this many workgroups keep both cuts in LDS

// Wave-wide maximum of one non-negative int32 per lane, in every lane: an inclusive
// max-scan with DPP moves (lanes with no source take 0), lane 63 read.
__device__ inline int32_t wave_max_nonneg(int32_t x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));   // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));   // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));   // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));   // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

// Block-wide maximum of one non-negative int32 per thread (256 threads); every thread gets
// it: the wave's maximum, then the four waves' through LDS.
__device__ inline int32_t block_max_nonneg(int32_t x, int64_t* s) {
  x = wave_max_nonneg(x);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  lds_barrier();
  const int64_t r = max(max(s[0], s[1]), max(s[2], s[3]));
  lds_barrier();  // s is reused by the next call
  return (int32_t)r;
}

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
  if (((n | d) >> 31) == 0) return (int64_t)((uint32_t)n / (uint32_t)d);   // both under 2^31
  int64_t q = (int64_t)((double)n / (double)d);
  if (q * d > n) --q;
  else if ((q + 1) * d <= n) ++q;
  return q;
}

// floor(n / d) of wave-uniform operands, divided by the vector unit: for uniform values the
// compiler divides on the scalar unit, whose sequence takes several times the cycles (one
// scalar unit serves the workgroup's four waves).  Operands of 2^31 or more go through
// floor_div.
__device__ inline int64_t floor_div_uniform(int64_t n, int64_t d) {
  if (((n | d) >> 31) != 0) return floor_div(n, d);
  uint32_t nv = (uint32_t)n, dv = (uint32_t)d;
  asm volatile("" : "+v"(nv), "+v"(dv));
  return (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(nv / dv));
}

// Workgroup holding global block position x (0 <= x < total): the largest w < num_wg
// with floor(w*total/num_wg) <= x.
__device__ inline int32_t wg_of(int64_t x, int64_t total, int64_t num_wg) {
  return (int32_t)floor_div((x + 1) * num_wg - 1, total);
}

// One workgroup's share of a plan, as plan_core leaves it in LDS (int32 words): its block
// range [pos, end), the units of its first and last blocks with each one's split count,
// first workgroup and partial-slot offset, the first unit's start and block count, the
// number of workgroups with work (0: the plan overflows and must not run), the input-fault
// flag.
enum ShareWord {
  kSharePos = 0, kShareEnd, kShareUFirst, kShareNsFirst, kShareFirstWgFirst, kSharePoffFirst,
  kShareULast, kShareNsLast, kShareFirstWgLast, kSharePoffLast, kShareNumWg, kShareErr,
  kShareStartFirst, kShareNbFirst, kShareWords
};

struct PlanParams {
  const int32_t* seqlens;
  int batch, rows, row_split, grid_wg, min_blocks, max_blocks, max_partials, fixed_blocks, split_rule,
      seg_cost, uniform_len;
};

// LDS the computation uses: scan[256], cu[kPlanLdsBatch + 1], ne[kPlanLdsBatch + 1], red[4],
// bp[kPlanLdsWg + 1], bc[kPlanLdsWg + 1], err[1], share[kShareWords].
struct PlanLds {
  int32_t* scan;
  int32_t* cu;
  int32_t* ne;
  int64_t* red;
  int32_t* bp;
  int32_t* bc;
  int32_t* err;
  int32_t* share;
};
constexpr int kPlanLdsBytes = 4 * (256 + 2 * (kPlanLdsBatch + 1) + 2 * (kPlanLdsWg + 1) + 1 + kShareWords) + 8 * 4 + 64;

// The whole plan for 256 threads.  write: store it into v (the planner kernel; in a decode
// launch, one workgroup); my_wg >= 0: also leave that workgroup's share in L.share.
// Batches over kPlanLdsBatch (CU_IN_LDS false) use the plan's arrays as scratch and must
// write.
template <bool CU_IN_LDS>
__device__ inline void plan_core(const PlanParams& p, const PlanLds& L, MetaView v, bool write, int my_wg) {
  const int t = threadIdx.x;
  constexpr bool cu_in_lds = CU_IN_LDS;
  const int32_t* seqlens = p.seqlens;
  const int batch = p.batch, rows = p.rows, row_split = p.row_split, grid_wg = p.grid_wg;
  const int min_blocks = p.min_blocks, max_blocks = p.max_blocks, max_partials = p.max_partials;
  const int fixed_blocks = p.fixed_blocks, split_rule = p.split_rule, seg_cost = p.seg_cost;
  const int uniform_len = p.uniform_len;
  // global stores: the whole plan, or (a decode workgroup that is not the writer) none;
  // larger batches use the plan's own arrays as scratch, so they always write
  const bool wr = write || !cu_in_lds;
  int32_t* s_scan = L.scan;
  int32_t* s_cu = L.cu;
  int32_t* s_ne = L.ne;
  int64_t* s_red = L.red;
  int32_t* s_bp = L.bp;
  int32_t* s_bc = L.bc;
  int32_t* s_share = L.share;
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
      if (wr) v.cu_blocks[b] = carry + excl;
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
    if (wr) v.cu_blocks[batch] = carry;
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
    if (my_wg >= 0 && t == 0) {   // no chunk of mine until a unit claims it
      s_share[kSharePos] = 0;
      s_share[kShareEnd] = 0;
      s_share[kShareUFirst] = -1;
      s_share[kShareULast] = -1;
    }
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
        if (wr) {
          v.num_splits[u] = ns;
          v.first_wg[u] = ns > 0 ? first : -1;
          v.part_off[u] = poff;
          for (int k = 0; k < ns; ++k)
            if (first + k < grid_wg) {
              v.wg_begin[first + k] = (int32_t)(ustart + (int64_t)k * fixed_blocks);
              wg_seq[first + k] = u / row_split;
            }
        }
        if (my_wg >= first && my_wg < first + ns) {   // my chunk: unit u, chunk my_wg - first
          const int64_t pos = ustart + (int64_t)(my_wg - first) * fixed_blocks;
          const int64_t nbu = (cu_in_lds ? s_cu[u / row_split + 1] : v.cu_blocks[u / row_split + 1]) -
                              (cu_in_lds ? s_cu[u / row_split] : v.cu_blocks[u / row_split]);
          const int32_t sh[14] = {(int32_t)pos, (int32_t)min<int64_t>(pos + fixed_blocks, ustart + nbu), u, ns, first,
                                  poff, u, ns, first, poff, 0, 0, (int32_t)ustart, (int32_t)nbu};
          for (int k = 0; k < 14; ++k) if (k != kShareNumWg && k != kShareErr) s_share[k] = sh[k];
        }
      }
      ccarry += ctot;
      pcarry += ptot;
    }
    num_wg = ccarry;
    if (num_wg > grid_wg) err = 1;   // cannot happen when grid_wg covers max_blocks
    if (wr)
      for (int w = (int)min<int64_t>(num_wg, grid_wg) + t; w <= grid_wg; w += 256) {
        v.wg_begin[w] = (int32_t)total;
        if (w < grid_wg) wg_seq[w] = 0;
      }
  } else {
    if (total > 0) {
      num_wg = floor_div(total + min_blocks - 1, min_blocks);
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
      const int64_t nbm = block_max_nonneg((int32_t)nb_max, s_red);   // nb_max <= max_blocks
      const int64_t share = floor_div(total, num_wg);
      if ((int64_t)carry == nbm * ne_carry && share * num_wg == total && nbm > 0 &&
          (share == floor_div(share, nbm) * nbm || nbm == floor_div(nbm, share) * share))
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
    if (wr && t == 0) {
      v.hdr[kHdrCostPages] = (int32_t)min<int64_t>(worst_p, INT32_MAX);
      v.hdr[kHdrCostBalanced] = (int32_t)min<int64_t>(worst_c, INT32_MAX);
    }

    // 3. workgroup ranges, and the sequence holding each one's first block
    if (wr)
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
    // my workgroup's range and the units of its first and last blocks (uniform values)
    int64_t my_pos = total, my_end = total;
    int u_first = -1, u_last = -1;
    if (my_wg >= 0 && my_wg < num_wg) {
      my_pos = use_cost ? cut_c(my_wg) : cut_p(my_wg);
      my_end = use_cost ? cut_c(my_wg + 1) : cut_p(my_wg + 1);
    }
    if (my_pos < my_end) {   // (uniform) the sequences of both ends counted over the block:
      // the largest b with rs * cu[b] <= q is the count of such b, less one
      int32_t cnt = 0;
      for (int b = t; b < batch; b += 256) {
        const int64_t cb = rs * cu_at(b);
        cnt += (cb <= my_pos ? 1 : 0) + (cb <= my_end - 1 ? 1 << 16 : 0);
      }
      int32_t tot;
      block_exclusive_scan(cnt, s_scan, &tot);
      const int bf = (tot & 0xffff) - 1, bl = (tot >> 16) - 1;
      auto unit_in = [&](int b, int64_t q) -> int {
        const int64_t nb = cu_at(b + 1) - cu_at(b);
        return b * rs + (rs == 1 ? 0 : (int)floor_div(q - rs * cu_at(b), nb));
      };
      u_first = unit_in(bf, my_pos);
      u_last = unit_in(bl, my_end - 1);
    }
    if (my_wg >= 0 && t == 0) {
      s_share[kSharePos] = (int32_t)my_pos;
      s_share[kShareEnd] = (int32_t)my_end;
      s_share[kShareUFirst] = u_first;
      s_share[kShareULast] = u_last;
      if (u_first >= 0) {
        const int b = u_first / rs;
        const int64_t nb = cu_at(b + 1) - cu_at(b);
        s_share[kShareStartFirst] = (int32_t)(rs * cu_at(b) + (int64_t)(u_first % rs) * nb);
        s_share[kShareNbFirst] = (int32_t)nb;
      }
    }
    if (cu_in_lds) {
      for (int base = 0; base < units; base += 256) {
        const int u = base + t;
        int32_t ns = 0, first = -1;
        if (u < units) {
          ns = unit_span(u, first);
          if (wr) {
            v.num_splits[u] = ns;
            v.first_wg[u] = first;
          }
        }
        int32_t tot;
        const int32_t excl = block_exclusive_scan(ns > 1 ? ns : 0, s_scan, &tot);
        if (u < units) {
          if (wr) v.part_off[u] = pcarry + excl;
          if (u == u_first) {
            s_share[kShareNsFirst] = ns;
            s_share[kShareFirstWgFirst] = first;
            s_share[kSharePoffFirst] = pcarry + excl;
          }
          if (u == u_last) {
            s_share[kShareNsLast] = ns;
            s_share[kShareFirstWgLast] = first;
            s_share[kSharePoffLast] = pcarry + excl;
          }
        }
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
  int32_t* s_err = L.err;
  if (t == 0) *s_err = 0;
  lds_barrier();
  if (err) atomicOr(s_err, 1);
  lds_barrier();
  const bool refuse = pcarry > max_partials || num_wg > grid_wg;   // a plan that overflows does not run
  if (my_wg >= 0 && t == 0) {
    s_share[kShareNumWg] = refuse ? 0 : (int32_t)num_wg;
    s_share[kShareErr] = (*s_err || pcarry > max_partials) ? 1 : 0;
  }
  if (wr && t == 0) {
    v.hdr[kHdrMagic] = kMetaMagic;
    v.hdr[kHdrBatch] = batch;
    v.hdr[kHdrRows] = rows;
    v.hdr[kHdrRowSplit] = row_split;
    v.hdr[kHdrRowsPerWg] = rows / row_split;
    v.hdr[kHdrNumWg] = (int32_t)num_wg;
    v.hdr[kHdrGridWg] = grid_wg;
    v.hdr[kHdrTotal] = (int32_t)total;
    v.hdr[kHdrNumPartials] = pcarry;
    // inside a decode launch other workgroups may already have raised the flag: only raise it
    if (my_wg < 0) v.hdr[kHdrError] = (*s_err || pcarry > max_partials) ? 1 : 0;
    else if (*s_err || pcarry > max_partials) v.hdr[kHdrError] = 1;
    v.hdr[kHdrMaxPartials] = max_partials;
    v.hdr[kHdrMaxBlocks] = max_blocks;
    v.hdr[kHdrRule] = fixed_blocks > 0 ? kRuleFixed : (use_cost ? kRuleCost : kRulePages);
    v.hdr[kHdrSegCost] = fixed_blocks > 0 ? 0 : seg_cost;
    if (fixed_blocks > 0) {
      v.hdr[kHdrCostPages] = 0;
      v.hdr[kHdrCostBalanced] = 0;
    }
    if (refuse) v.hdr[kHdrNumWg] = 0;  // refuse to run a plan that overflows
  }
  lds_barrier();   // the share words are complete
}


// The common case of a re-planning decode, computed by each wave on its own with wave-wide
// operations (no LDS, no barrier): at most 64 sequences, no row split, no fixed chunks,
// and the equal-share cut (forced, or the cost model's choice when every non-empty
// sequence holds the same number of blocks and the shares line up with them, where
// plan_core keeps it without evaluating).  Lane b holds sequence b.  Gives the same plan
// as plan_core; write: also store it into v (as plan_core does inside a decode launch).
// Returns false, with nothing written, when the case does not apply.
__device__ inline bool plan_share_wave(const PlanParams& p, MetaView v, bool write, int my_wg, int32_t* sh) {
  const int lane = threadIdx.x & 63;
  const int B = p.batch;
  if (B > 64 || p.row_split != 1 || p.fixed_blocks > 0 || p.split_rule == kRuleCost) return false;
  int err = 0;
  int32_t n = 0;
  if (lane < B) {
    int64_t L = p.uniform_len > 0 ? p.uniform_len : p.seqlens[lane];
    if (L < 0) { L = 0; err = 1; }
    int64_t nn = (L + kPage - 1) / kPage;
    if (nn > p.max_blocks) { nn = p.max_blocks; err = 1; }
    n = (int32_t)nn;
  }
  const int32_t incl = wave_inclusive_sum(n), excl = incl - n;
  const int32_t total = __builtin_amdgcn_readlane(incl, 63);
  const int32_t ne_carry = __builtin_amdgcn_readlane(wave_inclusive_sum(n > 0 ? 1 : 0), 63);
  const int32_t nbm = wave_max_nonneg(n);   // the largest sequence
  int32_t num_wg = 0;
  if (total > 0)
    num_wg = max(1, min(p.grid_wg, (int32_t)floor_div_uniform((int64_t)total + p.min_blocks - 1, p.min_blocks)));
  if (p.split_rule == kRuleAuto && num_wg > 0) {   // must be the even case plan_core skips
    const int64_t share = floor_div_uniform(total, num_wg);
    const bool even = (int64_t)total == (int64_t)nbm * ne_carry && share * num_wg == total && nbm > 0 &&
                      (share == floor_div_uniform(share, nbm) * nbm || nbm == floor_div_uniform(nbm, share) * share);
    if (!even) return false;
  }
  auto cut = [&](int64_t w) -> int64_t { return (w <= num_wg && num_wg > 0) ? floor_div(w * total, num_wg) : total; };
  auto cut_uniform = [&](int64_t w) -> int64_t {   // (w uniform)
    return (w <= num_wg && num_wg > 0) ? floor_div_uniform(w * total, num_wg) : total;
  };
  auto holder = [&](int64_t q) -> int32_t { return wg_of(q, total, num_wg); };
  // lane u's unit: its workgroups and partial slots
  int32_t ns = 0, first = -1;
  if (n > 0) {
    first = holder(excl);
    ns = holder((int64_t)excl + n - 1) - first + 1;
  }
  const int32_t pincl = wave_inclusive_sum(ns > 1 ? ns : 0), poff = pincl - (ns > 1 ? ns : 0);
  const int32_t num_partials = __builtin_amdgcn_readlane(pincl, 63);
  const bool refuse = num_partials > p.max_partials;
  const bool any_err = __builtin_amdgcn_ballot_w64(err != 0) != 0 || num_partials > p.max_partials;
  // my range and the sequences of its two ends
  const int64_t pos = my_wg < num_wg ? cut_uniform(my_wg) : total, end = my_wg < num_wg ? cut_uniform(my_wg + 1) : total;
  int uf = -1, ul = -1;
  if (pos < end) {
    uf = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < B && excl <= pos)) - 1;
    ul = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < B && excl <= end - 1)) - 1;
  }
  sh[kSharePos] = (int32_t)pos;
  sh[kShareEnd] = (int32_t)end;
  sh[kShareUFirst] = uf;
  sh[kShareULast] = ul;
  sh[kShareNumWg] = refuse ? 0 : num_wg;
  sh[kShareErr] = any_err ? 1 : 0;
  if (uf >= 0) {
    sh[kShareNsFirst] = __builtin_amdgcn_readlane(ns, uf);
    sh[kShareFirstWgFirst] = __builtin_amdgcn_readlane(first, uf);
    sh[kSharePoffFirst] = __builtin_amdgcn_readlane(poff, uf);
    sh[kShareStartFirst] = __builtin_amdgcn_readlane(excl, uf);
    sh[kShareNbFirst] = __builtin_amdgcn_readlane(n, uf);
    sh[kShareNsLast] = __builtin_amdgcn_readlane(ns, ul);
    sh[kShareFirstWgLast] = __builtin_amdgcn_readlane(first, ul);
    sh[kSharePoffLast] = __builtin_amdgcn_readlane(poff, ul);
  }
  if (write) {   // the plan, as plan_core stores it; the waves split the per-workgroup words
    const int wv = threadIdx.x >> 6;
    if (wv == 0) {
      if (lane < B) {
        v.cu_blocks[lane] = excl;
        v.num_splits[lane] = ns;
        v.first_wg[lane] = first;
        v.part_off[lane] = poff;
      }
      if (lane == 0) {
        v.cu_blocks[B] = total;
        v.hdr[kHdrMagic] = kMetaMagic;
        v.hdr[kHdrBatch] = B;
        v.hdr[kHdrRows] = p.rows;
        v.hdr[kHdrRowSplit] = 1;
        v.hdr[kHdrRowsPerWg] = p.rows;
        v.hdr[kHdrNumWg] = refuse ? 0 : num_wg;
        v.hdr[kHdrGridWg] = p.grid_wg;
        v.hdr[kHdrTotal] = total;
        v.hdr[kHdrNumPartials] = num_partials;
        if (any_err) v.hdr[kHdrError] = 1;   // other workgroups may already have raised it
        v.hdr[kHdrMaxPartials] = p.max_partials;
        v.hdr[kHdrMaxBlocks] = p.max_blocks;
        v.hdr[kHdrRule] = kRulePages;
        v.hdr[kHdrCostPages] = 0;
        v.hdr[kHdrCostBalanced] = 0;
        v.hdr[kHdrSegCost] = p.seg_cost;
      }
    }
    int32_t* wg_seq = meta_wg_seq(v, p.grid_wg);
    for (int w = threadIdx.x; w <= p.grid_wg; w += 256) {
      const int64_t begin = cut(w);
      v.wg_begin[w] = (int32_t)begin;
      if (w < p.grid_wg) {
        int seq = 0;
        if (w < num_wg && begin < total)   // the largest b with cu[b] <= begin
          for (int k = 1; k < B; ++k) seq += __builtin_amdgcn_readlane(excl, k) <= begin ? 1 : 0;
        wg_seq[w] = seq;
      }
    }
  }
  return true;
}

// Cuts one sequence may hold, under either rule, in plan_share_tables' form.
constexpr int kTablesMaxCuts = 64;
// LDS words plan_share_tables takes: the cuts of each rule and the owner of each cut
// (kPlanLdsWg + 1 words each); per sequence its rank's sequence, first block, block count,
// split count, first workgroup and partial-slot offset (256 words each, first blocks 257);
// 16 words of per-wave totals.
constexpr int kTablesLdsWords = 4 * (kPlanLdsWg + 1) + 6 * 256 + 1 + 16;

// The re-planning decode's form for ragged batches: at most 256 sequences (thread t holds
// sequence t), no row split, no fixed chunks, either rule or the cost model's choice
// between them, computed by the whole workgroup in LDS (tab: kTablesLdsWords words) with
// four barriers.  Instead of searching the sequences for the holder of each cut, every
// sequence writes the cuts that land in it, in closed form: under the equal-share rule the
// cuts w*total/num_wg inside its blocks, under the cost rule the cuts w*ctot/num_wg inside
// its stretch of the cost axis (its c quarters of overhead, then 4 per block).  Each cut is
// written with its owner's sequence, rank among the non-empty sequences, and whether it
// falls on the owner's first block; a workgroup then touches the units from its first cut's
// owner to the owner of its last block, so thread w prices workgroup w under each rule with
// no search.  Same plan as plan_core.  Returns false (every thread alike, before any
// table is written) when the case does not apply: more sequences, row split, fixed chunks,
// more than kPlanLdsWg workgroups, a cost axis whose products with num_wg reach 2^31, or a
// sequence that could hold more than kTablesMaxCuts cuts.  The LDS may be reused after the
// caller's next barrier.
__device__ inline bool plan_share_tables(const PlanParams& p, MetaView v, bool write, int my_wg, int32_t* sh,
                                         MLA_LDS int32_t* tab) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int B = p.batch;
  if (B > 256 || p.row_split != 1 || p.fixed_blocks > 0) return false;
  constexpr int kW = kPlanLdsWg + 1;
  MLA_LDS int32_t* cut_p = tab;
  MLA_LDS int32_t* own_p = tab + kW;
  MLA_LDS int32_t* cut_c = tab + 2 * kW;
  MLA_LDS int32_t* own_c = tab + 3 * kW;
  MLA_LDS int32_t* seq_of_rank = tab + 4 * kW;
  MLA_LDS int32_t* seq_s = seq_of_rank + 256;   // [257]: first block of each sequence, then the total
  MLA_LDS int32_t* seq_n = seq_s + 257;
  MLA_LDS int32_t* seq_ns = seq_n + 256;
  MLA_LDS int32_t* seq_fw = seq_ns + 256;
  MLA_LDS int32_t* seq_po = seq_fw + 256;
  MLA_LDS int32_t* wsum = seq_po + 256;          // [16]: per-wave totals

  // 1. blocks of sequence t; prefix sums and ranks over the workgroup (one barrier)
  int err = 0;
  int32_t n = 0;
  if (t < B) {
    int64_t L = p.uniform_len > 0 ? p.uniform_len : p.seqlens[t];
    if (L < 0) { L = 0; err = 1; }
    int64_t nn = (L + kPage - 1) / kPage;
    if (nn > p.max_blocks) { nn = p.max_blocks; err = 1; }
    n = (int32_t)nn;
  }
  const int32_t incl = wave_inclusive_sum(n);
  const uint64_t nzm = __builtin_amdgcn_ballot_w64(n > 0);
  const int32_t rw = (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(nzm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)nzm, 0));
  const int32_t wmax = wave_max_nonneg(n);
  const bool werr = __builtin_amdgcn_ballot_w64(err != 0) != 0;
  if (lane == 63) {
    wsum[4 * wv] = incl;
    wsum[4 * wv + 1] = (int32_t)__builtin_popcountll(nzm);
    wsum[4 * wv + 2] = wmax;
    wsum[4 * wv + 3] = werr ? 1 : 0;
  }
  lds_barrier();
  int32_t total = 0, ne = 0, nbm = 0, s = 0, r = 0;
  bool any_err = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int32_t ws = wsum[4 * k], wc = wsum[4 * k + 1];
    if (k < wv) {
      s += ws;
      r += wc;
    }
    total += ws;
    ne += wc;
    nbm = max(nbm, wsum[4 * k + 2]);
    any_err |= wsum[4 * k + 3] != 0;
  }
  s += incl - n;
  r += rw;

  // 2. the workgroups, the cost axis, which rules to form; every check before any table write
  int32_t num_wg = 0;
  if (total > 0)
    num_wg = max(1, min(p.grid_wg, (int32_t)floor_div_uniform((int64_t)total + p.min_blocks - 1, p.min_blocks)));
  const int32_t c = p.seg_cost;
  const int64_t ctot64 = 4 * (int64_t)total + (int64_t)c * ne;   // length of the cost axis
  if (num_wg > kPlanLdsWg || ctot64 * num_wg >= ((int64_t)1 << 31) || c < 0) return false;
  // below, every product with num_wg stays under 2^31: 32-bit unsigned arithmetic
  const uint32_t T = (uint32_t)total, C = (uint32_t)ctot64, W = (uint32_t)num_wg, uc = (uint32_t)c;
  bool evaluate = p.split_rule == kRuleAuto && num_wg > 0;
  if (evaluate) {   // the even case plan_core keeps without evaluating
    const int64_t share = floor_div_uniform(T, W);
    if (T == (uint32_t)nbm * (uint32_t)ne && share * W == T && nbm > 0 &&
        (share == floor_div_uniform(share, nbm) * nbm || nbm == floor_div_uniform(nbm, share) * share))
      evaluate = false;
  }
  const bool need_p = num_wg > 0 && p.split_rule != kRuleCost;
  const bool need_c = num_wg > 0 && (p.split_rule == kRuleCost || evaluate);
  // cuts inside one sequence of nb blocks: at most ceil(nb W / T), or ceil((c + 4 nb) W / C)
  if (need_p && floor_div_uniform((uint32_t)nbm * W + T - 1, T) > kTablesMaxCuts) return false;
  if (need_c && floor_div_uniform((uc + 4 * (uint32_t)nbm) * W + C - 1, C) > kTablesMaxCuts) return false;

  // 3. the cuts landing in sequence t, with their owner word: sequence (bits 0-11), rank
  // (12-23), cut on the owner's first block (24) (one barrier)
  const uint32_t cs = 4 * (uint32_t)s + uc * (uint32_t)r;   // the sequence's start on the cost axis
  if (t < B) {
    seq_s[t] = s;
    seq_n[t] = n;
    if (n > 0) {
      seq_of_rank[r] = t;
      const int32_t own = t | (r << 12);
      if (need_p) {
        const uint32_t w1 = ((uint32_t)(s + n) * W + T - 1) / T;
        for (uint32_t w = ((uint32_t)s * W + T - 1) / T; w < w1; ++w) {
          const uint32_t cut = w * T / W;
          cut_p[w] = (int32_t)cut;
          own_p[w] = own | ((cut == (uint32_t)s) << 24);
        }
      }
      if (need_c) {
        const uint32_t w1 = ((cs + uc + 4 * (uint32_t)n) * W + C - 1) / C;
        for (uint32_t w = (cs * W + C - 1) / C; w < w1; ++w) {
          const uint32_t off = w * C / W - cs;
          const uint32_t cut = (uint32_t)s + (off < uc ? 0 : (off - uc) >> 2);
          cut_c[w] = (int32_t)cut;
          own_c[w] = own | ((cut == (uint32_t)s) << 24);
        }
      }
    }
  }
  if (t == 0) {
    seq_s[B] = total;
    if (num_wg > 0) {   // the end: past the last non-empty rank
      cut_p[num_wg] = cut_c[num_wg] = total;
      own_p[num_wg] = own_c[num_wg] = B | (ne << 12) | (1 << 24);
    }
  }
  lds_barrier();

  // 4. the busiest workgroup of each rule (4 per block plus c per unit touched), and each
  // sequence's workgroups and partial slots under both rules (one barrier)
  auto range_cost = [&](MLA_LDS const int32_t* cut, MLA_LDS const int32_t* own, int w) -> int32_t {
    const int32_t lo = cut[w], hi = cut[w + 1];
    if (hi <= lo) return 0;
    const int32_t o0 = own[w], o1 = own[w + 1];
    const int32_t first = (o0 >> 12) & 0xfff, last = ((o1 >> 12) & 0xfff) - ((o1 >> 24) & 1);
    return 4 * (hi - lo) + c * (last - first + 1);
  };
  int32_t worst_p = 0, worst_c = 0;
  if (evaluate) {
    for (int w = t; w < num_wg; w += 256) {
      worst_p = max(worst_p, range_cost(cut_p, own_p, w));
      worst_c = max(worst_c, range_cost(cut_c, own_c, w));
    }
    worst_p = wave_max_nonneg(worst_p);
    worst_c = wave_max_nonneg(worst_c);
  }
  // the workgroup holding block q of this sequence, under each rule
  auto holder_p = [&](uint32_t q) -> int32_t { return (int32_t)(((q + 1) * W - 1) / T); };
  auto holder_c = [&](uint32_t q) -> int32_t {
    const uint32_t y = cs + uc + 4 * (q - (uint32_t)s) + 4;   // cost position just past block q
    return (int32_t)min((y * W - 1) / C, W - 1);
  };
  int32_t ns_p = 0, fw_p = -1, ns_c = 0, fw_c = -1;
  if (n > 0) {
    if (need_p) {
      fw_p = holder_p((uint32_t)s);
      ns_p = holder_p((uint32_t)(s + n - 1)) - fw_p + 1;
    }
    if (need_c) {
      fw_c = holder_c((uint32_t)s);
      ns_c = holder_c((uint32_t)(s + n - 1)) - fw_c + 1;
    }
  }
  // partial slots of both rules in one scan: at most num_wg + B < 2^16 each
  const int32_t xp = ns_p > 1 ? ns_p : 0, xc = ns_c > 1 ? ns_c : 0;
  const int32_t xincl = wave_inclusive_sum(xp | (xc << 16));
  if (lane == 63) {
    wsum[4 * wv] = xincl;
    wsum[4 * wv + 1] = worst_p;
    wsum[4 * wv + 2] = worst_c;
  }
  lds_barrier();
  int32_t xbase = 0, xtot = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int32_t x = wsum[4 * k];
    if (k < wv) xbase += x;
    xtot += x;
    worst_p = max(worst_p, wsum[4 * k + 1]);
    worst_c = max(worst_c, wsum[4 * k + 2]);
  }
  const bool use_cost = p.split_rule == kRuleCost || (evaluate && worst_c < worst_p);
  const int sh16 = use_cost ? 16 : 0;
  const int32_t ns = use_cost ? ns_c : ns_p, fw = use_cost ? fw_c : fw_p;
  const int32_t po = ((xbase + xincl) >> sh16 & 0xffff) - (use_cost ? xc : xp);
  const int32_t num_partials = (xtot >> sh16) & 0xffff;
  const bool refuse = num_partials > p.max_partials;
  any_err |= refuse;

  // 5. this workgroup's share (one barrier: the per-sequence words of its two end units)
  if (t < B) {
    seq_ns[t] = ns;
    seq_fw[t] = fw;
    seq_po[t] = po;
  }
  lds_barrier();
  MLA_LDS const int32_t* cut = use_cost ? cut_c : cut_p;
  MLA_LDS const int32_t* own = use_cost ? own_c : own_p;
  int32_t pos = total, end = total, uf = -1, ul = -1;
  if (my_wg < num_wg) {
    pos = __builtin_amdgcn_readfirstlane(cut[my_wg]);
    end = __builtin_amdgcn_readfirstlane(cut[my_wg + 1]);
  }
  if (pos < end) {
    const int32_t o0 = __builtin_amdgcn_readfirstlane(own[my_wg]);
    const int32_t o1 = __builtin_amdgcn_readfirstlane(own[my_wg + 1]);
    uf = o0 & 0xfff;
    ul = ((o1 >> 24) & 1) ? __builtin_amdgcn_readfirstlane(seq_of_rank[((o1 >> 12) & 0xfff) - 1]) : (o1 & 0xfff);
  }
  sh[kSharePos] = pos;
  sh[kShareEnd] = end;
  sh[kShareUFirst] = uf;
  sh[kShareULast] = ul;
  sh[kShareNumWg] = refuse ? 0 : num_wg;
  sh[kShareErr] = any_err ? 1 : 0;
  if (uf >= 0) {
    sh[kShareNsFirst] = __builtin_amdgcn_readfirstlane(seq_ns[uf]);
    sh[kShareFirstWgFirst] = __builtin_amdgcn_readfirstlane(seq_fw[uf]);
    sh[kSharePoffFirst] = __builtin_amdgcn_readfirstlane(seq_po[uf]);
    sh[kShareStartFirst] = __builtin_amdgcn_readfirstlane(seq_s[uf]);
    sh[kShareNbFirst] = __builtin_amdgcn_readfirstlane(seq_n[uf]);
    sh[kShareNsLast] = __builtin_amdgcn_readfirstlane(seq_ns[ul]);
    sh[kShareFirstWgLast] = __builtin_amdgcn_readfirstlane(seq_fw[ul]);
    sh[kSharePoffLast] = __builtin_amdgcn_readfirstlane(seq_po[ul]);
  }
  if (write) {   // the plan, as plan_core stores it
    if (t < B) {
      v.cu_blocks[t] = s;
      v.num_splits[t] = ns;
      v.first_wg[t] = fw;
      v.part_off[t] = po;
    }
    if (t == 0) {
      v.cu_blocks[B] = total;
      v.hdr[kHdrMagic] = kMetaMagic;
      v.hdr[kHdrBatch] = B;
      v.hdr[kHdrRows] = p.rows;
      v.hdr[kHdrRowSplit] = 1;
      v.hdr[kHdrRowsPerWg] = p.rows;
      v.hdr[kHdrNumWg] = refuse ? 0 : num_wg;
      v.hdr[kHdrGridWg] = p.grid_wg;
      v.hdr[kHdrTotal] = total;
      v.hdr[kHdrNumPartials] = num_partials;
      if (any_err) v.hdr[kHdrError] = 1;   // other workgroups may already have raised it
      v.hdr[kHdrMaxPartials] = p.max_partials;
      v.hdr[kHdrMaxBlocks] = p.max_blocks;
      v.hdr[kHdrRule] = use_cost ? kRuleCost : kRulePages;
      v.hdr[kHdrCostPages] = worst_p;
      v.hdr[kHdrCostBalanced] = worst_c;
      v.hdr[kHdrSegCost] = p.seg_cost;
    }
    int32_t* wg_seq = meta_wg_seq(v, p.grid_wg);
    for (int w = t; w <= p.grid_wg; w += 256) {
      const int32_t begin = (w <= num_wg && num_wg > 0) ? cut[w] : total;
      v.wg_begin[w] = begin;
      if (w < p.grid_wg) wg_seq[w] = (w < num_wg && begin < total) ? (own[w] & 0xfff) : 0;
    }
  }
  return true;
}

}  // namespace mla

// Split planner for MLA decode (the kernel behind mla_get_metadata).
//
// Every sequence b contributes row_split "units" (one per slice of its rows), each
// holding nblk_b = ceil(L_b / 64) KV blocks.  Units are laid end to end (sequence-
// major) and the concatenated block range [0, total) is cut into num_wg contiguous
// shares [floor(w*total/num_wg), floor((w+1)*total/num_wg)), so every workgroup
// streams the same number of blocks (+-1).  A unit cut across k > 1 workgroups gets
// k partial results, merged later by log-sum-exp; their slots are numbered unit by
// unit.  The pages give no scheduler for MLA; the nearest idea on them is the tile
// recommender's warp partition matched to the machine's topology (TileLang notes,
// "Key design 2: tile recommendation").  Deterministic, integer only.
#include "mla_args.h"
#include "mla_device.h"

namespace mla {

constexpr int kPlanLdsBatch = 4095;   // batches up to this size keep cu_blocks in LDS

// Block-wide exclusive scan of one value per thread (256 threads = 4 waves): a scan
// inside each wave, then the wave totals through LDS.  Returns the exclusive prefix and
// writes the block total to *total.
__device__ inline int32_t block_exclusive_scan(int32_t v, int32_t* s, int32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s[wv] = x;
  __syncthreads();
  int32_t base = 0;
  for (int k = 0; k < wv; ++k) base += s[k];
  *total = s[0] + s[1] + s[2] + s[3];
  __syncthreads();  // s is reused by the next scan
  return base + x - v;
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

__global__ __launch_bounds__(256) void mla_plan_kernel(const int32_t* __restrict__ seqlens,
                                                       int32_t* __restrict__ meta, int batch,
                                                       int rows, int row_split, int grid_wg,
                                                       int min_blocks, int max_blocks,
                                                       int max_partials, int fixed_blocks) {
  __shared__ int32_t s_scan[256];
  __shared__ int32_t s_cu[kPlanLdsBatch + 1];   // cu_blocks, when the batch fits
  const int t = threadIdx.x;
  const bool cu_in_lds = batch <= kPlanLdsBatch;
  MetaView v = meta_view(meta, batch, row_split);
  int err = 0;

  // 1. blocks per sequence and their prefix sums
  int32_t carry = 0;
  for (int base = 0; base < batch; base += 256) {
    const int b = base + t;
    int32_t nb = 0;
    if (b < batch) {
      int64_t L = seqlens[b];
      if (L < 0) { L = 0; err = 1; }
      int64_t n = (L + kPage - 1) / kPage;
      if (n > max_blocks) { n = max_blocks; err = 1; }
      nb = (int32_t)n;
    }
    int32_t tot;
    const int32_t excl = block_exclusive_scan(nb, s_scan, &tot);
    if (b < batch) {
      v.cu_blocks[b] = carry + excl;
      if (cu_in_lds) s_cu[b] = carry + excl;
    }
    carry += tot;
  }
  if (t == 0) {
    v.cu_blocks[batch] = carry;
    if (cu_in_lds) s_cu[batch] = carry;
  }
  __syncthreads();  // cu_blocks visible to the whole workgroup

  const int64_t total = (int64_t)row_split * carry;
  const int units = batch * row_split;
  int64_t num_wg = 0;
  int32_t pcarry = 0;
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
          if (first + k < grid_wg) v.wg_begin[first + k] = (int32_t)(ustart + (int64_t)k * fixed_blocks);
      }
      ccarry += ctot;
      pcarry += ptot;
    }
    num_wg = ccarry;
    if (num_wg > grid_wg) err = 1;   // cannot happen when grid_wg covers max_blocks
    for (int w = (int)min<int64_t>(num_wg, grid_wg) + t; w <= grid_wg; w += 256) v.wg_begin[w] = (int32_t)total;
  } else {
    if (total > 0) {
      num_wg = (total + min_blocks - 1) / min_blocks;
      if (num_wg > grid_wg) num_wg = grid_wg;
      if (num_wg < 1) num_wg = 1;
    }

    // 2. workgroup shares
    for (int w = t; w <= grid_wg; w += 256)
      v.wg_begin[w] = (w <= num_wg && num_wg > 0) ? (int32_t)floor_div((int64_t)w * total, num_wg) : (int32_t)total;

    // 3. units: which workgroups cover each, and the partial slots of the split ones
    for (int base = 0; base < units; base += 256) {
      const int u = base + t;
      int32_t ns = 0, first = -1;
      if (u < units) {
        const int b = u / row_split, g = u % row_split;
        const int32_t cb0 = cu_in_lds ? s_cu[b] : v.cu_blocks[b];
        const int32_t cb1 = cu_in_lds ? s_cu[b + 1] : v.cu_blocks[b + 1];
        const int32_t nb = cb1 - cb0;
        if (nb > 0) {
          const int64_t start = (int64_t)row_split * cb0 + (int64_t)g * nb;
          first = wg_of(start, total, num_wg);
          const int32_t last = wg_of(start + nb - 1, total, num_wg);
          ns = last - first + 1;
        }
        v.num_splits[u] = ns;
        v.first_wg[u] = first;
      }
      int32_t tot;
      const int32_t excl = block_exclusive_scan(ns > 1 ? ns : 0, s_scan, &tot);
      if (u < units) v.part_off[u] = pcarry + excl;
      pcarry += tot;
    }
  }

  // 4. header (the error flag is the OR over threads)
  __shared__ int32_t s_err;
  if (t == 0) s_err = 0;
  __syncthreads();
  if (err) atomicOr(&s_err, 1);
  __syncthreads();
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
    if (pcarry > max_partials || num_wg > grid_wg) v.hdr[kHdrNumWg] = 0;  // refuse to run a plan that overflows
  }
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_plan(const int32_t* seqlens, int32_t* meta, int batch, int rows,
                                      int row_split, int grid_wg, int min_blocks, int max_blocks,
                                      int max_partials, int fixed_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(mla::mla_plan_kernel, dim3(1), dim3(256), 0, stream, seqlens, meta, batch,
                     rows, row_split, grid_wg, min_blocks, max_blocks, max_partials, fixed_blocks);
  return hipGetLastError();
}

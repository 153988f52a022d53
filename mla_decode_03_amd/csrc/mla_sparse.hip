// Sparse (top-k) decode, first step: each (b, t) list of token positions -> pool rows.
//
// The dynamic sparse attention the DeepSeek-V4 TileLang note mentions has every query
// token attend to a list of token positions of its sequence, shared by all heads.  This
// kernel turns list (b, t) into the pool row numbers (page * 64 + slot) the decode
// kernel copies from, with the unused entries (-1) squeezed out so the decode masks by
// position alone, and the padding up to whole 64-token blocks filled with row 0 (read,
// then masked).  It writes the kept count as the unit's length; a bad entry (below -1,
// at or past cache_seqlens[b], or on a page outside the pool), or a bad length, writes
// -1 instead, which the decode turns into a NaN row and the plan's error flag.
// One workgroup per (b, t), 256 threads, a block scan per 2048 entries.
#include "mla_args.h"
#include "mla_device.h"

namespace mla {

__global__ __launch_bounds__(256) void mla_sparse_rows_kernel(SparseArgs a) {
  __shared__ int32_t s_scan[256];
  __shared__ int32_t s_bad;
  const int u = blockIdx.x, t = threadIdx.x;
  const int b = u / a.q_len;
  const int64_t L = a.seqlens[b];
  int bad = (L < 0 || L > (int64_t)kPage * a.max_blocks) ? 1 : 0;
  if (t == 0) s_bad = 0;
  const int32_t* list = a.indices + (size_t)u * a.topk;
  int32_t* rows = a.rows + (size_t)u * a.row_stride;
  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;
  // 16-byte accesses where both lists and both row arrays are 16-byte aligned
  const bool vec = ((reinterpret_cast<uintptr_t>(list) | reinterpret_cast<uintptr_t>(rows)) & 15) == 0;
  // 8 consecutive entries per thread and round, every load of a round in flight at once
  // (index, then its block-table entry), then one scan of the per-thread counts keeps
  // the list order.
  constexpr int kPer = 8;
  int32_t carry = 0;
  for (int base = 0; base < a.topk; base += 256 * kPer) {
    int32_t p[kPer], row[kPer];
    const int k0 = base + kPer * t;
    if (vec && k0 + kPer <= a.topk) {   // two 16-byte loads; a wave reads 2 KB in a row
      const int4 v0 = *(const int4*)(list + k0), v1 = *(const int4*)(list + k0 + 4);
      p[0] = v0.x; p[1] = v0.y; p[2] = v0.z; p[3] = v0.w;
      p[4] = v1.x; p[5] = v1.y; p[6] = v1.z; p[7] = v1.w;
    } else {
#pragma unroll
      for (int e = 0; e < kPer; ++e) p[e] = (k0 + e < a.topk) ? list[k0 + e] : -1;
    }
    int32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      row[e] = 0;
      if (p[e] == -1) continue;
      ++cnt;
      if (p[e] < 0 || p[e] >= L || bad) {
        bad = 1;
      } else {
        const int32_t pg = bt_row[p[e] / kPage];   // p < L <= 64 * max_blocks: inside the row
        if (pg < 0 || pg >= a.num_pages) bad = 1;
        else row[e] = pg * kPage + p[e] % kPage;
      }
    }
    int32_t tot;
    int32_t pos = carry + block_exclusive_scan(cnt, s_scan, &tot);
    if (vec && cnt == kPer && (pos & 3) == 0) {   // a full run of kept entries, aligned
      *(int4*)(rows + pos) = int4{row[0], row[1], row[2], row[3]};
      *(int4*)(rows + pos + 4) = int4{row[4], row[5], row[6], row[7]};
    } else {
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (p[e] != -1) rows[pos++] = row[e];
    }
    carry += tot;
  }
  for (int k = carry + t; k < a.row_stride; k += 256) rows[k] = 0;   // whole blocks
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (t == 0) a.lens[u] = s_bad ? -1 : carry;
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_sparse_rows(const mla::SparseArgs* args, hipStream_t stream) {
  if (args->units == 0) return hipSuccess;
  hipLaunchKernelGGL(mla::mla_sparse_rows_kernel, dim3(args->units), dim3(256), 0, stream, *args);
  return hipGetLastError();
}

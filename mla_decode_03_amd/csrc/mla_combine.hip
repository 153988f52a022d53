// Log-sum-exp merge of split-KV partials (the second kernel of a split decode).
//
// A unit (rows of one sequence) cut across k > 1 workgroups left k partial results
// (o_s = normalised output over its key range, lse_s = natural-log sum of exp over
// it; o_s stored as bf16).  Over the union of the disjoint ranges:
//     lse = M + ln(sum_s exp(lse_s - M)),  M = max_s lse_s
//     out = sum_s exp(lse_s - lse) * o_s
// A partial with lse_s = -inf weighs 0; a NaN partial (a poisoned segment) makes the row NaN.  Units with no blocks at all get out = 0,
// lse = -inf.  Units decoded by one workgroup were written directly and are skipped.
// With attention sinks the merged row takes its head's sink here (one more softmax term
// with a zero value row): the partials never include it.
// Memory-bound: 8 rows per workgroup, 32 threads per row, 16 output dims per thread.
#include "mla_args.h"
#include "mla_device.h"

namespace mla {


constexpr int kCombineRows = 8;   // rows per workgroup (256 threads)

__global__ __launch_bounds__(256) void mla_combine_kernel(CombineArgs a) {
  MetaView v = meta_view(const_cast<int32_t*>(a.meta), a.batch, a.row_split);
  const int chunks = (a.rows_per_wg + kCombineRows - 1) / kCombineRows;
  const int u = blockIdx.x / chunks;
  const int rl = (blockIdx.x % chunks) * kCombineRows + (threadIdx.x >> 5);
  if (u >= a.batch * a.row_split || rl >= a.rows_per_wg) return;
  const int ns = v.num_splits[u];
  if (ns == 1) return;
  const int b = u / a.row_split, g = u % a.row_split;
  const int r = g * a.rows_per_wg + rl;
  const int t = threadIdx.x & 31;
  uint16_t* orow = a.out + ((size_t)b * a.rows + r) * kDv + 16 * t;
  if (ns == 0) {
    *(u32x4*)orow = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(orow + 8) = u32x4{0u, 0u, 0u, 0u};
    if (t == 0) a.lse[(size_t)b * a.rows + r] = a.sinks ? a.sinks[r % a.heads] : -INFINITY;
    return;
  }
  const int s0 = v.part_off[u];
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float tot = 0.f, Ms = 0.f;
  // o_s rows of this thread: 16 bf16 = two 16-byte loads per split
  auto part = [&](int sidx) { return (const u32x4*)(a.ws_o + ((size_t)(s0 + sidx) * a.rows_per_wg + rl) * kDv + 16 * t); };
  auto accumulate = [&](float wgt, u32x4 x0, u32x4 x1) {
    tot += wgt;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += wgt * __uint_as_float(x0[j] << 16);
      acc[2 * j + 1] += wgt * __uint_as_float(x0[j] & 0xffff0000u);
      acc[8 + 2 * j] += wgt * __uint_as_float(x1[j] << 16);
      acc[8 + 2 * j + 1] += wgt * __uint_as_float(x1[j] & 0xffff0000u);
    }
  };
  // M = the largest partial LSE (8 loads in flight per step)
  float M = -INFINITY;
  for (int base = 0; base < ns; base += 8) {
    float ls[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      ls[k] = (base + k < ns) ? a.ws_lse[(size_t)(s0 + base + k) * a.rows_per_wg + rl] : -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, ls[k]);
  }
  Ms = (M == -INFINITY) ? 0.f : M;
  // weighted sum, 4 splits per step with all their loads issued before any is used
  for (int base = 0; base < ns; base += 4) {
    float ls[4];
    u32x4 x[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (base + k < ns) {
        ls[k] = a.ws_lse[(size_t)(s0 + base + k) * a.rows_per_wg + rl];
        x[k][0] = part(base + k)[0];
        x[k][1] = part(base + k)[1];
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (base + k < ns) accumulate(expf(ls[k] - Ms), x[k][0], x[k][1]);
  }
  const bool empty = tot == 0.f;  // NaN (a poisoned split) propagates
  float inv = empty ? 0.f : 1.f / tot;
  float lse_v = empty ? -INFINITY : Ms + logf(tot);
  if (a.sinks) {
    const SinkFold f = fold_sink<false>(Ms, tot, a.sinks[r % a.heads]);
    inv = f.scale_o;
    lse_v = f.lse;
  }
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    packed[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *(u32x4*)orow = u32x4{packed[0], packed[1], packed[2], packed[3]};
  *(u32x4*)(orow + 8) = u32x4{packed[4], packed[5], packed[6], packed[7]};
  if (t == 0) a.lse[(size_t)b * a.rows + r] = lse_v;
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_combine(const mla::CombineArgs* args, hipStream_t stream) {
  const int chunks = (args->rows_per_wg + mla::kCombineRows - 1) / mla::kCombineRows;
  const int grid = args->batch * args->row_split * chunks;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(mla::mla_combine_kernel, dim3(grid), dim3(256), 0, stream, *args);
  return hipGetLastError();
}

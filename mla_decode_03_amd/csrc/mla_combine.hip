// Log-sum-exp merge of split-KV partials (the second kernel of a split decode).
//
// A unit (rows of one sequence) cut across k > 1 workgroups left k partial results
// (o_s = normalised output over its key range, lse_s = natural-log sum of exp over
// it).  o_s is stored unnormalised, u_s = o_s / f_s with its factor f_s (1 / row sum)
// beside lse_s, as the bf16 rounding hi_s of u_s, plus lo_s = bf16(u_s - hi_s) for the
// quarters of a row (128 values each) whose flag bit says the decode wrote it (quarters
// with a large |o_s|), so each f_s * (hi_s + lo_s) reaches the merge within
// 0.0039 + 2^-16 |o_s| of o_s.  Over the union of the disjoint ranges:
//     lse = M + ln(sum_s exp(lse_s - M)),  M = max_s lse_s
//     out = sum_s exp(lse_s - lse) * f_s * u_s
// A partial with lse_s = -inf weighs 0; a NaN partial (a poisoned segment) makes the row NaN.  Units with no blocks at all get out = 0,
// lse = -inf.  Units decoded by one workgroup were written directly and are skipped.
// With attention sinks the merged row takes its head's sink here (one more softmax term
// with a zero value row): the partials never include it.
// Memory-bound, in two forms the host picks from the plan's shape (never from the lengths):
//  * 8 rows per workgroup, 32 threads per row, the row's partials merged in groups of 4 in
//    one pass (units that average under 8 partials);
//  * 2 rows per workgroup, 128 threads per row in 4 groups of 32: group q merges the row's
//    partials q, q+4, q+8, ..., and one LDS exchange merges the 4 groups (units of 8 or
//    more partials: a row of 32 takes 2 rounds of loads per thread, not 8, and a launch
//    holds 4 times the workgroups).
// Thread t of a row (or group) owns dims 8t .. 8t+7 and 256+8t .. 256+8t+7, so each 16-byte
// load or store instruction of a wave covers whole 512-byte runs.
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
  uint16_t* orow = a.out + ((size_t)b * a.rows + r) * kDv + 8 * t;
  if (ns == 0) {
    *(u32x4*)orow = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(orow + kDv / 2) = u32x4{0u, 0u, 0u, 0u};
    if (t == 0) a.lse[(size_t)b * a.rows + r] = a.sinks ? a.sinks[r % a.heads] : -INFINITY;
    return;
  }
  const int s0 = v.part_off[u];
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // One pass over the splits, 4 at a time with every load of a group issued before any
  // is used: a running shift Ms (the largest partial LSE so far, 0 while there is none)
  // and the sums rescaled whenever it grows, so the partials are read once and no load
  // waits on an earlier group's LSE.  The low-half flags of the workgroup's 8 rows (word
  // rl0/8 of each slot's mask) are scalar loads issued first, so the few low halves a
  // group needs are requested while its high halves are still in flight.
  float tot = 0.f, Ms = 0.f, M = -INFINITY;
  const int rl0 = (blockIdx.x % chunks) * kCombineRows;
  auto prow = [&](int sidx) { return ((size_t)(s0 + sidx) * a.rows_per_wg + rl); };
  for (int base = 0; base < ns; base += 4) {
    uint32_t mw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      mw[k] = base + k < ns ? a.ws_lo_mask[(size_t)(s0 + base + k) * kLoMaskWords + (rl0 >> 3)] : 0u;
    float ls[4], fs[4];
    u32x4 x[4][2], y[4][2];
    // Past the last split the group reads that split again (no branch around the loads,
    // whose results would otherwise be waited for where the branches join) and gives it
    // no weight.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t pr = prow(min(base + k, ns - 1));
      const float2 lf = *(const float2*)(a.ws_lse + 2 * pr);   // (lse_s, f_s)
      ls[k] = base + k < ns ? lf.x : -INFINITY;
      fs[k] = base + k < ns ? lf.y : 0.f;
      x[k][0] = *(const u32x4*)(a.ws_hi + pr * kDv + 8 * t);
      x[k][1] = *(const u32x4*)(a.ws_hi + pr * kDv + kDv / 2 + 8 * t);
    }
    // this thread's values 8t .. 8t+7 lie in quarter t/16 of its row, 256+8t .. in 2 + t/16
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[k][0] = y[k][1] = u32x4{0u, 0u, 0u, 0u};
      if (mw[k] != 0) {                                  // uniform over the workgroup
        const uint32_t fl = mw[k] >> (4 * (rl & 7));     // this row's 4 bits
        const size_t pr = prow(base + k);
        if (fl & (1u << (t >> 4))) y[k][0] = *(const u32x4*)(a.ws_lo + pr * kDv + 8 * t);
        if (fl & (4u << (t >> 4))) y[k][1] = *(const u32x4*)(a.ws_lo + pr * kDv + kDv / 2 + 8 * t);
      }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < 4; ++k) Mn = fmaxf(Mn, ls[k]);
    const float Msn = (Mn == -INFINITY) ? 0.f : Mn;
    // Rescale once a finite shift grows (uniform over the row's 32 threads).  While M is
    // -inf every weight so far was 0 (or NaN, which stays NaN), so nothing to rescale;
    // a finite M never exceeds Mn, so r <= 1 here.
    if (M != -INFINITY && Msn != Ms) {
      const float r = expf(Ms - Msn);
      tot *= r;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] *= r;
    }
    M = Mn;
    Ms = Msn;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (base + k < ns) {
        const float e = expf(ls[k] - Ms);
        tot += e;
        const float wgt = e * fs[k];   // a poisoned partial's NaN factor makes the row NaN
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v0 = __uint_as_float(x[k][h][j] << 16) + __uint_as_float(y[k][h][j] << 16);
            const float v1 = __uint_as_float(x[k][h][j] & 0xffff0000u) + __uint_as_float(y[k][h][j] & 0xffff0000u);
            acc[8 * h + 2 * j] += wgt * v0;
            acc[8 * h + 2 * j + 1] += wgt * v1;
          }
      }
    }
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
  *(u32x4*)(orow + kDv / 2) = u32x4{packed[4], packed[5], packed[6], packed[7]};
  if (t == 0) a.lse[(size_t)b * a.rows + r] = lse_v;
}

constexpr int kCombineGroupRows = 2;   // rows per workgroup of the grouped form (256 threads)
constexpr int kCombineGroups = 4;   // groups of 32 threads per row

// One group's share of a row's merge: a running shift Ms (the largest partial LSE so far,
// 0 while there is none), the sum of exp(lse_s - Ms) and the weighted sums of the values,
// rescaled whenever the shift grows, so the partials are read once.  Splits go BATCH at a
// time with every load of a batch issued before any is used and no branch around them
// (past the group's last split a batch reads that split again with no weight: behind a
// branch, the compiler waits for each load where the branches join).  The low-half flag
// words (one per slot and 8 rows) are loaded first, so the few low halves a batch needs
// are requested while its high halves are still in flight.
struct GroupMerge {
  float M = -INFINITY, Ms = 0.f, tot = 0.f;
  float acc[16] = {};
};
template <int BATCH>
__device__ __forceinline__ void merge_group(const CombineArgs& a, GroupMerge& m, int s0, int ns, int q, int rl,
                                            int t) {
  const int cnt = ns > q ? (ns - q + kCombineGroups - 1) / kCombineGroups : 0;   // splits q, q+4, ...
  const int cmax = (ns + kCombineGroups - 1) / kCombineGroups;                  // the most any group has
  auto prow = [&](int sidx) { return ((size_t)(s0 + sidx) * a.rows_per_wg + rl); };
  for (int i0 = 0; i0 < cmax; i0 += BATCH) {
    int sk[BATCH];
    bool ok[BATCH];
    uint32_t mw[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      ok[k] = i0 + k < cnt;
      sk[k] = min(q + kCombineGroups * min(i0 + k, max(cnt - 1, 0)), ns - 1);   // a split of this unit
      mw[k] = a.ws_lo_mask[(size_t)(s0 + sk[k]) * kLoMaskWords + (rl >> 3)];
    }
    float ls[BATCH], fs[BATCH];
    u32x4 x[BATCH][2], y[BATCH][2];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const size_t pr = prow(sk[k]);
      const float2 lf = *(const float2*)(a.ws_lse + 2 * pr);   // (lse_s, f_s)
      ls[k] = ok[k] ? lf.x : -INFINITY;
      fs[k] = ok[k] ? lf.y : 0.f;
      x[k][0] = *(const u32x4*)(a.ws_hi + pr * kDv + 8 * t);
      x[k][1] = *(const u32x4*)(a.ws_hi + pr * kDv + kDv / 2 + 8 * t);
    }
    // this thread's values 8t .. 8t+7 lie in quarter t/16 of its row, 256+8t .. in 2 + t/16
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      y[k][0] = y[k][1] = u32x4{0u, 0u, 0u, 0u};
      const uint32_t fl = ok[k] ? mw[k] >> (4 * (rl & 7)) : 0u;   // this row's 4 bits
      if (fl != 0) {
        const size_t pr = prow(sk[k]);
        if (fl & (1u << (t >> 4))) y[k][0] = *(const u32x4*)(a.ws_lo + pr * kDv + 8 * t);
        if (fl & (4u << (t >> 4))) y[k][1] = *(const u32x4*)(a.ws_lo + pr * kDv + kDv / 2 + 8 * t);
      }
    }
    float Mn = m.M;
#pragma unroll
    for (int k = 0; k < BATCH; ++k) Mn = fmaxf(Mn, ls[k]);
    const float Msn = (Mn == -INFINITY) ? 0.f : Mn;
    // Rescale once a finite shift grows.  While M is -inf every weight so far was 0 (or
    // NaN, which stays NaN), so nothing to rescale; a finite M never exceeds Mn, so r <= 1.
    if (m.M != -INFINITY && Msn != m.Ms) {
      const float r = expf(m.Ms - Msn);
      m.tot *= r;
#pragma unroll
      for (int i = 0; i < 16; ++i) m.acc[i] *= r;
    }
    m.M = Mn;
    m.Ms = Msn;
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (ok[k]) {
        const float e = expf(ls[k] - m.Ms);
        m.tot += e;
        const float wgt = e * fs[k];   // a poisoned partial's NaN factor makes the row NaN
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v0 = __uint_as_float(x[k][h][j] << 16) + __uint_as_float(y[k][h][j] << 16);
            const float v1 = __uint_as_float(x[k][h][j] & 0xffff0000u) + __uint_as_float(y[k][h][j] & 0xffff0000u);
            m.acc[8 * h + 2 * j] += wgt * v0;
            m.acc[8 * h + 2 * j + 1] += wgt * v1;
          }
      }
    }
  }
}

__global__ __launch_bounds__(256) void mla_combine_grouped_kernel(CombineArgs a) {
  // groups 1..3 of each row hand their (M, tot, acc[16]) to group 0: [row][group - 1][18][thread]
  __shared__ float red[kCombineGroupRows][kCombineGroups - 1][18][32];
  MetaView v = meta_view(const_cast<int32_t*>(a.meta), a.batch, a.row_split);
  const int chunks = (a.rows_per_wg + kCombineGroupRows - 1) / kCombineGroupRows;
  const int u = blockIdx.x / chunks;
  if (u >= a.batch * a.row_split) return;
  const int ns = v.num_splits[u];                 // uniform over the workgroup
  if (ns == 1) return;
  const int rw = threadIdx.x >> 7, q = (threadIdx.x >> 5) & 3, t = threadIdx.x & 31;
  const int rl = (blockIdx.x % chunks) * kCombineGroupRows + rw;
  const bool row_ok = rl < a.rows_per_wg;        // uniform over the row's 128 threads
  const int b = u / a.row_split, g = u % a.row_split;
  const int r = g * a.rows_per_wg + rl;
  uint16_t* orow = a.out + ((size_t)b * a.rows + r) * kDv + 8 * t;
  if (ns == 0) {                                  // no blocks at all (uniform: no barrier follows)
    if (row_ok && q == 0) {
      *(u32x4*)orow = u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(orow + kDv / 2) = u32x4{0u, 0u, 0u, 0u};
      if (t == 0) a.lse[(size_t)b * a.rows + r] = a.sinks ? a.sinks[r % a.heads] : -INFINITY;
    }
    return;
  }
  GroupMerge m;
  if (row_ok) {
    const int s0 = v.part_off[u];
    if (ns <= kCombineGroups) merge_group<1>(a, m, s0, ns, q, rl, t);
    else if (ns <= 2 * kCombineGroups) merge_group<2>(a, m, s0, ns, q, rl, t);
    else merge_group<4>(a, m, s0, ns, q, rl, t);
  }
  if (q > 0) {
    float* dst = &red[rw][q - 1][0][t];
    dst[0] = m.M;
    dst[32] = m.tot;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[32 * (2 + i)] = m.acc[i];
  }
  __syncthreads();
  if (q > 0 || !row_ok) return;
  // group 0 merges the four groups under their common shift
  float M = m.M;
#pragma unroll
  for (int k = 0; k < kCombineGroups - 1; ++k) M = fmaxf(M, red[rw][k][0][t]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  const float r0 = m.M == -INFINITY ? 0.f : expf(m.Ms - Ms);
  float tot = m.tot * r0;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = m.acc[i] * r0;
#pragma unroll
  for (int k = 0; k < kCombineGroups - 1; ++k) {
    const float Mk = red[rw][k][0][t];
    const float rk = Mk == -INFINITY ? 0.f : expf(Mk - Ms);   // a group with no split weighs 0
    tot += red[rw][k][1][t] * rk;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += red[rw][k][2 + i][t] * rk;
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
  *(u32x4*)(orow + kDv / 2) = u32x4{packed[4], packed[5], packed[6], packed[7]};
  if (t == 0) a.lse[(size_t)b * a.rows + r] = lse_v;
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_combine(const mla::CombineArgs* args, hipStream_t stream) {
  const int rows_per = args->grouped ? mla::kCombineGroupRows : mla::kCombineRows;
  const int chunks = (args->rows_per_wg + rows_per - 1) / rows_per;
  const int grid = args->batch * args->row_split * chunks;
  if (grid == 0) return hipSuccess;
  if (args->grouped) hipLaunchKernelGGL(mla::mla_combine_grouped_kernel, dim3(grid), dim3(256), 0, stream, *args);
  else hipLaunchKernelGGL(mla::mla_combine_kernel, dim3(grid), dim3(256), 0, stream, *args);
  return hipGetLastError();
}

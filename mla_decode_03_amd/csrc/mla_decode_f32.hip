// Plain float32 MLA decode (one wave per query row).
//
// Serves float32 problems, where speed is not the point: every step is the
// definition done directly on the vector ALUs.  Per 64-token page, lane j scores
// token p0 + j (a 576-long dot product against the q row held in LDS, in four
// interleaved partial sums), the wave
// takes the running max / sum by shuffles (online softmax, natural exp), and then
// every lane accumulates 8 of the 512 value dims over the page's tokens.
#include "mla_args.h"
#include "mla_device.h"

namespace mla {


__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__global__ __launch_bounds__(256) void mla_decode_f32_kernel(F32Args a) {
  __shared__ __attribute__((aligned(16))) float qs[4][kDqk];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int chunks = (a.rows + 3) / 4;
  const int b = blockIdx.x / chunks;
  const int r = (blockIdx.x % chunks) * 4 + w;
  if (r >= a.rows) return;  // whole wave leaves; no workgroup barrier below
  const float* qrow = a.q + ((size_t)b * a.rows + r) * kDqk;
  for (int d = l; d < kDqk; d += 64) qs[w][d] = qrow[d];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0);

  const int L = a.seqlens[b];
  bool poison = (L < 0) || ((int64_t)L > (int64_t)kPage * a.max_blocks);
  int n = poison ? 0 : L;
  if (a.causal && a.q_len > 1) n = n - a.q_len + 1 + r / a.heads;
  n = max(n, 0);

  float m = -INFINITY, lsum = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int p0 = 0; p0 < n; p0 += kPage) {
    const int page = a.block_table[(size_t)b * a.bt_stride + p0 / kPage];
    if (page < 0 || page >= a.num_pages) { poison = true; break; }
    const float* pbase = a.kv + (size_t)page * kPage * kDqk;
    const bool valid = p0 + l < n;
    float s = -INFINITY;
    if (valid) {
      // 16-byte loads and four independent partial sums (one per vector component), so
      // the 576-term dot product is not one dependent chain of scalar loads and FMAs
      const f32x4* krow = (const f32x4*)(pbase + (size_t)l * kDqk);
      const f32x4* qv = (const f32x4*)qs[w];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int d = 0; d < kDqk / 4; ++d) {
        const f32x4 kq = krow[d], qq = qv[d];
        acc[0] = fmaf(qq[0], kq[0], acc[0]);
        acc[1] = fmaf(qq[1], kq[1], acc[1]);
        acc[2] = fmaf(qq[2], kq[2], acc[2]);
        acc[3] = fmaf(qq[3], kq[3], acc[3]);
      }
      s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * a.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = expf(m - mn);
    const float pw = valid ? expf(s - mn) : 0.f;
    lsum = lsum * alpha + wave_sum(pw);
    m = mn;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    const int cnt = min(kPage, n - p0);
    // token k's weight from lane k (a scalar read: k is uniform); eight tokens at a time,
    // so that their value rows are in flight together
    int k = 0;
    for (; k + 8 <= cnt; k += 8) {
      float wk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) wk[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), k + u));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* vrow = pbase + (size_t)(k + u) * kDqk;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(wk[u], vrow[l + 64 * i], o[i]);
      }
    }
    for (; k < cnt; ++k) {
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), k));
      const float* vrow = pbase + (size_t)k * kDqk;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(wk, vrow[l + 64 * i], o[i]);
    }
  }
  if (poison && a.err && l == 0) *a.err = 1;   // the plan's fault flag, when there is a plan
  const bool empty = lsum == 0.f;  // no visible key; NaN propagates
  float inv = poison ? __builtin_nanf("") : (empty ? 0.f : 1.f / lsum);
  float lse_v = poison ? __builtin_nanf("") : (empty ? -INFINITY : m + logf(lsum));
  if (a.sinks && !poison) {   // attention sink: one more softmax term, zero value row
    const SinkFold f = fold_sink<false>(m, lsum, a.sinks[r % a.heads]);
    inv = f.scale_o;
    lse_v = f.lse;
  }
  float* orow = a.out + ((size_t)b * a.rows + r) * kDv;
#pragma unroll
  for (int i = 0; i < 8; ++i) orow[l + 64 * i] = o[i] * inv;
  if (l == 0)
    a.lse[(size_t)b * a.rows + r] = lse_v;
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_decode_f32(const mla::F32Args* args, hipStream_t stream) {
  const int grid = args->batch * ((args->rows + 3) / 4);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(mla::mla_decode_f32_kernel, dim3(grid), dim3(256), 0, stream, *args);
  return hipGetLastError();
}

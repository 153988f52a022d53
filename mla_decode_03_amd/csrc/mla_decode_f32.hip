// Float32 MLA decode on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Serves float32 problems, where speed is not the point but the arithmetic is the
// decode's own: both products of the TileLang notes' FlashMLA example (S = Q K^T, then
// O = P V; "A complete example: two-stage optimisation of FlashMLA") run on 32x32
// matrix tiles with fp32 inputs and fp32 accumulation.  One workgroup (4 waves) takes one
// sequence's rows in tiles of 32, and walks its keys 32 at a time:
//   1. the 32 keys' 576-float rows go into LDS (masked keys as zeros);
//   2. S^T (32 keys x 32 rows) = K . Q^T: wave w takes dims 144w .. 144w+143 (72
//      two-dim MFMA steps, its Q fragments held in registers) and the four partial
//      tiles are summed through LDS;
//   3. one thread per row updates the row's running max and sum (online softmax,
//      natural exp) and writes the chunk's weights P into LDS;
//   4. O^T (512 values x 32 rows) += V^T . P^T: wave w takes value tiles 4w .. 4w+3
//      (16 two-key steps each), after scaling its accumulators by the rows' factor.
// The MFMA tile layout (32x32 result, 16 registers per lane): lane l holds column l%32,
// rows 8(i/4) + 4(l/32) + i%4 of register i; an A or B operand element sits in lane
// (row or column) + 32 * (k index).
#include "mla_args.h"
#include "mla_device.h"

namespace mla {

constexpr int kF32Tile = 32;                   // rows per tile, keys per chunk
constexpr int kF32DimsPerWave = kDqk / 4;      // 144
// LDS row pitch of a key row (floats): 16-byte aligned rows, and the 32 rows of a score
// step's A operand spread over the banks (a 576-float pitch would put them in one)
constexpr int kF32Pitch = kDqk + 4;

__global__ __launch_bounds__(256, 1) void mla_decode_f32_kernel(F32Args a) {
  __shared__ __attribute__((aligned(16))) float kc[kF32Tile][kF32Pitch];  // the chunk's key rows
  __shared__ float sp[4][16][64];                                         // partial S tiles, per wave
  __shared__ float pt[kF32Tile][kF32Tile + 1];                            // P [key][row]
  __shared__ float alpha_s[kF32Tile];                                     // rows' rescale factors
  __shared__ int poison_s;
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int tiles = (a.rows + kF32Tile - 1) / kF32Tile;
  const int b = blockIdx.x / tiles;
  const int row0 = (blockIdx.x % tiles) * kF32Tile;
  const int col = l & 31, kh = l >> 5;          // operand element: row/column, k index

  const int L = a.seqlens[b];
  bool poison = (L < 0) || ((int64_t)L > (int64_t)kPage * a.max_blocks);
  const int Lc = poison ? 0 : L;
  // the most keys any row of the tile sees (causal rows see fewer)
  auto visible = [&](int r) {
    int n = Lc;
    if (a.causal && a.q_len > 1) n = n - a.q_len + 1 + r / a.heads;
    return max(n, 0);
  };
  const int nmax = visible(min(row0 + kF32Tile, a.rows) - 1);

  // this wave's Q fragments: B operand of step j (dims 144w + 2j + kh), row row0 + col
  float qf[kF32DimsPerWave / 2];
  {
    const int r = row0 + col;
    const float* qrow = a.q + ((size_t)b * a.rows + (r < a.rows ? r : row0)) * kDqk + kF32DimsPerWave * w + kh;
#pragma unroll
    for (int j = 0; j < kF32DimsPerWave / 2; ++j) qf[j] = r < a.rows ? qrow[2 * j] : 0.f;
  }
  // softmax state of row row0 + t (threads 0..31)
  float m_run = -INFINITY, l_run = 0.f;
  const int nvis_t = visible(row0 + (t < kF32Tile ? t : 0));
  f32x16 o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[v][i] = 0.f;
  if (t == 0) poison_s = 0;

  for (int p0 = 0; p0 < nmax; p0 += kF32Tile) {
    __syncthreads();   // the previous chunk's reads of kc and pt are done
    // 1. key rows p0 .. p0+31 (one page holds them: pages are 64 keys, chunks 32-aligned)
    const int page = a.block_table[(size_t)b * a.bt_stride + p0 / kPage];
    const bool bad = page < 0 || page >= a.num_pages;
    if (bad && t == 0) poison_s = 1;
    const float* base = a.kv + (size_t)(bad ? 0 : page) * kPage * kDqk + (size_t)(p0 % kPage) * kDqk;
    const int nkeys = min(kF32Tile, nmax - p0);
    for (int e = t; e < kF32Tile * kDqk / 4; e += 256) {
      const int k = e / (kDqk / 4), d4 = e % (kDqk / 4);
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (k < nkeys && !bad) v = *(const f32x4*)(base + (size_t)k * kDqk + 4 * d4);
      *(f32x4*)&kc[k][4 * d4] = v;
    }
    __syncthreads();
    // 2. partial S^T over this wave's dims
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int j = 0; j < kF32DimsPerWave / 2; ++j)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[col][kF32DimsPerWave * w + 2 * j + kh], qf[j], s, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) sp[w][i][l] = s[i];
    __syncthreads();
    // 3. softmax update, one thread per row: key k of the chunk is register i = 4(k/8) + k%4
    // of lane 32(k/4 % 2) + row
    if (t < kF32Tile) {
      const int r = t;
      float sv[kF32Tile];
      float mx = m_run;
#pragma unroll
      for (int k = 0; k < kF32Tile; ++k) {
        const int i = 4 * (k >> 3) + (k & 3), ln = 32 * ((k >> 2) & 1) + r;
        float x = (sp[0][i][ln] + sp[1][i][ln]) + (sp[2][i][ln] + sp[3][i][ln]);
        x = (p0 + k < nvis_t) ? x * a.scale : -INFINITY;
        sv[k] = x;
        mx = fmaxf(mx, x);
      }
      // nothing visible yet: keep the shift at 0 so exp(-inf - 0) = 0
      const float ms = mx == -INFINITY ? 0.f : mx;
      const float al = m_run == -INFINITY ? 0.f : expf(m_run - ms);
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < kF32Tile; ++k) {
        const float p = expf(sv[k] - ms);
        pt[k][r] = p;
        ls += p;
      }
      l_run = l_run * al + ls;
      m_run = mx;
      alpha_s[r] = al;
    }
    __syncthreads();
    // 4. O^T += V^T . P^T over the chunk's 32 keys, value tiles 4w .. 4w+3
    const float al = alpha_s[col];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[v][i] *= al;
#pragma unroll 4
    for (int ks = 0; ks < kF32Tile / 2; ++ks) {
      const float pb = pt[2 * ks + kh][col];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        o[v] = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[2 * ks + kh][128 * w + 32 * v + col], pb, o[v], 0, 0, 0);
    }
  }
  __syncthreads();
  poison = poison || poison_s;
  if (poison && a.err && t == 0) *a.err = 1;   // the plan's fault flag, when there is a plan
  // row factors and LSE, then the output: O^T register i of lane l is value
  // 128w + 32v + 8(i/4) + 4(l/32) + i%4 of row row0 + l%32
  if (t < kF32Tile) {
    const bool empty = l_run == 0.f;  // no visible key; NaN propagates
    float inv = poison ? __builtin_nanf("") : (empty ? 0.f : 1.f / l_run);
    float lse_v = poison ? __builtin_nanf("") : (empty ? -INFINITY : m_run + logf(l_run));
    if (a.sinks && !poison && row0 + t < a.rows) {   // attention sink: one more term, zero value row
      const SinkFold f = fold_sink<false>(m_run, l_run, a.sinks[(row0 + t) % a.heads]);
      inv = f.scale_o;
      lse_v = f.lse;
    }
    alpha_s[t] = inv;
    if (row0 + t < a.rows) a.lse[(size_t)b * a.rows + row0 + t] = lse_v;
  }
  __syncthreads();
  const int r = row0 + col;
  if (r < a.rows) {
    const float inv = alpha_s[col];
    float* orow = a.out + ((size_t)b * a.rows + r) * kDv + 128 * w + 4 * kh;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(orow + 32 * v + 8 * q) =
            f32x4{o[v][4 * q] * inv, o[v][4 * q + 1] * inv, o[v][4 * q + 2] * inv, o[v][4 * q + 3] * inv};
  }
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_decode_f32(const mla::F32Args* args, hipStream_t stream) {
  const int grid = args->batch * ((args->rows + mla::kF32Tile - 1) / mla::kF32Tile);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(mla::mla_decode_f32_kernel, dim3(grid), dim3(256), 0, stream, *args);
  return hipGetLastError();
}

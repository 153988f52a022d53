// Split-KV MLA decode on bf16 MFMA for gfx950 (CDNA4).
//
// One workgroup = 4 waves on one CU walks a contiguous range of 64-token KV blocks
// (its share from the split planner; NULL plan = one whole sequence).  Per block:
//
//   S^T = K . Q^T          MFMA 16x16x32 bf16, K tile from LDS, Q fragments in VGPRs
//   online softmax         per row, exp2 with the scale folded into log2(e)
//   O^T += V^T . P^T       MFMA 16x16x32 bf16, V read from the same LDS tile with the
//                          gfx950 transposing LDS read, P straight from registers
//
// This is the two-GEMM structure of the TileLang notes' FlashMLA example ("TileLang:
// bridging programmability and performance in modern neural kernels", section "A
// complete example: two-stage optimisation of FlashMLA": Q and KV tiles staged on
// chip, S kept in registers, down-cast, second GEMM), and the exp2 / log2(e) form of
// the online softmax shown in the DeepSeek-V4 TileLang note (section "The essence of
// TileLang's design").  Placement is re-derived for gfx950: the 128x576 Q tile
// (147 KB) and two 73.7 KB KV pages cannot share the 160 KB LDS, so Q lives in VGPRs,
// O (128x512 fp32, 256 regs per wave) in the accumulation registers (AGPRs), and LDS
// holds only the double-buffered KV stream, fed by global_load_lds (no VGPR staging).
// S is computed transposed (tokens x rows) so that its accumulator layout is already
// the B operand of the second MFMA: no shuffle between the GEMMs.  O is never rescaled
// inside the loop (so its accumulators never leave the AGPRs): each row fixes its
// reference max at its first visible keys and accumulates exp2(x - m_ref) <= 2^16; if a
// later score exceeds m_ref + 16 (log2 units), the segment is decoded again with m_ref
// = the row's true running max, which no score can exceed.
//
// Waves split the rows (TG = 1: 32 rows each, all 64 tokens), or rows and tokens
// (TG = 2, 4) when a sequence has <= 64 / <= 32 rows; token groups merge their
// softmax states through LDS at the end of a segment.
#include "mla_args.h"
#include "mla_device.h"

namespace mla {

// ---- LDS layout of one KV page buffer (73728 B) -------------------------------------
//   [0, 65536)      value/latent part: token t, 16-byte chunk c < 64 at t*1024 + (c ^ swz(t))*16
//   [65536, 73728)  rope part:         token t, chunk 64 + c   at 65536 + t*128 + (c ^ swz(t))*16
// swz maps any 8 consecutive tokens to 8 distinct values (conflict-free K reads: 8 lanes
// read 8 tokens at one chunk) and any 4 consecutive tokens to distinct swz >> 1
// (conflict-free transposing V reads: 4 tokens x 2 adjacent chunks per 16 lanes).
constexpr int kRopeOff = 65536;
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// One wave-wide 16 B/lane global->LDS copy: lane i's 16 bytes from base + voff land at
// LDS address lds + 16*i.  Issued as assembly so the compiler does not treat it as an
// LDS store that every later LDS read must wait for; the decode loop orders these copies
// itself (vmcnt(0) + barrier before a buffer is read, barrier before it is refilled).
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, MLA_LDS uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  // s_nop: one wait state between the SALU write of M0 and the copy that reads it
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

// Enqueue the copy of one KV page into an LDS buffer: 18 wave-wide copies per wave
// (16 value rows + 2 x 8 rope rows).  Tokens >= valid (the tail of a sequence's last
// page) copy token 0 instead: their scores are masked to -inf, so the finite stand-in
// rows contribute exactly 0 and never leak NaN or garbage.  w must be wave-uniform.
__device__ __forceinline__ void issue_page(const uint8_t* __restrict__ kv, int page, int valid,
                                           MLA_LDS uint8_t* buf, int w, int l) {
  const uint8_t* base = kv + (size_t)page * kBlockBytes;   // uniform
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = 16 * w + i;
    const int te = (t < valid) ? t : 0;                     // uniform
    dma16(base + te * kRowBytes, (uint32_t)(l ^ swz(i)) << 4, buf + t * 1024);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int k = 2 * w + i;
    const int t = 8 * k + (l >> 3);
    const int te = (t < valid) ? t : 0;
    dma16(base, (uint32_t)(te * kRowBytes + ((64 + ((l & 7) ^ swz(l >> 3))) << 4)),
          buf + kRopeOff + k * 1024);
  }
}

__device__ __forceinline__ bf16x8 lds_read_b128(const MLA_LDS uint8_t* p) {
  return *(const MLA_LDS bf16x8*)p;
}
__device__ __forceinline__ bf16x4 lds_read_tr(const MLA_LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  bf16x4 r;
  r[0] = (__bf16)v[0];
  r[1] = (__bf16)v[1];
  r[2] = (__bf16)v[2];
  r[3] = (__bf16)v[3];
  return r;
}

// Keep an O tile in AGPRs across a point where vector ALU code touched it.
__device__ __forceinline__ void pin_agpr(f32x4& t) { asm volatile("" : "+a"(t)); }

// Per-wave softmax state and accumulators: rows rbase + 16*nt + (lane % 16), nt < 2.
struct WaveState {
  f32x4 o[32][2];   // O^T tiles [dv tile][row tile]; lane holds dv 16*dt + 4*(lane/16) + j
  float m[2];       // reference max of x = s * scale * log2(e); o and lsum are relative to it
  float lsum[2];    // sum of exp2(x - m)
  float mtrue[2];   // running max of every x seen (for the restart pass)
  bool over;        // some x exceeded m + kRefSlack: the pass must be redone
};

constexpr float kRefSlack = 16.0f;          // scores may exceed the reference max by 2^16
constexpr int kPrefK = 1;                   // K-fragment prefetch distance (32-dim steps)
constexpr int kPrefV = 1;                   // V-fragment prefetch distance (16-dim tiles)
constexpr int kStateSlotFloats = (256 + 4) * 64;

__device__ __forceinline__ void store_state(const WaveState& st, MLA_LDS float* slot, int l) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) slot[((dt * 2 + nt) * 4 + j) * 64 + l] = st.o[dt][nt][j];
    slot[256 * 64 + nt * 64 + l] = st.m[nt];
    slot[256 * 64 + 128 + nt * 64 + l] = st.lsum[nt];
  }
}
__device__ __forceinline__ void merge_state(WaveState& st, const MLA_LDS float* slot, int l) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float mb = slot[256 * 64 + nt * 64 + l];
    const float lb = slot[256 * 64 + 128 + nt * 64 + l];
    const float mn = fmaxf(st.m[nt], mb);
    const float ms = (mn == -INFINITY) ? 0.f : mn;
    const float fa = __builtin_amdgcn_exp2f(st.m[nt] - ms), fb = __builtin_amdgcn_exp2f(mb - ms);
    st.lsum[nt] = st.lsum[nt] * fa + lb * fb;
    st.m[nt] = mn;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st.o[dt][nt][j] = st.o[dt][nt][j] * fa + slot[((dt * 2 + nt) * 4 + j) * 64 + l] * fb;
      pin_agpr(st.o[dt][nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One K step (32 dims) of S^T for NMT token tiles x 2 row tiles, VGPR accumulators.
template <int NMT>
__device__ __forceinline__ void mfma_s_step(f32x4 (&s)[NMT][2], const bf16x8 (&ka)[NMT],
                                            const bf16x8& q0, const bf16x8& q1, int kk) {
  if constexpr (NMT == 2) {
    if (kk == 0) {
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_16x16x32_bf16 %0, %4, %6, 0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %4, %7, 0\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %5, %6, 0\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %5, %7, 0"
          : "=&v"(s[0][0]), "=&v"(s[0][1]), "=&v"(s[1][0]), "=&v"(s[1][1])
          : "v"(ka[0]), "v"(ka[1]), "v"(q0), "v"(q1));
    } else if (kk < 17) {
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %5, %6, %2\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %5, %7, %3"
          : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1])
          : "v"(ka[0]), "v"(ka[1]), "v"(q0), "v"(q1));
    } else {
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %5, %6, %2\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %5, %7, %3\n\t"
          "s_nop 15\n\t"
          "s_nop 4"
          : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1])
          : "v"(ka[0]), "v"(ka[1]), "v"(q0), "v"(q1));
    }
  } else {
    if (kk == 0) {
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_16x16x32_bf16 %0, %2, %3, 0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %2, %4, 0"
          : "=&v"(s[0][0]), "=&v"(s[0][1])
          : "v"(ka[0]), "v"(q0), "v"(q1));
    } else if (kk < 17) {
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %2, %4, %1"
          : "+v"(s[0][0]), "+v"(s[0][1])
          : "v"(ka[0]), "v"(q0), "v"(q1));
    } else {
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %2, %4, %1\n\t"
          "s_nop 15\n\t"
          "s_nop 4"
          : "+v"(s[0][0]), "+v"(s[0][1])
          : "v"(ka[0]), "v"(q0), "v"(q1));
    }
  }
}

// One 16-wide dv tile of O^T += V^T . P^T for both row tiles, accumulators pinned to
// AGPRs.  "s_nop 1" covers a VALU write of an operand right before (2 wait states);
// `last` appends 21 wait states so later VALU reads of O (rescale, epilogue) see the
// final results.
__device__ __forceinline__ void mfma_pv32(f32x4& o0, f32x4& o1, const bf16x8& va, const bf16x8& p0,
                                          const bf16x8& p1, bool last) {
  if (!last)
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %2, %4, %1"
        : "+a"(o0), "+a"(o1)
        : "v"(va), "v"(p0), "v"(p1));
  else
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %2, %4, %1\n\t"
        "s_nop 15\n\t"
        "s_nop 4"
        : "+a"(o0), "+a"(o1)
        : "v"(va), "v"(p0), "v"(p1));
}
__device__ __forceinline__ void mfma_pv16(f32x4& o0, f32x4& o1, const s16x4& va, const s16x4& p0,
                                          const s16x4& p1, bool last) {
  if (!last)
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_16x16x16_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_16x16x16_bf16 %1, %2, %4, %1"
        : "+a"(o0), "+a"(o1)
        : "v"(va), "v"(p0), "v"(p1));
  else
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_16x16x16_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_16x16x16_bf16 %1, %2, %4, %1\n\t"
        "s_nop 15\n\t"
        "s_nop 4"
        : "+a"(o0), "+a"(o1)
        : "v"(va), "v"(p0), "v"(p1));
}

// Lane constants for LDS reads.
struct LaneOffsets {
  int k_v;      // K read, value part: token li row + chunk bits
  int kx;       // K read chunk xor: chunk (4*kk + lq) ^ swz(li) == (4*kk) ^ kx
  int k_r;      // K read, rope part
  int v_base;   // V read: token 4*lq + li/4, byte 8*(li&1)
  int vy[4];    // V read chunk offsets for dv tile dt with dt % 4 == d
};

// One sub-block of NMT 16-token tiles starting at token tokA of the LDS page `cur`:
// scores, lazy online softmax, and the P.V update.
template <int NMT>
__device__ __forceinline__ void sub_block(WaveState& st, const bf16x8 (&qf)[2][18],
                                          const MLA_LDS uint8_t* cur, int tokA, const LaneOffsets& lo,
                                          bool need_mask, int pos0, const int (&nvis)[2],
                                          float scale_log2, int l) {
  const int lq = l >> 4;
  // ---- S^T = K . Q^T over all 576 dims ---------------------------------------------
  // The S accumulators are kept in VGPRs (the AGPRs hold O): these MFMAs are written
  // out so the register class can be pinned.  Chains accumulate into exactly the same
  // registers (no wait states needed); the first step takes C = 0; the last step ends
  // with 21 wait states so VALU reads of S see the final MFMA results.
  f32x4 s[NMT][2];
  auto load_k = [&](int kk, bf16x8(&ka)[NMT]) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int t = tokA + 16 * mt;
      if (kk < 16)
        ka[mt] = lds_read_b128(cur + lo.k_v + t * 1024 + (((4 * kk) ^ lo.kx) << 4));
      else
        ka[mt] = lds_read_b128(cur + lo.k_r + t * 128 + (((4 * (kk - 16)) ^ lo.kx) << 4));
    }
  };
  // K fragments are fetched kPrefK steps ahead through a small ring; the scheduling
  // fences keep the compiler from hoisting further (each fragment costs 4 VGPRs and Q
  // already holds 144).
  bf16x8 kring[kPrefK + 1][NMT];
#pragma unroll
  for (int kk = 0; kk < kPrefK; ++kk) load_k(kk, kring[kk]);
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    if (kk + kPrefK < 18) load_k(kk + kPrefK, kring[(kk + kPrefK) % (kPrefK + 1)]);
    mfma_s_step<NMT>(s, kring[kk % (kPrefK + 1)], qf[0][kk], qf[1][kk], kk);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- softmax: lane owns rows li and 16 + li; its 4*NMT values per row --------------
  float mx[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = s[mt][nt][e] * scale_log2;
        if (need_mask) x = (pos0 + 16 * mt + 4 * lq + e < nvis[nt]) ? x : -INFINITY;
        s[mt][nt][e] = x;
        m = fmaxf(m, x);
      }
    m = wave_max_xor(m, 16);
    mx[nt] = wave_max_xor(m, 32);
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    st.mtrue[nt] = fmaxf(st.mtrue[nt], mx[nt]);
    if (st.m[nt] == -INFINITY) st.m[nt] = mx[nt];     // nothing accumulated yet: exact
    st.over |= mx[nt] > st.m[nt] + kRefSlack;
  }
  bf16x4 pb[NMT][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float msub = (st.m[nt] == -INFINITY) ? 0.f : st.m[nt];
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      f32x4 p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f(s[mt][nt][e] - msub);
        rs += p[e];
      }
      pb[mt][nt] = to_bf16x4(p);
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    st.lsum[nt] += rs;
  }

  // ---- O^T += V^T . P^T (V = first 512 dims of the same tokens) ---------------------
  const MLA_LDS uint8_t* vrow = cur + lo.v_base + tokA * 1024;
  if constexpr (NMT == 2) {
    bf16x8 pk[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) pk[nt] = cat8(pb[0][nt], pb[1][nt]);
    auto load_v = [&](int dt) {
      const MLA_LDS uint8_t* vp = vrow + (dt >> 2) * 128 + lo.vy[dt & 3];
      return cat8(lds_read_tr(vp), lds_read_tr(vp + 16 * 1024));
    };
    bf16x8 vring[kPrefV + 1];
#pragma unroll
    for (int dt = 0; dt < kPrefV; ++dt) vring[dt] = load_v(dt);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      if (dt + kPrefV < 32) vring[(dt + kPrefV) % (kPrefV + 1)] = load_v(dt + kPrefV);
      const bf16x8 va = vring[dt % (kPrefV + 1)];
      mfma_pv32(st.o[dt][0], st.o[dt][1], va, pk[0], pk[1], dt == 31);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    s16x4 pk[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) pk[nt] = __builtin_bit_cast(s16x4, pb[0][nt]);
    auto load_v = [&](int dt) {
      const MLA_LDS uint8_t* vp = vrow + (dt >> 2) * 128 + lo.vy[dt & 3];
      return __builtin_bit_cast(s16x4, lds_read_tr(vp));
    };
    s16x4 vring[kPrefV + 1];
#pragma unroll
    for (int dt = 0; dt < kPrefV; ++dt) vring[dt] = load_v(dt);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      if (dt + kPrefV < 32) vring[(dt + kPrefV) % (kPrefV + 1)] = load_v(dt + kPrefV);
      const s16x4 va = vring[dt % (kPrefV + 1)];
      mfma_pv16(st.o[dt][0], st.o[dt][1], va, pk[0], pk[1], dt == 31);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One segment: rows [row0, row0 + rows_per_wg) of sequence b, blocks [blk_lo, blk_hi).
// slot < 0: write out/lse directly; else write normalised partials to that slot.
template <int TG>
__device__ __forceinline__ void decode_segment(const DecodeArgs& a, MLA_LDS uint8_t* lds, int b,
                                               int row0, int blk_lo, int blk_hi, int slot) {
  constexpr int RG = 4 / TG;       // waves along rows
  constexpr int WTOK = 64 / TG;    // tokens per wave per block
  const int w = wave_id(), l = threadIdx.x & 63;
  const int rg = w % RG, tg = w / RG;
  const int lq = l >> 4, li = l & 15;
  const int R = a.rows;
  const int row_end = min(row0 + a.rows_per_wg, R);
  const int rbase = row0 + 32 * rg;

  const int L = ld_const(a.seqlens, b);
  const bool bad_len = (L < 0) || ((int64_t)L > (int64_t)kPage * a.max_blocks);
  const int Lc = bad_len ? 0 : L;

  int nvis[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = min(rbase + 16 * nt + li, R - 1);
    int n = Lc;
    if (a.causal && a.q_len > 1) n = Lc - a.q_len + 1 + r / a.heads;
    nvis[nt] = max(n, 0);
  }
  // fewest visible keys over the workgroup's rows: masking starts at that position
  int nmin = Lc;
  if (a.causal && a.q_len > 1) nmin = max(Lc - a.q_len + 1 + row0 / a.heads, 0);

  // Q fragments (B operand of S^T = K Q^T): lane holds q[row][32*kk + 8*lq .. +8]
  bf16x8 qf[2][18];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = rbase + 16 * nt + li;
    const bool ok = r < row_end;
    const bf16x8* src = (const bf16x8*)(a.q + ((size_t)b * R + (ok ? r : row0)) * kRowBytes) + lq;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      const bf16x8 v = src[4 * kk];
      qf[nt][kk] = ok ? v : bf16x8{};
    }
  }

  LaneOffsets lo;
  lo.kx = lq ^ swz(li);
  lo.k_v = li * 1024;
  lo.k_r = kRopeOff + li * 128;
  const int vg = (((li >> 2) & 3) << 1) | (lq & 1);   // swz of token 4*lq + li/4
  lo.v_base = (4 * lq + (li >> 2)) * 1024 + 8 * (li & 1);
#pragma unroll
  for (int d = 0; d < 4; ++d) lo.vy[d] = ((2 * d + ((li & 3) >> 1)) ^ vg) << 4;
  const int tok0 = WTOK * tg;

  WaveState st;
  bool bad_page = false;
  float mref_init[2] = {-INFINITY, -INFINITY};
  // Pass 0 fixes each row's reference max at its first visible keys.  Pass 1 runs only
  // if some score outgrew that reference by more than 2^kRefSlack, and starts from the
  // true running max seen in pass 0, which no score of the segment can exceed.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      st.m[nt] = mref_init[nt];
      st.mtrue[nt] = -INFINITY;
      st.lsum[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        st.o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        pin_agpr(st.o[dt][nt]);
      }
    }
    st.over = false;

    __syncthreads();  // LDS free (a previous segment or pass may still be reading it)
    if (blk_lo < blk_hi) {
      const int page = ld_const(a.block_table, (size_t)b * a.bt_stride + blk_lo);
      const bool bad = page < 0 || page >= a.num_pages;
      bad_page |= bad;
      issue_page(a.kv, bad ? 0 : page, bad ? 1 : min(kPage, Lc - blk_lo * kPage), lds, w, l);
    }
    for (int j = blk_lo; j < blk_hi; ++j) {
      const int it = j - blk_lo;
      const MLA_LDS uint8_t* cur = lds + (it & 1) * kBlockBytes;
      MLA_LDS uint8_t* nxt = lds + ((it + 1) & 1) * kBlockBytes;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of block j have landed
      __syncthreads();                // ... and every wave's; block j-1 fully consumed
      if (j + 1 < blk_hi) {
        const int page = ld_const(a.block_table, (size_t)b * a.bt_stride + j + 1);
        const bool bad = page < 0 || page >= a.num_pages;
        bad_page |= bad;
        issue_page(a.kv, bad ? 0 : page, bad ? 1 : min(kPage, Lc - (j + 1) * kPage), nxt, w, l);
      }
      if constexpr (WTOK >= 32) {
#pragma unroll
        for (int sb = 0; sb < WTOK / 32; ++sb) {
          const int tokA = tok0 + 32 * sb;
          const int pos0 = j * kPage + tokA;
          sub_block<2>(st, qf, cur, tokA, lo, pos0 + 32 > nmin, pos0, nvis, a.scale_log2, l);
        }
      } else {
        const int pos0 = j * kPage + tok0;
        sub_block<1>(st, qf, cur, tok0, lo, pos0 + 16 > nmin, pos0, nvis, a.scale_log2, l);
      }
    }
    if (!__syncthreads_or(st.over ? 1 : 0)) break;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) mref_init[nt] = st.mtrue[nt];
  }

  // ---- merge token groups through LDS (the KV buffers are free once all waves pass) --
  if constexpr (TG > 1) {
    MLA_LDS float* slots = (MLA_LDS float*)lds;
#pragma unroll
    for (int step = TG / 2; step >= 1; step /= 2) {
      __syncthreads();
      if (tg >= step && tg < 2 * step) store_state(st, slots + (rg * step + (tg - step)) * kStateSlotFloats, l);
      __syncthreads();
      if (tg < step) merge_state(st, slots + (rg * step + tg) * kStateSlotFloats, l);
    }
  }

  // ---- epilogue -----------------------------------------------------------------------
  const bool poison = bad_len || __syncthreads_or(bad_page ? 1 : 0);
  if (poison && a.meta && threadIdx.x == 0) a.meta[kHdrError] = 1;
  if (tg != 0) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = rbase + 16 * nt + li;
    if (r >= row_end) continue;
    const float ls = st.lsum[nt];
    const bool empty = ls == 0.f;   // no visible key; NaN propagates
    const float nanv = __builtin_nanf("");
    const float scale_o = poison ? nanv : (empty ? 0.f : 1.f / ls);
    const float lse_v = poison ? nanv : (empty ? -INFINITY : (st.m[nt] + __log2f(ls)) * kLn2);
    if (slot < 0) {
      uint16_t* orow = a.out + ((size_t)b * R + r) * kDv + 4 * lq;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const f32x4 o = st.o[dt][nt] * scale_o;
        const uint32_t lo2 = f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
        const uint32_t hi2 = f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
        *(u32x2*)(orow + 16 * dt) = u32x2{lo2, hi2};
      }
      if (lq == 0) a.lse[(size_t)b * R + r] = lse_v;
    } else {
      float* prow = a.ws_o + ((size_t)slot * a.rows_per_wg + (r - row0)) * kDv + 4 * lq;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) *(f32x4*)(prow + 16 * dt) = st.o[dt][nt] * scale_o;
      if (lq == 0) a.ws_lse[(size_t)slot * a.rows_per_wg + (r - row0)] = lse_v;
    }
  }
}

template <int TG>
__global__ __launch_bounds__(256, 1) void mla_decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[2 * kBlockBytes];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)lds_raw;
  const bool planned = a.meta != nullptr;
  MetaView v = meta_view(a.meta, a.batch, a.row_split);
  // XCD-aware numbering: workgroups are dealt round-robin to the 8 XCDs, so logical
  // neighbours (the splits of one sequence) are made to share an XCD and its L2.
  int wg = blockIdx.x;
  if (planned && (gridDim.x & 7) == 0) wg = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  int pos = 0, end = 1;                       // unsplit: one segment, the whole sequence
  if (planned) {
    if (wg >= ld_const(v.hdr, kHdrNumWg)) return;
    pos = ld_const(v.wg_begin, wg);
    end = ld_const(v.wg_begin, wg + 1);
  }
  const int rs = a.row_split;
  while (pos < end) {
    int b, g, blk_lo, blk_hi, slot;
    if (planned) {
      // sequence holding global position pos: the largest b with rs * cu_blocks[b] <= pos
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rs * ld_const(v.cu_blocks, mid) <= pos) lo = mid; else hi = mid - 1;
      }
      b = lo;
      const int cb = ld_const(v.cu_blocks, b);
      const int nb = ld_const(v.cu_blocks, b + 1) - cb;
      g = (pos - rs * cb) / nb;
      const int unit_start = rs * cb + g * nb;
      const int u = b * rs + g;
      blk_lo = pos - unit_start;
      blk_hi = min(end - unit_start, nb);
      slot = (ld_const(v.num_splits, u) > 1) ? ld_const(v.part_off, u) + (wg - ld_const(v.first_wg, u)) : -1;
      pos = unit_start + blk_hi;
    } else {
      b = wg;
      g = 0;
      const int L = ld_const(a.seqlens, b);
      blk_lo = 0;
      blk_hi = min(L > 0 ? (L + kPage - 1) / kPage : 0, a.max_blocks);
      slot = -1;
      pos = end;
    }
    decode_segment<TG>(a, lds, b, g * a.rows_per_wg, blk_lo, blk_hi, slot);
  }
}

}  // namespace mla

extern "C" MLA_INTERNAL hipError_t mla_launch_decode_bf16(const mla::DecodeArgs* args, int grid, hipStream_t stream) {
  const int rpw = args->rows_per_wg;
  if (rpw > 64)
    hipLaunchKernelGGL(mla::mla_decode_bf16_kernel<1>, dim3(grid), dim3(256), 0, stream, *args);
  else if (rpw > 32)
    hipLaunchKernelGGL(mla::mla_decode_bf16_kernel<2>, dim3(grid), dim3(256), 0, stream, *args);
  else
    hipLaunchKernelGGL(mla::mla_decode_bf16_kernel<4>, dim3(grid), dim3(256), 0, stream, *args);
  return hipGetLastError();
}

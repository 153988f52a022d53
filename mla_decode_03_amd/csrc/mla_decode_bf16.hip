// Split-KV MLA decode on bf16 MFMA for gfx950 (CDNA4).
//
// One workgroup = 4 waves on one CU walks a contiguous range of 64-token KV pages (its
// share from the split planner; NULL plan = one whole sequence), a page at a time:
//
//   S^T = K . Q^T          bf16 MFMA, K from LDS, Q fragments held in VGPRs
//   online softmax         per row, exp2 with the scale folded into log2(e)
//   O^T += V^T . P^T       bf16 MFMA, V read from the same LDS page with the gfx950
//                          transposing LDS read, O in the accumulation registers
//
// This is the two-GEMM structure of the TileLang notes' FlashMLA example ("TileLang:
// bridging programmability and performance in modern neural kernels", section "A
// complete example: two-stage optimisation of FlashMLA": Q and KV tiles staged on chip,
// S kept in registers, down-cast, second GEMM), and the exp2 / log2(e) form of the
// online softmax shown in the DeepSeek-V4 TileLang note (section "The essence of
// TileLang's design").  Placement is re-derived for gfx950: the 128x576 Q tile (147 KB)
// and two 73.7 KB pages cannot share the 160 KB LDS, so Q passes through LDS once and
// then lives in VGPRs (32 rows x 576 per wave), O (fp32) in the accumulation registers,
// and LDS holds the double-buffered KV stream fed by global_load_lds (no VGPR staging).
// S is computed transposed (tokens x rows): one query row per lane for the softmax, and
// the accumulator's token order is the B operand order of the second MFMA.
//
// Work split over the 4 waves: each wave scores its own 32 rows (one row tile; waves
// beyond the workgroup's row tiles score nothing), writes its bf16 P fragments to LDS,
// and then accumulates O for ALL rows over its quarter of the 512 value columns (each
// page's V is read from LDS once, not four times).  Everything runs on 32x32x16 MFMA
// tiles; pages stream in as column blocks (see the copies below).
// O is never rescaled inside the loop: each row fixes its reference max at its first
// visible keys and accumulates exp2(x - m_ref) <= 2^kRefSlack; if a later page's sum
// exceeds that, the segment is decoded again with m_ref at or above every score of the
// row (exact: no term can overflow, and the row's largest term is at least 2^-kRefSlack).
#include <hip/hip_ext.h>

#include "mla_args.h"
#include "mla_device.h"
#include "mla_plan_core.h"

namespace mla {

// ---- LDS layout ---------------------------------------------------------------------
// Two page buffers of 73728 B each (column-block layout, defined with the copies below),
// then a 16 KB P buffer: [K step 0..3][row tile 0..3][lane][8 x bf16].
constexpr int kPBufOff = 2 * kBlockBytes;          // 147456
constexpr int kPBufBytes = 16384;                 // P of one page
constexpr int kLdsBytes = kPBufOff + kPBufBytes;   // 163840 = all of it

constexpr float kRefSlack = 16.0f;  // scores may exceed the reference max by 2^16
constexpr float kSumCap = 65536.0f; // 2^kRefSlack: a half-row page sum above it flags
constexpr int kPrefK = 2;           // K-fragment prefetch distance (32-dim steps)
constexpr int kPrefV = 4;           // V-fragment prefetch distance (16-wide value tiles)
// A split partial row is stored unnormalised, u = o / so (so = 1 / row sum, stored beside
// its LSE), as its bf16 rounding hi, within 2^-8 |u| of the fp32 value; each quarter of the
// row (128 values) whose largest normalised |o| exceeds kLoCut also stores lo = bf16(u - hi),
// and hi + lo is within 2^-16 |u|.  Scaled by so in the merge, a partial is never off by
// more than 2^-8 * kLoCut = 0.0039 plus 2^-16 of its own size, however much the partials
// of a row cancel in the merge.
constexpr float kLoCut = 1.0f;
// Compile-time flags and counts passed as tag arguments (one code copy per value).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};
template <int N>
struct IntC {
  static constexpr int value = N;
};
// The low half of one row's quarter (the wave's 128 value columns) of an unnormalised split
// partial, straight from the accumulators: lane (l/32) of the row's pair holds values
// 32 t + 8 i + 4 (l/32) .. +3 of tile t, so `dst` points at the quarter's first value plus
// 4 (l/32), and each 4-value piece is one 8-byte store.  tile(t) gives the accumulator of
// value tile t (0..3).
template <class Tile>
__device__ __forceinline__ void store_lo_quarter(uint16_t* dst, Tile tile) {
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x16& t = tile(t4);
      uint32_t lw[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float x0 = t[4 * i + 2 * h], x1 = t[4 * i + 2 * h + 1];
        const uint32_t hi2 = pack_bf16x2(x0, x1);
        lw[h] = pack_bf16x2(x0 - __uint_as_float(hi2 << 16), x1 - __uint_as_float(hi2 & 0xffff0000u));
      }
      *(u32x2*)(dst + 32 * t4 + 8 * i) = u32x2{lw[0], lw[1]};
    }
}
// Word m of a partial slot's low-half flags: rows 8m .. 8m+7 (of `rows`), 4 bits each, bit
// q set where quarter q (values 128q .. 128q+127) of the row stored its low half, i.e.
// where that quarter's largest |o| (amax[q][row], the value the storing wave compared)
// exceeds kLoCut.
__device__ __forceinline__ uint32_t lo_mask_word(const MLA_LDS float* amax, int m, int rows) {
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rr = 8 * m + j;
    if (rr < rows)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (amax[128 * q + rr] > kLoCut) word |= 1u << (4 * j + q);
  }
  return word;
}

// One wave-wide 16 B/lane global->LDS copy: lane i's 16 bytes from base + voff land at
// LDS address lds + 16*i.  Issued as assembly so the compiler does not treat it as an
// LDS store that every later LDS read must wait for; the decode loop orders these copies
// itself (vmcnt(0) + barrier before a buffer is read, barrier before it is refilled).
// The copy is streaming (nt): a KV page is read once per launch, and keeping it out of the
// L2's retained lines leaves them to Q and the tables (headline decode 85.1 -> 82.7 us).
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, MLA_LDS uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  // s_nop: one wait state between the SALU write of M0 and the copy that reads it
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

// Enqueue the copy of one KV page into an LDS buffer: 18 wave-wide copies per wave
// (16 value rows + 2 x 8 rope rows).  Tokens >= valid (the tail of a sequence's last
// page) copy token 0 instead: their scores are masked to -inf, so the finite stand-in
// rows contribute exactly 0 and never leak NaN or garbage.  w must be wave-uniform.
// A page's global->LDS copy, issued piecewise: each wave issues 18 one-KB copies, 16 of
// value rows (token 16w + i) and 2 of rope rows (8 tokens each).  Tokens at or past
// `valid` re-read token 0 of the page (never used; keeps every read inside the page).
struct PageCopy {
  const uint8_t* base;    // page start in the pool (uniform); sparse: the pool
  int valid;              // tokens of the page in the sequence
  MLA_LDS uint8_t* buf;   // page buffer
  int row_a, row_b;       // sparse: 9 x the pool rows of this lane's two copy tokens
};

// The same copy from a per-lane 64-bit address (sparse blocks gather rows from anywhere
// in the pool).
__device__ __forceinline__ void dma16_at(uint64_t addr, MLA_LDS uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(addr), "{m0}"(m0) : "memory");
}

__device__ __forceinline__ bf16x8 lds_read_b128(const MLA_LDS uint8_t* p) {
  return *(const MLA_LDS bf16x8*)p;
}
__device__ __forceinline__ void lds_write_b128(MLA_LDS uint8_t* p, const bf16x8& v) {
  *(MLA_LDS bf16x8*)p = v;
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

// Workgroup-wide OR of two flag bits (bit 0, bit 1 of `bits`) through 4 words of
// caller-provided LDS (the decode uses every byte of LDS, so the OR cannot reserve its
// own).  The first barrier lets every wave finish its earlier reads of those words before
// any wave overwrites them.
__device__ __forceinline__ int wg_or_bits(int bits, MLA_LDS int* scratch) {
  const int w = wave_id();
  const int wf = (__builtin_amdgcn_ballot_w64(bits & 1) != 0 ? 1 : 0) | (__builtin_amdgcn_ballot_w64(bits & 2) != 0 ? 2 : 0);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = wf;
  __syncthreads();
  const int r = scratch[0] | scratch[1] | scratch[2] | scratch[3];
  __syncthreads();  // every wave has read before the words are reused
  return r;
}

// Keep an O tile in AGPRs across a point where vector ALU code touched it.



// Score step (32x32x16 tiles): two 32-token tiles x the wave's 32 rows, one
// 16-dim K step; accumulators in VGPRs.
__device__ __forceinline__ void mfma32_s_step(f32x16& s0, f32x16& s1, const bf16x8& k0, const bf16x8& k1,
                                              const bf16x8& q, int kk) {
  if (kk == 0)
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %4, 0"
        : "=&v"(s0), "=&v"(s1)
        : "v"(k0), "v"(k1), "v"(q));
  else if (kk < 35)
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
        : "+v"(s0), "+v"(s1)
        : "v"(k0), "v"(k1), "v"(q));
  else
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %4, %1\n\t"
        "s_nop 15\n\t"
        "s_nop 4"
        : "+v"(s0), "+v"(s1)
        : "v"(k0), "v"(k1), "v"(q));
}
// O^T step: one 32-wide value tile x the NRT live row tiles (32 rows each), one 16-token
// K step; accumulators in AGPRs.  `last` drains the pipeline before AGPRs are read.
template <int NRT>
__device__ __forceinline__ void mfma32_pv_step(f32x16 (&o)[NRT], const bf16x8& va, const bf16x8 (&p)[4],
                                               bool last) {
  if constexpr (NRT == 4) {
    if (!last)
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %4, %6, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %4, %7, %2\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %4, %8, %3"
          : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3])
          : "v"(va), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]));
    else
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %4, %6, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %4, %7, %2\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %4, %8, %3\n\t"
          "s_nop 15\n\t"
          "s_nop 4"
          : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3])
          : "v"(va), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]));
  } else if constexpr (NRT == 2) {
    if (!last)
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1"
          : "+a"(o[0]), "+a"(o[1]) : "v"(va), "v"(p[0]), "v"(p[1]));
    else
      asm volatile(
          "s_nop 1\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1\n\t"
          "s_nop 15\n\t"
          "s_nop 4"
          : "+a"(o[0]), "+a"(o[1]) : "v"(va), "v"(p[0]), "v"(p[1]));
  } else {
    static_assert(NRT == 1, "1, 2 or 4 row tiles");
    if (!last)
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o[0]) : "v"(va), "v"(p[0]));
    else
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 4"
                   : "+a"(o[0]) : "v"(va), "v"(p[0]));
  }
}







// Copy description of page j (pool index `page`), checking the index (a bad index reads
// page 0 and poisons the segment).
__device__ __forceinline__ PageCopy page_copy(const DecodeArgs& a, int page, int j, int Lc, MLA_LDS uint8_t* buf,
                                              bool& bad_page) {
  const bool bad = page < 0 || page >= a.num_pages;
  bad_page |= bad;
  return PageCopy{a.kv + (size_t)(bad ? 0 : page) * kBlockBytes, bad ? 1 : min(kPage, Lc - j * kPage), buf, 0, 0};
}

// v[s] for a lane-dependent s < 8 over uniform (scalar) values: a select tree written
// with bit masks.  (Written as conditionals, the first level of the tree was turned into
// an indexed load from a scratch copy of the values, whose wait drained every copy in
// flight, at each block.)
__device__ __forceinline__ int pick(int a, int b, int m) { return (a & ~m) | (b & m); }   // m: 0 or -1
__device__ __forceinline__ int sel8(const int32_t* v, int s) {
  const int m0 = -(s & 1), m1 = -((s >> 1) & 1), m2 = -((s >> 2) & 1);
  const int a0 = pick(v[0], v[1], m0), a1 = pick(v[2], v[3], m0);
  const int a2 = pick(v[4], v[5], m0), a3 = pick(v[6], v[7], m0);
  return pick(pick(a0, a1, m1), pick(a2, a3, m1), m2);
}

// Copy description of block j of a sparse unit: the pool rows of the 16 tokens this wave
// copies (scalar loads of the unit's row list), one per copy token of each lane.  The
// list was checked and padded to whole blocks with row 0 when it was built.
__device__ __forceinline__ PageCopy sparse_copy(const DecodeArgs& a, int b, int j, int Lc, MLA_LDS uint8_t* buf,
                                                int w, int l) {
  const int32_t* r = a.sparse_rows + (size_t)b * a.sparse_stride + j * kPage + 16 * w;
  int32_t v[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) v[m] = ld_const(r, m);
  return PageCopy{a.kv, min(kPage, Lc - j * kPage), buf, 9 * sel8(v, l >> 3), 9 * sel8(v + 8, l >> 3)};
}

template <bool SPARSE>
__device__ __forceinline__ PageCopy block_copy(const DecodeArgs& a, const int* bt_row, int page, int b, int j,
                                               int Lc, MLA_LDS uint8_t* buf, bool& bad_page, int w, int l) {
  if constexpr (SPARSE) return sparse_copy(a, b, j, Lc, buf, w, l);
  else return page_copy(a, page, j, Lc, buf, bad_page);
}

// ===== page stream and decode segment ==================================================
// 32x32x16 MFMA tiles.  Wave w scores rows row0 + 32w .. +31 (one row tile) over the
// page's two 32-token tiles, publishes P (bf16) through LDS, and accumulates O^T for
// value columns 128w .. 128w + 127 of all four row tiles:
//   o[dt][rt] lane l, index 4i + j:  column 128w + 32dt + 8i + 4(l/32) + j,  row row0 + 32rt + l%32.
// P buffer (16 KB after the two page buffers): [K step ks 0..3][row tile 0..3][lane][8 bf16],
// the B operand of O^T += V^T . P^T for tokens 16ks .. 16ks + 15.
// A page is stored in LDS as 9 column blocks (dims 64c .. 64c + 63 of all 64
// tokens, 8 KB each, the rope block last): token t, 16-byte chunk p of block c at
// c*8192 + t*128 + (p ^ cswz(t))*16.  The score loop walks the dims in block order, so it
// can start on a page once its first blocks have landed.
constexpr int kColBlock = 8192;
// Chunk swizzle of the column-block layout.  gfx950 LDS serves 256 bytes per cycle, so a
// 16-lane quarter of a 128-bit read is conflict-free when its 16 slots are distinct
// modulo 256 B.  K reads (16 consecutive tokens, one chunk; rows 128 B apart, so the
// token's low bit picks the 128-B half) need cswz(2i) and cswz(2i+1) to be permutations
// of 0..7; the transposing V reads (4 consecutive tokens x one aligned group of 4 chunks)
// need cswz(t) ^ cswz(t+2) to flip bit 2.  Both hold for:
__device__ __forceinline__ int cswz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }
struct WideLane {
  int k_base;   // K read: token (l % 32)
  int ky[4];    // K read chunk offsets for dims 16kk + 8(l/32): ((2(kk&3) + l/32) ^ swz) * 16
  int v_base;   // V read: token 4(l/32) + (l%16)/4, byte 8(l&1), the wave's first block
  int vy[2][2]; // V read chunk offsets [dt odd][second read: token + 8]
};
__device__ __forceinline__ WideLane wide_lane(int l, int w) {
  WideLane o;
  const int g = l >> 5, q = l >> 4, jj = l & 15;
  const int sk = cswz(l & 31);                        // tokens l%32 and l%32 + 32 alike
  o.k_base = (l & 31) * 128;
#pragma unroll
  for (int m = 0; m < 4; ++m) o.ky[m] = ((2 * m + g) ^ sk) << 4;
  const int tv = 4 * g + (jj >> 2);                   // V token (+ 16 ks; + 8 for the second read)
  o.v_base = tv * 128 + 8 * (jj & 1) + 2 * w * kColBlock;
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int r = 0; r < 2; ++r) o.vy[e][r] = ((4 * e + 2 * (q & 1) + ((jj & 3) >> 1)) ^ cswz(tv + 8 * r)) << 4;
  return o;
}
// Copy i (0..17) of this wave's share of a page in the column-block layout: block i/2,
// tokens 8k .. 8k + 7 with k = 2w + (i & 1); lane l brings chunk (l&7) ^ cswz(t) of token
// t = 8k + l/8.  Copies go out in block order, two per wave per block.
// Sparse blocks: the token's own pool row (tail tokens were given row 0).  A row is
// 9 lines of 128 B, so the chunk's address is pool + ((9 row + cb) << 7) + its 16-byte
// slot: one 32-bit add and one 64-bit shift-add per copy, with only the two per-parity
// lane bases (pool + slot) loop-invariant (the 64-bit per-copy offsets would otherwise
// be hoisted out of the loop and spilled).
template <bool SPARSE = false>
__device__ __forceinline__ void issue_col_copy(const PageCopy& c, int i, int w, int l) {
  const int cb = i >> 1, k = 2 * w + (i & 1);
  const int t = 8 * k + (l >> 3);
  if constexpr (SPARSE) {
    const uint32_t line = (uint32_t)((i & 1) ? c.row_b : c.row_a) + (uint32_t)cb;
    const uint64_t lane_base = (uint64_t)(uintptr_t)c.base + (uint32_t)(((l & 7) ^ cswz(t)) << 4);
    dma16_at(((uint64_t)line << 7) + lane_base, c.buf + cb * kColBlock + k * 1024);
  } else {
    const int te = (t < c.valid) ? t : 0;
    dma16(c.base, (uint32_t)(te * kRowBytes + cb * 128 + (((l & 7) ^ cswz(t)) << 4)),
          c.buf + cb * kColBlock + k * 1024);
  }
}
// Where the next page's 18 copies (per wave, in copy order) go inside one page's
// compute.  Score loop: the block-group waits cut the 36 steps into 5 windows; each
// window carries up to 2 copies per wave, at fixed steps (the first step of the window
// and 4 steps before its end), the same for every wave, so the copy sites are
// compile-time and every wave issues the same copies before each wait.  Then kCopySm
// after the softmax and the rest spread over the 16 P.V steps.  (Staggering the waves'
// copy steps by wave id needed a runtime condition at every step and was 5% slower.)
constexpr int win_start(int W) { return W == 0 ? 0 : 8 * W - kPrefK; }
constexpr int win_end(int W) { return W == 4 ? 36 : 8 * (W + 1) - kPrefK; }
constexpr int win_of(int kk) { return kk < win_start(1) ? 0 : kk < win_start(2) ? 1 : kk < win_start(3) ? 2 : kk < win_start(4) ? 3 : 4; }
constexpr int win_len(int W) { return win_end(W) - win_start(W); }
// copies per window: slot 0 at the window's first step, slot 1 four steps before its end
constexpr int win_copies(int W) { return win_len(W) >= 6 ? 2 : win_len(W) >= 4 ? 1 : 0; }
// windows 1-3 are 8 steps long (2 copies each)
constexpr int copies_before_win(int W) {
  return W == 0 ? 0 : W <= 4 ? win_copies(0) + 2 * (W - 1) : win_copies(0) + 6 + win_copies(4);
}
constexpr int kCopyS = copies_before_win(5), kCopySm = 2;
constexpr int kCopyPV = 18 - kCopyS - kCopySm;
static_assert(kCopyPV >= 0 && kCopyPV <= 16, "copy schedule");
static_assert(win_len(1) == 8 && win_len(2) == 8 && win_len(3) == 8, "copy schedule");
// Copies this wave issued in the score loop before step kk (kk a window start).
constexpr int s_copies_before(int kk) { return copies_before_win(win_of(kk)); }
// This page's copies issued after block group G (blocks 2G, 2G+1; G = 4: the rope block).
constexpr int copies_after_group(int G) { return G < 4 ? 14 - 4 * G : 0; }
// Wait until this wave's copies of the current page up to a block group have landed,
// then meet the other waves (their copies of those blocks have landed too).  N = copies
// this wave issued after that group (they may still be in flight; loads complete in
// order): the page's later groups plus the next page's copies issued so far.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
  __syncthreads();
}
// Which block group each wait point covers: point 0 is the page head, point S (1..4) the
// score step that first loads block group S.  A point covers a group at or past its own
// (loads complete in order, so covering a later group covers the earlier ones too);
// -1 = no wait there, which needs an earlier point to have covered that group.
constexpr int kWaitCover[5] = {0, 1, 2, 3, 4};
constexpr bool wait_plan_ok() {
  int covered = kWaitCover[0];
  if (covered < 0) return false;
  for (int S = 1; S <= 4; ++S) {
    if (kWaitCover[S] >= 0) {
      if (kWaitCover[S] < S || kWaitCover[S] <= covered) return false;
      covered = kWaitCover[S];
    }
    if (covered < S) return false;
  }
  return true;
}
static_assert(wait_plan_ok(), "every block group is waited for before it is read");
template <int S>
__device__ __forceinline__ void wait_point(bool pre) {
  if constexpr (kWaitCover[S] >= 0) {
    constexpr int kk = 8 * S - kPrefK;   // the step that first loads block group S
    if (pre) wait_vm_barrier<copies_after_group(kWaitCover[S]) + s_copies_before(kk)>();
    else wait_vm_barrier<copies_after_group(kWaitCover[S])>();
  }
}

// NRT = row tiles of 32 rows the workgroup holds (rows_per_wg <= 32 NRT).  Wave w scores
// row tile w; waves w >= NRT score zero query rows (no branch around their MFMAs: the
// MFMAs are assembly the compiler cannot see, so it must never have to move their
// accumulators between branches), and only the NRT live row tiles enter P.V.
template <int NRT, bool SPARSE>
__device__ __forceinline__ void decode_segment_wide(const DecodeArgs& a, MLA_LDS uint8_t* lds, int b,
                                                    int row0, int blk_lo, int blk_hi, int slot) {
  const int w = wave_id(), l = threadIdx.x & 63;
  const int g = l >> 5, lr = l & 31;
  const int R = a.rows;
  const int row_end = min(row0 + a.rows_per_wg, R);
  const int myrow = row0 + 32 * w + lr;

  const int L = ld_const(a.seqlens, b);
  // more keys than the block table's row can hold: ceil(L / kPage) > max_blocks, in 32 bits
  const bool bad_len = (L < 0) || (L > 0 && (L - 1) / kPage >= a.max_blocks);
  const int Lc = bad_len ? 0 : L;
  int nvis = Lc;
  if (a.causal && a.q_len > 1) nvis = Lc - a.q_len + 1 + min(myrow, R - 1) / a.heads;
  nvis = max(nvis, 0);
  int nmin = Lc;  // fewest visible keys over the workgroup's rows: masking starts there
  if (a.causal && a.q_len > 1) nmin = max(Lc - a.q_len + 1 + row0 / a.heads, 0);

  // Q fragments (B operand of S^T = K Q^T): dims 16kk + 8g .. +8 of row myrow.  The
  // workgroup's rows are contiguous in q, so they come in as (up to) two 64-row "pages"
  // through the page buffers, with the KV pages' column-block copies (whole 128-byte
  // lines per copy); each wave then reads its 32 rows' fragments.
  // With 64 rows or fewer Q fits the second buffer, and page blk_lo streams into the
  // first one meanwhile.
  bf16x8 qf[36];
  const int nq = row_end - row0;
  const bool q_one = nq <= 64;
  const int* bt_row = a.block_table + (size_t)b * a.bt_stride;
  bool bad_page = false, first_issued = false;
  {
    __syncthreads();   // LDS free (a previous segment may still be reading it)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (64 * h < nq) {
        const PageCopy qc{a.q + ((size_t)b * R + row0 + 64 * h) * kRowBytes, min(64, nq - 64 * h),
                          lds + (q_one ? 1 : h) * kBlockBytes};
#pragma unroll
        for (int i = 0; i < 18; ++i) issue_col_copy(qc, i, w, l);
      }
    if (q_one && blk_lo < blk_hi) {
      const PageCopy first = block_copy<SPARSE>(a, bt_row, SPARSE ? 0 : ld_const(bt_row, blk_lo), b, blk_lo, Lc,
                                                lds, bad_page, w, l);
#pragma unroll
      for (int i = 0; i < 18; ++i) issue_col_copy<SPARSE>(first, i, w, l);
      first_issued = true;
    }
    if (first_issued) wait_vm_barrier<18>();   // Q's copies (page blk_lo's may still fly)
    else wait_vm_barrier<0>();
    const int rr = (32 * w + lr) & 63;                        // row within its 64-row half
    const MLA_LDS uint8_t* qb = lds + (q_one ? 1 : (w >> 1)) * kBlockBytes + rr * 128;
    const int sq = cswz(rr);
    const bool ok = myrow < row_end;
#pragma unroll
    for (int kk = 0; kk < 36; ++kk) {
      const bf16x8 v = lds_read_b128(qb + (kk >> 2) * kColBlock + (((2 * (kk & 3) + g) ^ sq) << 4));
      qf[kk] = ok ? v : bf16x8{};
    }
  }
  const WideLane wl = wide_lane(l, w);
  MLA_LDS uint8_t* pbuf = lds + kPBufOff;

  f32x16 o[4][NRT];
  float m_ref = -INFINITY, mtrue = -INFINITY, lsum = 0.f;
  bool over = false, bad_wg = false;   // bad_wg: some wave read a bad page
  float mref_init = -INFINITY;
  for (int pass = 0; pass < 2; ++pass) {
    m_ref = mref_init;
    mtrue = -INFINITY;
    lsum = 0.f;
    over = false;
    // Zeros from an opaque scalar formed in this pass: a plain zero vector is one value the
    // compiler keeps (and spills) from the kernel's start to every pass.
    int zi = 0;
    asm volatile("" : "+s"(zi));
    const float zf = __int_as_float(zi);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        o[dt][rt] = f32x16{zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf};
        asm volatile("" : "+a"(o[dt][rt]));
      }

    __syncthreads();  // LDS free (a previous segment or pass may still be reading it)
    if (blk_lo < blk_hi && !(pass == 0 && first_issued)) {
      const PageCopy first = block_copy<SPARSE>(a, bt_row, SPARSE ? 0 : ld_const(bt_row, blk_lo), b, blk_lo, Lc,
                                                lds, bad_page, w, l);
#pragma unroll
      for (int i = 0; i < 18; ++i) issue_col_copy<SPARSE>(first, i, w, l);
    }
    int pg_ahead = (!SPARSE && blk_lo + 1 < blk_hi) ? ld_const(bt_row, blk_lo + 1) : 0;   // page j+1's index
    for (int j = blk_lo; j < blk_hi; ++j) {
      const int it = j - blk_lo;
      const MLA_LDS uint8_t* cur = lds + (it & 1) * kBlockBytes;
      // page j's first block groups have landed (all waves); page j-1 and its P are consumed
      wait_vm_barrier<copies_after_group(kWaitCover[0])>();
      // Page j+1 streams into the other buffer while this page is computed: its 18 copies
      // per wave go out in block order, spread over the MFMA loops below (the copy
      // schedule above; the waits in S count on it),
      // so no wave stalls for long on a full memory queue with its matrix unit idle, and
      // the later blocks of page j are waited for only where S reaches them.
      const bool pre = j + 1 < blk_hi;
      PageCopy nxt{};
      if (pre)
        nxt = block_copy<SPARSE>(a, bt_row, pg_ahead, b, j + 1, Lc, lds + ((it + 1) & 1) * kBlockBytes, bad_page,
                                 w, l);
      pg_ahead = (!SPARSE && j + 2 < blk_hi) ? ld_const(bt_row, j + 2) : 0;   // read a page ahead

      // ---- S^T: 2 token tiles x 32 rows x 576 dims ----------------------------------
      f32x16 s0, s1;
      {
        auto load_k = [&](int kk, bf16x8& k0, bf16x8& k1) {
          const MLA_LDS uint8_t* p = cur + (kk >> 2) * kColBlock + wl.k_base + wl.ky[kk & 3];
          k0 = lds_read_b128(p);
          k1 = lds_read_b128(p + 32 * 128);
        };
        // Sparse blocks hold two more per-lane values (their copy rows) through the page;
        // a one-step K prefetch there frees the registers.  The block-group waits stay
        // where the two-step schedule puts them (one step early for the one-step loads).
        constexpr int PK = SPARSE ? 1 : kPrefK;
        bf16x8 kr0[PK + 1], kr1[PK + 1];
#pragma unroll
        for (int kk = 0; kk < PK; ++kk) load_k(kk, kr0[kk], kr1[kk]);
#pragma unroll
        for (int kk = 0; kk < 36; ++kk) {
          // before the first read of blocks 2G, 2G+1: wait for them
          const int kl = kk + kPrefK;            // the wait schedule's load step
          if (kl == 8) wait_point<1>(pre);
          if (kl == 16) wait_point<2>(pre);
          if (kl == 24) wait_point<3>(pre);
          if (kl == 32) wait_point<4>(pre);
          if (kk + PK < 36) load_k(kk + PK, kr0[(kk + PK) % (PK + 1)], kr1[(kk + PK) % (PK + 1)]);
          mfma32_s_step(s0, s1, kr0[kk % (PK + 1)], kr1[kk % (PK + 1)], qf[kk], kk);
          // a copy issued behind the step's MFMAs stalls (on a full memory queue) while
          // they run rather than ahead of them
          if (pre) {
            const int W = win_of(kk), d = kk - win_start(W), d1 = d - (win_len(W) - 4);
            if (win_copies(W) >= 1 && d == 0) issue_col_copy<SPARSE>(nxt, copies_before_win(W), w, l);
            if (win_copies(W) == 2 && d1 == 0) issue_col_copy<SPARSE>(nxt, copies_before_win(W) + 1, w, l);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax of the wave's row myrow over the page's 64 keys -------------------
      // Scores stay unscaled (scale > 0 commutes with max); the scale is folded into the
      // exponent's FMA below.  Only a sequence's last pages (or causal rows) mask.
      if (j * kPage + kPage > nmin) {
        asm volatile("");   // keep this a branch: the full pages skip it
        const int lim = nvis - j * kPage;                        // visible tokens of the page
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t0 = 8 * (e >> 2) + 4 * g + (e & 3);          // token of s0[e] in the page
          s0[e] = (t0 < lim) ? s0[e] : -INFINITY;
          s1[e] = (t0 + 32 < lim) ? s1[e] : -INFINITY;
        }
      }
      // A row takes its reference max from the first page where it sees a key (both
      // lane halves of the row agree on it).  Only while some row of the wave has none
      // does the wave take the page's row maxima.
      if (__builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0) {
        float mr = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) mr = fmaxf(mr, fmaxf(s0[e], s1[e]));
        const float mx = wave_max_xor(mr, 32) * a.scale_log2;
        if (m_ref == -INFINITY) m_ref = mx;      // nothing accumulated yet: exact
      }
      const float msub = (m_ref == -INFINITY) ? 0.f : m_ref;
      float rs = 0.f;
      f32x16 p0, p1;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p0[e] = __builtin_amdgcn_exp2f(fmaf(s0[e], a.scale_log2, -msub));
        p1[e] = __builtin_amdgcn_exp2f(fmaf(s1[e], a.scale_log2, -msub));
        rs += p0[e] + p1[e];
      }
      // lsum holds this lane's half of the row (its 32 of the page's 64 keys); the halves
      // are added once, in the epilogue.  Every term is at most the half-row sum, so
      // no term exceeds 2^kRefSlack unless that sum does (an overflow to inf included);
      // only then does the wave take this page's maxima, for the second pass's max.
      lsum += rs;
      if (__builtin_amdgcn_ballot_w64(rs > kSumCap) != 0) {
        over |= rs > kSumCap;
        float mr = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) mr = fmaxf(mr, fmaxf(s0[e], s1[e]));
        mtrue = fmaxf(mtrue, mr * a.scale_log2);
      }
      // B operands per 16-token K step: ks -> tile ks/2, C indices 8(ks&1) .. +7
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x16& pt = (ks < 2) ? p0 : p1;
        const int base = 8 * (ks & 1);
        f32x4 lo4 = {pt[base + 0], pt[base + 1], pt[base + 2], pt[base + 3]};
        f32x4 hi4 = {pt[base + 4], pt[base + 5], pt[base + 6], pt[base + 7]};
        lds_write_b128(pbuf + ((ks * 4 + w) * 64 + l) * 16, cat8(to_bf16x4(lo4), to_bf16x4(hi4)));
      }
      if (pre) {
#pragma unroll
        for (int i = 0; i < kCopySm; ++i) issue_col_copy<SPARSE>(nxt, kCopyS + i, w, l);
      }
      __syncthreads();  // every wave's P visible

      // ---- O^T += V^T . P^T over the wave's 128 value columns, all 128 rows ----------
      auto load_v = [&](int t) {   // t = 4 ks + dt
        const int ks = t >> 2, dt = t & 3;
        const MLA_LDS uint8_t* vp = cur + wl.v_base + ks * 16 * 128 + (dt >> 1) * kColBlock;
        return cat8(lds_read_tr(vp + wl.vy[dt & 1][0]), lds_read_tr(vp + 8 * 128 + wl.vy[dt & 1][1]));
      };
      bf16x8 vring[kPrefV + 1];
#pragma unroll
      for (int t = 0; t < kPrefV; ++t) vring[t] = load_v(t);
      bf16x8 pf[2][4];   // P fragments of K step ks (all 4 row tiles), read one step ahead
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) pf[0][rt] = lds_read_b128(pbuf + (rt * 64 + l) * 16);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int ks = t >> 2, dt = t & 3;
        if (dt == 0 && ks < 3) {
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) pf[(ks + 1) & 1][rt] = lds_read_b128(pbuf + (((ks + 1) * 4 + rt) * 64 + l) * 16);
        }
        if (t + kPrefV < 16) vring[(t + kPrefV) % (kPrefV + 1)] = load_v(t + kPrefV);
        mfma32_pv_step<NRT>(o[dt], vring[t % (kPrefV + 1)], pf[ks & 1], t == 15);
        if (pre) {
#pragma unroll
          for (int i = 0; i < kCopyPV; ++i)
            if (i * 16 / kCopyPV == t) issue_col_copy<SPARSE>(nxt, kCopyS + kCopySm + i, w, l);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the page buffers and P buffer are idle until the next pass starts.  One OR gives
    // both the second-pass flag and the bad-page flag (the second pass streams the same
    // pages, so it gives the same bad-page flag).
    const int flags = wg_or_bits((over ? 1 : 0) | (bad_page ? 2 : 0), (MLA_LDS int*)pbuf);
    bad_wg = (flags & 2) != 0;
    if (!(flags & 1)) break;
    // Second pass from an upper bound of every score of the row: pages that did not flag
    // stayed within m_ref + kRefSlack, the flagged ones gave their maxima.
    {
      const float mt = fmaxf(mtrue, m_ref + kRefSlack);
      mref_init = fmaxf(mt, __shfl_xor(mt, 32, 64));
    }
  }

  // ---- epilogue: every wave needs the row statistics of all 128 rows ---------------------
  const bool poison = bad_len || bad_wg;
  if (poison && a.meta && threadIdx.x == 0) a.meta[kHdrError] = 1;
  // Per row, once: the factor that normalises O and the natural-log LSE.  The attention
  // sink enters a row once, where its final result is formed: here for an unsplit range,
  // in the combine for the partials of a split one.
  MLA_LDS float* stats = (MLA_LDS float*)pbuf;   // [row][scale_o, lse]
  MLA_LDS float* amax = stats + 2 * 128;         // [wave][row]: largest |o| over the wave's columns
  lsum += __shfl_xor(lsum, 32, 64);              // the row's two halves
  const float nanv = __builtin_nanf("");
  // The epilogue's lane indices, formed here from an opaque copy of the thread index, so
  // that the addresses derived from them are not computed before the page loop and kept
  // (spilled) across it.
  int tid_e = threadIdx.x;
  asm volatile("" : "+v"(tid_e));
  const int l_e = tid_e & 63, g_e = l_e >> 5, lr_e = l_e & 31;
  if (g_e == 0) {
    const int rr = 32 * w + lr_e;
    float so, lse_v;
    if (poison) {
      so = nanv;
      lse_v = nanv;
    } else if (slot < 0 && a.sinks) {
      const SinkFold f = fold_sink<true>(m_ref, lsum, a.sinks[(row0 + rr) % a.heads] * kLog2e);
      so = f.scale_o;
      lse_v = f.lse * kLn2;
    } else {
      const bool empty = lsum == 0.f;   // no visible key; NaN propagates
      so = empty ? 0.f : 1.f / lsum;
      lse_v = empty ? -INFINITY : (m_ref + __log2f(lsum)) * kLn2;
    }
    stats[2 * rr] = so;
    stats[2 * rr + 1] = lse_v;
  }
  __syncthreads();
  // O goes through LDS as bf16 so that every store writes a whole 1 KB row: row rr of the
  // workgroup at rr*1024, 16-byte chunk c (values 8c .. 8c+7) at (c ^ (rr & 15))*16.  The
  // page buffers are idle now.  An unsplit row is normalised here; a split partial stays
  // unnormalised (the merge applies the factor, stored beside its LSE), and the same pass
  // takes each row's largest |o| over the wave's columns, in normalised units (NaN is
  // ignored here; the row's factor carries it).
  MLA_LDS uint8_t* ob = lds;
  const bool part = slot >= 0;
  const size_t prow = (size_t)slot * a.rows_per_wg;   // the partial slot's first row
  auto stage = [&](auto norm_tag) {
    constexpr bool kNorm = decltype(norm_tag)::value;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int rr = 32 * rt + lr_e;
      const float scale_o = stats[2 * rr];
      float mx = 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x16& t = o[dt][rt];
          float x0 = t[4 * i], x1 = t[4 * i + 1], x2 = t[4 * i + 2], x3 = t[4 * i + 3];
          if constexpr (kNorm) {
            x0 *= scale_o;
            x1 *= scale_o;
            x2 *= scale_o;
            x3 *= scale_o;
          } else {
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))));
          }
          const int c = 16 * w + 4 * dt + i;
          *(MLA_LDS u32x2*)(ob + rr * 1024 + ((c ^ (rr & 15)) << 4) + 8 * g_e) =
              u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      if constexpr (!kNorm) {
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_o;   // over the wave's 128 columns of the row
        if (g_e == 0) amax[w * 128 + rr] = mx;
        if (mx > kLoCut && row0 + rr < row_end)            // this quarter of the row keeps its low half
          store_lo_quarter(a.ws_lo + (prow + rr) * kDv + 128 * w + 4 * g_e, [&](int dt) -> const f32x16& { return o[dt][rt]; });
      }
    }
  };
  if (part) stage(BoolC<false>{});
  else stage(BoolC<true>{});
  __syncthreads();
  for (int k = 0; k < 32; ++k) {                  // the wave's rows 32w .. 32w+31
    const int rr = 32 * w + k;
    if (row0 + rr >= row_end) break;              // uniform
    const u32x4 v = *(const MLA_LDS u32x4*)(ob + rr * 1024 + ((l_e ^ (rr & 15)) << 4));
    uint16_t* dst = part ? a.ws_hi + (prow + rr) * kDv : a.out + ((size_t)b * R + row0 + rr) * kDv;
    __builtin_nontemporal_store(v, (u32x4*)(dst + 8 * l_e));   // streamed: this launch never reads it
  }
  if (tid_e < 128 && row0 + tid_e < row_end) {
    const int rr = tid_e;
    const float lse_v = stats[2 * rr + 1];
    if (!part) {
      a.lse[(size_t)b * R + row0 + rr] = lse_v;
    } else {
      *(float2*)(a.ws_lse + 2 * (prow + rr)) = float2{lse_v, stats[2 * rr]};
    }
  }
  if (part && tid_e < kLoMaskWords) a.ws_lo_mask[(size_t)slot * kLoMaskWords + tid_e] = lo_mask_word(amax, tid_e, row_end - row0);
}

// ===== 128 rows: half pages through a four-slot ring =====================================
// The page stream moves in half pages (32 tokens, 36,864 B) through a ring of four LDS
// slots.  Each wave scores its own 32 rows (S^T = K . Q^T, one MFMA chain over the 36
// 16-dim steps) and takes their softmax; its bf16 P goes to a double-buffered P area
// after the ring.  P.V is split by value columns: wave w accumulates O^T over value
// tiles 4w .. 4w+3 for all four row tiles (all 256 AGPRs), so a half page's V is read
// from LDS once per workgroup, and every wave reads the other waves' P.  The waves meet
// once per half page.  Iteration i runs P.V of half page i and the score MFMAs of half
// page i+1 as one interleaved schedule, the softmax of half page i+1 under its last P.V
// MFMAs; the copies of half page i+3 go out meanwhile, into the slot that half page i-1
// freed.  (Every instruction between two MFMAs must issue within the MFMA's 32 cycles:
// the schedule is built around that budget, with scalar work kept out of the slots.)
// A half page in LDS is 9 column blocks of 64 dims x 32 tokens (4 KB each, rope last):
// token t, 16-byte chunk p of block c at c*4096 + t*128 + (p ^ cswz(t))*16.
constexpr int kHalf = 32;                          // tokens per half page
constexpr int kSlotBytes = kHalf * kRowBytes;      // 36864
constexpr int kSlotBlock = kHalf * 128;            // 4096: one column block of a half page
constexpr int kRingScratch = 4 * kSlotBytes;       // 147456: the P area after the ring
static_assert(kRingScratch + 2 * 8192 <= kLdsBytes, "ring and P area fit the LDS");
constexpr int kRingPK = 2;                         // K-fragment prefetch distance (score steps)

struct HalfPage {
  const uint8_t* base;   // page start in the pool
  int tok0;              // 0 or 32: which half of the page
  int valid;             // tokens of the page in the sequence (later tokens read token 0)
};
// Half page h of a sequence (h counts 32-token halves from its start) held by pool page
// `page`; a page index outside the pool reads page 0 and poisons the segment.
__device__ __forceinline__ HalfPage half_page(const DecodeArgs& a, int page, int h, int Lc, bool& bad_page) {
  const bool bad = page < 0 || page >= a.num_pages;
  bad_page |= bad;
  return HalfPage{a.kv + (size_t)(bad ? 0 : page) * kBlockBytes, (h & 1) * kHalf,
                  bad ? 1 : min(kPage, Lc - (h >> 1) * kPage)};
}
// One wave-wide copy: column block i, tokens 8k .. 8k+7 of the half page, into `slot`.  The
// slot address is made opaque per copy, so that the destinations of a run of copies are
// each one scalar add here, not dozens of precomputed scalars held (and spilled) across it.
__device__ __forceinline__ void half_copy(const HalfPage& h, MLA_LDS uint8_t* slot, int i, int k, int l) {
  const int t = 8 * k + (l >> 3);
  const int tp = h.tok0 + t;
  const int te = tp < h.valid ? tp : 0;
  uint32_t dst = (uint32_t)(uintptr_t)slot;
  asm volatile("" : "+s"(dst));
  dma16(h.base, (uint32_t)(te * kRowBytes + i * 128 + (((l & 7) ^ cswz(t)) << 4)),
        (MLA_LDS uint8_t*)(uintptr_t)(dst + (uint32_t)(i * kSlotBlock + k * 1024)));
}
// The lane's byte offset in a half page for the copies of tokens 8k .. 8k+7 (column block 0;
// block i adds 128 i): formed once per half page, so that each copy is one vector add and
// one scalar add.
__device__ __forceinline__ uint32_t half_copy_lane(const HalfPage& h, int k, int l) {
  const int t = 8 * k + (l >> 3);
  const int tp = h.tok0 + t;
  const int te = tp < h.valid ? tp : 0;
  return __umul24((uint32_t)te, (uint32_t)kRowBytes) + (uint32_t)(((l & 7) ^ cswz(t)) << 4);
}
// P.V MFMA with no wait states ahead: for operands that no vector instruction has just
// written (LDS reads, or registers written many instructions earlier).
__device__ __forceinline__ void mfma_pv_ds(f32x16& o, const bf16x8& v, const bf16x8& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}
// Score MFMA of one chain (accumulator in VGPRs); `first` starts the chain from zero.
__device__ __forceinline__ void mfma_s(f32x16& acc, const bf16x8& k, const bf16x8& q, bool first) {
  if (first)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "v"(q));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "v"(q));
}
// MFMA results retire before vector instructions read their accumulators.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 4" : : : "memory"); }

__device__ __forceinline__ void decode_segment_cols(const DecodeArgs& a, MLA_LDS uint8_t* lds, int b, int row0,
                                                    int blk_lo, int blk_hi, int slot) {
  const int w = wave_id(), l = threadIdx.x & 63;
  const int g = l >> 5, lr = l & 31;
  const int R = a.rows;
  const int row_end = min(row0 + a.rows_per_wg, R);
  const int myrow = row0 + 32 * w + lr;
  const float c = a.scale_log2;

  // The sequence's length and the page of half pages 0 and 1 (scalar loads) go out
  // together, and Q's loads are issued while they are in flight: no vector load waits for
  // a scalar round trip, and the two round trips overlap.  blk_lo < blk_hi <= max_blocks,
  // so the entry is inside the block table's row.
  const int* bt_row = a.block_table + (size_t)b * a.bt_stride;
  const int L = ld_const(a.seqlens, b);
  const int pg01 = blk_lo < blk_hi ? ld_const(bt_row, blk_lo) : 0;
  // ---- Q: each lane loads its row's fragments straight into registers (dims 16kk + 8g .. +8
  // of row myrow: the B operand of S^T = K . Q^T).  A row past the workgroup's reads row
  // row0; it is scored but never stored.
  bf16x8 qf[36];
  {
    int tq = threadIdx.x;   // opaque: the address is formed here, not kept across the kernel
    asm volatile("" : "+v"(tq));
    // a scalar base for the workgroup's rows and a 32-bit lane offset (under 148 KB)
    const uint8_t* qb = a.q + ((size_t)b * R + row0) * kRowBytes;
    const int rq = 32 * w + (tq & 31);
    const uint32_t qo = (uint32_t)((row0 + rq < row_end ? rq : 0) * kRowBytes + 16 * ((tq >> 5) & 1));
#pragma unroll
    for (int kk = 0; kk < 36; ++kk) qf[kk] = *(const bf16x8*)(qb + qo + 32 * kk);
  }
  // more keys than the block table's row can hold: ceil(L / kPage) > max_blocks, in 32 bits
  const bool bad_len = (L < 0) || (L > 0 && (L - 1) / kPage >= a.max_blocks);
  const int Lc = bad_len ? 0 : L;
  const int hp0 = 2 * blk_lo;                                                   // first half page
  const int H = max(0, (min(blk_hi * kPage, Lc) + kHalf - 1) / kHalf - hp0);   // half pages with keys
  bool bad_page = false;
  // P of two half pages after the ring: [half page & 1][row tile][K step][lane] x 16 B.
  // After the page loop the same bytes hold the workgroup-OR words and the row statistics.
  MLA_LDS uint8_t* pbuf = lds + kRingScratch;
  MLA_LDS int* or_words = (MLA_LDS int*)pbuf;

  __syncthreads();   // LDS free (a previous segment may still be reading it)
  // Half page n (0 or 1) into slot n, each wave its 9 pieces (tokens 8w .. 8w+7).  The
  // lane index comes from an opaque copy of the thread index, so that the copies' lane
  // terms are formed here and not kept (spilled) across the kernel; a reload between these
  // copies would wait for all of them.
  auto first_copy = [&](int n) {
    if (n < H) {
      int tl = threadIdx.x;
      asm volatile("" : "+v"(tl));
      const HalfPage h = half_page(a, pg01, hp0 + n, Lc, bad_page);
#pragma unroll
      for (int i = 0; i < 9; ++i) half_copy(h, lds + n * kSlotBytes, i, w, tl & 63);
    }
  };
  // Q's 36 loads, then half pages 0 and 1: the first score loop starts once Q and half page
  // 0 are in.  At most 54 loads are in flight per wave, under the 63 the counter holds.
  first_copy(0);
  first_copy(1);
  // Causal rows' visible keys, formed here from an opaque copy of the flag (a flag the
  // compiler kept from the kernel's start was reloaded from scratch right after the copies,
  // and that reload waited for all of them).
  int causal = a.causal, qlen = a.q_len;
  asm volatile("" : "+s"(causal), "+s"(qlen));
  causal = causal && qlen > 1;
  int nvis = Lc;
  if (causal) nvis = Lc - a.q_len + 1 + min(myrow, R - 1) / a.heads;
  nvis = max(nvis, 0);
  int nmin = Lc;   // fewest visible keys over the wave's rows: masking starts there
  if (causal) nmin = max(Lc - a.q_len + 1 + min(row0 + 32 * w, R - 1) / a.heads, 0);
  // lane terms of the K reads (token lr, dims 16kk + 8g) and the transposing V reads
  int ky[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) ky[m] = lr * 128 + (((2 * m + g) ^ cswz(lr)) << 4);
  const int jj = l & 15, qh = (l >> 4) & 1;
  const int tv = 4 * g + (jj >> 2);
  const int v_base = tv * 128 + 8 * (jj & 1);
  int vy[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int r = 0; r < 2; ++r) vy[e][r] = v_base + 1024 * r + (((4 * e + 2 * qh + ((jj & 3) >> 1)) ^ cswz(tv + 8 * r)) << 4);

  f32x16 o[16];   // O^T: value tile 4w + vt (values 128w + 32vt ..), row tile (w + r) % 4 at o[4 vt + r]
  float m_ref = -INFINITY, mtrue = -INFINITY, lsum = 0.f;
  bool over = false, bad_wg = false;   // bad_wg: some wave read a bad page
  float mref_init = -INFINITY;
  for (int pass = 0; pass < 2; ++pass) {
    m_ref = mref_init;
    mtrue = -INFINITY;
    lsum = 0.f;
    over = false;
    // zeros from an opaque scalar formed in this pass (a plain zero vector is one value the
    // compiler would keep, and spill, from the kernel's start to every pass)
    int zi = 0;
    asm volatile("" : "+s"(zi));
    const float zf = __int_as_float(zi);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      o[t] = f32x16{zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf, zf};
      asm volatile("" : "+a"(o[t]));
    }
    if (pass == 1) {                // the second pass streams them again
      first_copy(0);
      first_copy(1);
    }

    // Wait for half page n, then meet the other waves: it has landed in every wave's copies,
    // every wave's P of half page n-1 is in the P buffer, and every wave is past P.V of half
    // page n-2 (its slot and P buffer are free).  Every wave issues 9 copies per half page,
    // in half-page order, and at the wait for half page n only half page n+1 can be in
    // flight behind it.
    auto wait_half = [&](int n) {
      if (n + 1 < H) asm volatile("s_waitcnt vmcnt(9)" : : : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      __syncthreads();
    };
    // The wait for half page 0 (and, in the first pass, Q's loads issued before it): only
    // half page 1's copies may still be in flight behind it.
    auto wait_first = [&]() { wait_half(0); };

    f32x16 sc;                    // the score chain, then the softmax's terms in place
    u32x4 pn0, pn1;               // the wave's own P (bf16 B operands of the two K steps)
    float rs = 0.f, rmax = -INFINITY, msub = 0.f;
    auto sm_mask = [&](f32x16& s, int hpa) {
      if ((hpa + 1) * kHalf > nmin) {
        asm volatile("");
        // element e holds token 8(e/4) + 4g + e%4 of the half page; lim is formed here (an
        // opaque value), so that the compares stay inside this rarely taken branch
        int lz = threadIdx.x;
        asm volatile("" : "+v"(lz));
        const int lim = nvis - hpa * kHalf - 4 * ((lz >> 5) & 1);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = (8 * (e >> 2) + (e & 3) < lim) ? s[e] : -INFINITY;
      }
    };
    // Softmax set-up of the (masked) scores in sc: the reference max where the row has none
    // yet, from these scores and `extra` (the lane's max over the rest of the page).
    auto sm_ref = [&](float extra) {
      if (__builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0) {
        float mr = extra;
#pragma unroll
        for (int e = 0; e < 16; ++e) mr = fmaxf(mr, sc[e]);
        const float mx = half_max(mr) * c;
        if (m_ref == -INFINITY) m_ref = mx;   // nothing accumulated yet: exact
      }
      msub = (m_ref == -INFINITY) ? 0.f : m_ref;
      rs = 0.f;
      rmax = -INFINITY;
    };
    auto sm_elem = [&](int e) {
      rmax = fmaxf(rmax, sc[e]);
      sc[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], c, -msub));
      rs += sc[e];
    };
    auto sm_pack = [&](int m) {
      const uint32_t x = pack_bf16x2(sc[4 * m], sc[4 * m + 1]), y = pack_bf16x2(sc[4 * m + 2], sc[4 * m + 3]);
      if (m < 2) { pn0[2 * m] = x; pn0[2 * m + 1] = y; }
      else { pn1[2 * (m - 2)] = x; pn1[2 * (m - 2) + 1] = y; }
    };
    // After the 16 terms: this lane's half of the row sum.  No term exceeds 2^kRefSlack
    // unless this half-row sum does (an overflow to inf included), and only then does the
    // row take the half page's max, for the second pass's bound.
    auto sm_finish = [&]() {
      lsum += rs;
      if (__builtin_amdgcn_ballot_w64(rs > kSumCap) != 0) {
        over |= rs > kSumCap;
        mtrue = fmaxf(mtrue, rmax * c);
      }
    };
    auto softmax_alone = [&](float extra) {
      sm_ref(extra);
#pragma unroll
      for (int e = 0; e < 16; ++e) sm_elem(e);
#pragma unroll
      for (int m = 0; m < 4; ++m) sm_pack(m);
      sm_finish();
    };
    // The wave's P of half page n into the P buffer: row tile w, both K steps.
    auto put_p = [&](int n) {
      MLA_LDS uint8_t* pb = pbuf + (n & 1) * 8192 + (2 * w * 64 + l) * 16;
      *(MLA_LDS u32x4*)pb = pn0;
      *(MLA_LDS u32x4*)(pb + 64 * 16) = pn1;
    };
    // (poff: byte offset of the half page's P buffer, (n & 1) * 8192)
    auto put_p_half = [&](uint32_t poff, int ks) {
      MLA_LDS uint8_t* pb = pbuf + poff + ((2 * w + ks) * 64 + l) * 16;
      *(MLA_LDS u32x4*)pb = ks == 0 ? pn0 : pn1;
    };
    auto get_p = [&](uint32_t poff, int rt, int ks) {
      return lds_read_b128(pbuf + poff + ((2 * rt + ks) * 64 + l) * 16);
    };
    // Score loop over the half page in `ks` alone: one MFMA per step (one dependent chain
    // issues at the full MFMA rate); when cp, this wave's 9 copies of `nxt` into `nslot` go
    // out at steps 2, 6, ..., 34, each behind its step's MFMA.  Ends with the scores in sc.
    auto score = [&](const MLA_LDS uint8_t* ks, bool cp, const HalfPage& nxt, MLA_LDS uint8_t* nslot) {
      auto load_k = [&](int kk) { return lds_read_b128(ks + (kk >> 2) * kSlotBlock + ky[kk & 3]); };
      bf16x8 kr[kRingPK + 1];
      int lc = threadIdx.x;                  // lane index formed here, not kept across the kernel
      asm volatile("" : "+v"(lc));
      const uint32_t coff = cp ? half_copy_lane(nxt, w, lc & 63) : 0u;
      MLA_LDS uint8_t* nw = nslot + w * 1024;
#pragma unroll
      for (int kk = 0; kk < kRingPK; ++kk) kr[kk] = load_k(kk);
#pragma unroll
      for (int kk = 0; kk < 36; ++kk) {
        if (kk + kRingPK < 36) kr[(kk + kRingPK) % (kRingPK + 1)] = load_k(kk + kRingPK);
        mfma_s(sc, kr[kk % (kRingPK + 1)], qf[kk], kk == 0);
        if (cp && (kk & 3) == 2) dma16(nxt.base, coff + (kk >> 2) * 128, nw + (kk >> 2) * kSlotBlock);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_drain();
    };
    // V^T fragment of value tile 4w + vt, K step ks, of the half page in slot `vs`.
    auto load_v = [&](const MLA_LDS uint8_t* vs, int vt, int ks) {
      const int t = 4 * w + vt;
      const MLA_LDS uint8_t* vp = vs + ks * 16 * 128 + (t >> 1) * kSlotBlock;
      return cat8(lds_read_tr(vp + vy[t & 1][0]), lds_read_tr(vp + vy[t & 1][1]));
    };
    // P.V of half page n as 32 steps q: K step q/16, value tile (q/4)%4, row tile
    // (w + q%4)%4, so that each step group starts on the wave's own row tile, whose P is
    // still in registers (pn0, pn1).  V fragments: one group ahead, in vq[group & 1]; the
    // last group reads the next half page's first one (slot `nvs`).  Other row tiles' P
    // come from the P buffer: K step 0's at the start, K step 1's each right after its
    // last K-step-0 use.
    bf16x8 vq[2];
    bf16x8 pq[3];                 // P of row tiles w+1, w+2, w+3 for the current K step
    auto pv_begin = [&](uint32_t poff) {
#pragma unroll
      for (int r = 1; r < 4; ++r) pq[r - 1] = get_p(poff, (w + r) & 3, 0);
    };
    auto pv_step = [&](uint32_t poff, const MLA_LDS uint8_t* vs, const MLA_LDS uint8_t* nvs, bool pre, int q) {
      const int ks = q >> 4, vt = (q >> 2) & 3, r = q & 3;
      if (r == 0) {
        const int gq = (q >> 2) + 1;   // the next group
        if (gq < 8) vq[gq & 1] = load_v(vs, gq & 3, gq >> 2);
        else if (pre) vq[0] = load_v(nvs, 0, 0);
      }
      const bf16x8 pb = (r == 0) ? __builtin_bit_cast(bf16x8, ks == 0 ? pn0 : pn1) : pq[r - 1];
      mfma_pv_ds(o[4 * vt + r], vq[(q >> 2) & 1], pb);   // o[4 vt + r]: row tile (w + r) % 4
      if (ks == 0 && vt == 3 && r > 0) pq[r - 1] = get_p(poff, (w + r) & 3, 1);
    };
    auto pv_alone = [&](int n, const MLA_LDS uint8_t* vs, bool pre, const MLA_LDS uint8_t* nvs) {
      pv_begin((n & 1) * 8192);
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        pv_step((n & 1) * 8192, vs, nvs, pre, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // One fused iteration i (1 <= i <= H-2), after the barrier at its top: P.V of half page
    // i (slot i&3), the scores of half page i+1 (slot (i+1)&3) and their softmax, as one
    // schedule of 68 MFMA slots:
    //   0-1    P.V steps 0-1 (the first on registers alone: V read ahead, the wave's own P);
    //   2-49   16 x (score, score, P.V): score steps 0-31, P.V steps 2-17;
    //   50-53  score steps 32-35;
    //   54-67  P.V steps 18-31 with the softmax between them; its K-step-1 P replaces pn1
    //          only after P.V step 28, the last to read it.
    // Then the wave's new P goes to the P buffer (other waves read it after the next barrier).
    // The 9 copies of half page i+3 into slot (i+3)&3 go out every 7 slots from slot 5.
    HalfPage nn{};                // the next iteration's copy source, formed in slot 14
    int pg_ahead = 0;             // page entry of the half page after it
    auto fused = [&](int i, auto cp_tag, auto pos_tag, const HalfPage& nxt) {
      constexpr bool cp = decltype(cp_tag)::value;
      // ring position i & 3 (a template value, or -1: taken from i)
      constexpr int RS = decltype(pos_tag)::value;
      const int R = RS >= 0 ? RS : (i & 3);
      const uint32_t kso = ((R + 1) & 3) * kSlotBytes, vso = R * kSlotBytes, nso = ((R + 3) & 3) * kSlotBytes;
      const MLA_LDS uint8_t* ks = lds + kso;
      const MLA_LDS uint8_t* vs = lds + vso;
      MLA_LDS uint8_t* nslot = lds + nso + w * 1024;
      int lc = threadIdx.x;                  // lane index formed here, not kept across the kernel
      asm volatile("" : "+v"(lc));
      const uint32_t coff = cp ? half_copy_lane(nxt, w, lc & 63) : 0u;
      auto load_k = [&](int kk) { return lds_read_b128(ks + (kk >> 2) * kSlotBlock + ky[kk & 3]); };
      bf16x8 kr[kRingPK + 1];
      // P buffers by half-page parity
      const uint32_t pcur = (R & 1) * 8192, pnxt = ((R + 1) & 1) * 8192;
      pv_begin(pcur);
#pragma unroll
      for (int kk = 0; kk < kRingPK; ++kk) kr[kk] = load_k(kk);
      auto s_step = [&](int kk) {
        if (kk + kRingPK < 36) kr[(kk + kRingPK) % (kRingPK + 1)] = load_k(kk + kRingPK);
        mfma_s(sc, kr[kk % (kRingPK + 1)], qf[kk], kk == 0);
      };
      // what slot j carries besides its MFMA: a copy, or a piece of the softmax (each
      // piece's results pass through an empty asm statement, which keeps the piece in its
      // slot: pure arithmetic would otherwise sink to its first use)
      auto extra = [&](int j) {
        if (cp && j % 7 == 5) dma16(nxt.base, coff + (j / 7) * 128, nslot + (j / 7) * kSlotBlock);
        if (cp && j == 14 && i + 4 < H) {    // half page i+4's source
          if ((R & 1) == 0) {                // a new page: its entry came in at the top
            nn = half_page(a, pg_ahead, hp0 + i + 4, Lc, bad_page);
            asm volatile("" : "+s"(nn.base), "+s"(nn.tok0), "+s"(nn.valid));
          } else {                           // the second half of half page i+3's page
            nn.tok0 = kHalf;
          }
        }
        // the softmax terms: slot 55 (the last score MFMA's result has retired) takes the
        // set-up and term 0, slots 56-58 two terms each, slots 59-66 one or two more
        constexpr int kT0[12] = {0, 1, 3, 5, 7, 8, 9, 10, 11, 12, 13, 15};   // first term of slot 55 + n
        if (j >= 55 && j <= 66) {
          if (j == 55) {
            mfma_drain();
            sm_mask(sc, hp0 + i + 1);
            sm_ref(-INFINITY);
          }
          const int e0 = kT0[j - 55], e1 = (j == 66) ? 16 : kT0[j - 54];
#pragma unroll
          for (int e = e0; e < e1; ++e) {
            sm_elem(e);
            asm volatile("" : "+v"(sc[e]), "+v"(rs));
          }
        }
        if (j == 58 || j == 59) {            // pn0 is free after P.V step 12 (slot 34)
          sm_pack(j - 58);
          asm volatile("" : "+v"(pn0));
        }
        if (j == 60) put_p_half(pnxt, 0);
        if (j == 65 || j == 66) {            // pn1 after P.V step 28 (slot 64)
          sm_pack(2 + (j - 65));
          asm volatile("" : "+v"(pn1));
        }
        if (j == 66) {
          sm_finish();
          put_p_half(pnxt, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
#pragma unroll
      for (int q = 0; q < 2; ++q) {          // slots 0-1
        pv_step(pcur, vs, ks, true, q);
        extra(q);
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) {         // slots 2-49
        s_step(2 * m);
        extra(2 + 3 * m);
        s_step(2 * m + 1);
        extra(3 + 3 * m);
        pv_step(pcur, vs, ks, true, 2 + m);
        extra(4 + 3 * m);
      }
#pragma unroll
      for (int kk = 32; kk < 36; ++kk) {     // slots 50-53
        s_step(kk);
        extra(18 + kk);
      }
#pragma unroll
      for (int q = 18; q < 32; ++q) {        // slots 54-67
        pv_step(pcur, vs, ks, true, q);
        extra(36 + q);
      }
    };

    if (H > 0) {
      pg_ahead = (H > 4) ? ld_const(bt_row, (hp0 + 4) >> 1) : 0;   // page of half page 4
      // half pages 2 and 3 go out in the first two score loops
      HalfPage h2{}, h3{};
      if (H > 2) h2 = half_page(a, ld_const(bt_row, (hp0 + 2) >> 1), hp0 + 2, Lc, bad_page);
      if (H > 3) h3 = half_page(a, ld_const(bt_row, (hp0 + 3) >> 1), hp0 + 3, Lc, bad_page);
      // Half pages 0 and 1 are scored before the first softmax, so that a row's reference
      // max comes from the segment's whole first page, as keys are laid out in pages.
      wait_first();
      score(lds, H > 2, h2, lds + 2 * kSlotBytes);
      sm_mask(sc, hp0);
      f32x16 s1 = sc;
      float ex = -INFINITY;
      if (H > 1) {
        wait_half(1);
        score(lds + kSlotBytes, H > 3, h3, lds + 3 * kSlotBytes);
        sm_mask(sc, hp0 + 1);
#pragma unroll
        for (int e = 0; e < 16; ++e) ex = fmaxf(ex, sc[e]);
        const f32x16 t = sc;
        sc = s1;
        s1 = t;
      }
      softmax_alone(ex);                     // half page 0
      put_p(0);
      vq[0] = load_v(lds, 0, 0);
      __syncthreads();                       // every wave's P of half page 0
      pv_alone(0, lds, H > 1, lds + kSlotBytes);
      if (H > 1) {
        sc = s1;
        softmax_alone(-INFINITY);            // half page 1 (its P goes to the other buffer)
        put_p(1);
      }
      // Iterations that copy half page i+3, then the last two that do not: two copies of the
      // fused schedule, so that no copy carries a branch.
      if (H > 4) nn = half_page(a, pg_ahead, hp0 + 4, Lc, bad_page);
      int i = 1;
      for (; i + 3 < H; ++i) {
        const HalfPage nxt = nn;             // half page i+3
        // Even i: the page entry of half page i+4 (the next page), a scalar load issued
        // before the barrier and waited for right after it.  Scalar loads share the LDS
        // wait counter and may return out of order, so one still in flight would turn the
        // iteration's LDS waits into full waits.
        if ((i & 1) == 0) pg_ahead = ld_const(bt_row, (hp0 + min(i + 4, H - 1)) >> 1);
        wait_half(i + 1);
        asm volatile("" : : "s"(pg_ahead));
        fused(i, BoolC<true>{}, IntC<-1>{}, nxt);
      }
      for (; i + 1 < H; ++i) {
        wait_half(i + 1);
        fused(i, BoolC<false>{}, IntC<-1>{}, HalfPage{});
      }
      if (H > 1) {                           // the last half page
        __syncthreads();                     // every wave's P of it
        pv_alone(H - 1, lds + ((H - 1) & 3) * kSlotBytes, false, lds);
      }
    }
    mfma_drain();
    // One OR (its barriers: every slot is idle) gives both the second-pass flag and the
    // bad-page flag (the second pass streams the same pages, so it gives the same one).
    const int flags = wg_or_bits((over ? 1 : 0) | (bad_page ? 2 : 0), or_words);
    bad_wg = (flags & 2) != 0;
    if (!(flags & 1)) break;
    // Second pass from an upper bound of every score of the row: half pages that did not
    // flag stayed within m_ref + kRefSlack, the flagged ones gave their maxima.
    {
      const float mt = fmaxf(mtrue, m_ref + kRefSlack);
      mref_init = fmaxf(mt, __shfl_xor(mt, 32, 64));
    }
  }

  // ---- epilogue: every wave needs the row statistics of all 128 rows ---------------------
  const bool poison = bad_len || bad_wg;
  if (poison && a.meta && threadIdx.x == 0) a.meta[kHdrError] = 1;
  MLA_LDS float* stats = (MLA_LDS float*)pbuf + 16;   // [row][scale_o, lse], after the OR words
  MLA_LDS float* amax = stats + 2 * 128;              // [wave][row]: largest |o| over the wave's columns
  lsum += __shfl_xor(lsum, 32, 64);                   // the row's two halves
  int tid_e = threadIdx.x;                            // lane terms formed after the loop (not kept across it)
  asm volatile("" : "+v"(tid_e));
  const int l_e = tid_e & 63, g_e = l_e >> 5, lr_e = l_e & 31;
  if (g_e == 0) {
    const int rr = 32 * w + lr_e;
    float so, lse_v;
    if (poison) {
      so = __builtin_nanf("");
      lse_v = __builtin_nanf("");
    } else if (slot < 0 && a.sinks) {
      const SinkFold f = fold_sink<true>(m_ref, lsum, a.sinks[(row0 + rr) % a.heads] * kLog2e);
      so = f.scale_o;
      lse_v = f.lse * kLn2;
    } else {
      const bool empty = lsum == 0.f;   // no visible key; NaN propagates
      so = empty ? 0.f : 1.f / lsum;
      lse_v = empty ? -INFINITY : (m_ref + __log2f(lsum)) * kLn2;
    }
    stats[2 * rr] = so;
    stats[2 * rr + 1] = lse_v;
  }
  __syncthreads();
  // O goes through the idle ring as bf16 so that every store writes a whole 1 KB row: row rr
  // at rr*1024, 16-byte chunk cc (values 8cc .. 8cc+7) at (cc ^ (rr & 15))*16.  An unsplit
  // row is normalised here.  A split partial stays unnormalised (the merge applies the
  // factor, stored beside its LSE: one multiply per row there instead of 512 here), and
  // the same pass takes each row's largest |o| over the wave's columns, in normalised units.
  const bool part = slot >= 0;
  const size_t prow = (size_t)slot * a.rows_per_wg;   // the partial slot's first row
  auto stage = [&](auto norm_tag) {
    constexpr bool kNorm = decltype(norm_tag)::value;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 32 * ((w + r) & 3) + lr_e;
      const float so = stats[2 * rr];
      float mx = 0.f;
#pragma unroll
      for (int vt = 0; vt < 4; ++vt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x16& t = o[4 * vt + r];
          float x0 = t[4 * i], x1 = t[4 * i + 1], x2 = t[4 * i + 2], x3 = t[4 * i + 3];
          if constexpr (kNorm) {
            x0 *= so;
            x1 *= so;
            x2 *= so;
            x3 *= so;
          } else {
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))));
          }
          const int cc = 16 * w + 4 * vt + i;
          *(MLA_LDS u32x2*)(lds + rr * 1024 + ((cc ^ (rr & 15)) << 4) + 8 * g_e) =
              u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      if constexpr (!kNorm) {
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * so;   // over the wave's 128 columns of the row
        if (g_e == 0) amax[w * 128 + rr] = mx;
        if (mx > kLoCut && row0 + rr < row_end)        // this quarter of the row keeps its low half
          store_lo_quarter(a.ws_lo + (prow + rr) * kDv + 128 * w + 4 * g_e, [&](int vt) -> const f32x16& { return o[4 * vt + r]; });
      }
    }
  };
  if (part) stage(BoolC<false>{});
  else stage(BoolC<true>{});
  __syncthreads();
  for (int k = 0; k < 32; ++k) {                      // the wave's rows 32w .. 32w+31
    const int rr = 32 * w + k;
    if (row0 + rr >= row_end) break;                  // uniform
    const u32x4 v = *(const MLA_LDS u32x4*)(lds + rr * 1024 + ((l_e ^ (rr & 15)) << 4));
    uint16_t* dst = part ? a.ws_hi + (prow + rr) * kDv : a.out + ((size_t)b * R + row0 + rr) * kDv;
    __builtin_nontemporal_store(v, (u32x4*)(dst + 8 * l_e));   // streamed: this launch never reads it
  }
  if (tid_e < 128 && row0 + tid_e < row_end) {
    const int rr = tid_e;
    const float lse_v = stats[2 * rr + 1];
    if (!part) {
      a.lse[(size_t)b * R + row0 + rr] = lse_v;
    } else {
      *(float2*)(a.ws_lse + 2 * (prow + rr)) = float2{lse_v, stats[2 * rr]};
    }
  }
  if (part && tid_e < kLoMaskWords) a.ws_lo_mask[(size_t)slot * kLoMaskWords + tid_e] = lo_mask_word(amax, tid_e, row_end - row0);
}

// ===== a decode launch that plans for itself =============================================
// Blocks of unit-holding sequence b, as the planner counts them.
__device__ __forceinline__ int plan_blocks(const DecodeArgs& a, int b) {
  int64_t L = a.plan_uniform_len > 0 ? a.plan_uniform_len : ld_const(a.seqlens, b);
  if (L < 0) L = 0;
  return (int)min<int64_t>((L + kPage - 1) / kPage, a.max_blocks);
}
// The whole planner computation on the lengths given to this launch, in LDS (idle until
// the first segment starts); the workgroup numbered 0 also writes the plan, which the
// combine reads.  Then this workgroup's share: its range, and the split units at its two
// ends (units strictly inside the range are whole, so unsplit).  The units after the
// first are walked in order, each starting where the previous one ended.
template <int NRT, bool SPARSE>
__device__ __forceinline__ void decode_replanned(const DecodeArgs& a, MLA_LDS uint8_t* lds, MetaView v, int wg) {
  constexpr int kOffCu = 1024, kOffNe = kOffCu + 4 * (kPlanLdsBatch + 1), kOffRed = kOffNe + 4 * (kPlanLdsBatch + 1);
  constexpr int kOffBp = kOffRed + 32, kOffBc = kOffBp + 4 * (kPlanLdsWg + 1), kOffErr = kOffBc + 4 * (kPlanLdsWg + 1);
  constexpr int kOffShare = kOffErr + 4;
  static_assert(kOffShare + 4 * kShareWords <= kRingScratch, "the planner's LDS fits the ring");
  const PlanLds L{(int32_t*)(lds), (int32_t*)(lds + kOffCu), (int32_t*)(lds + kOffNe), (int64_t*)(lds + kOffRed),
                  (int32_t*)(lds + kOffBp), (int32_t*)(lds + kOffBc), (int32_t*)(lds + kOffErr),
                  (int32_t*)(lds + kOffShare)};
  const PlanParams p{a.seqlens, a.batch, a.rows, a.row_split, (int)gridDim.x, a.plan_min_blocks, a.max_blocks,
                     a.plan_max_partials, a.plan_fixed_blocks, a.plan_split_rule, a.plan_seg_cost, a.plan_uniform_len};
  // The table form's LDS lies in ring slots 2 and 3, apart from plan_core's (which it
  // leaves to when it does not apply) and from the first two half pages' copies; the
  // segment's first barrier comes before any copy into it.
  static_assert(4 * kTablesLdsWords <= 2 * kSlotBytes && kOffShare + 4 * kShareWords <= 2 * kSlotBytes,
                "the planners' LDS fits");
  int sh[kShareWords];
  if (plan_share_wave(p, v, wg == 0, wg, sh)) {
    // even batches of up to 64 sequences: registers only
  } else if (plan_share_tables(p, v, wg == 0, wg, sh, (MLA_LDS int32_t*)(lds + 2 * kSlotBytes))) {
    // ragged batches of up to 256 sequences: tables in LDS
  } else {   // the general case: the block-wide computation
    plan_core<true>(p, L, v, wg == 0, wg);
#pragma unroll
    for (int k = 0; k < kShareWords; ++k) sh[k] = L.share[k];
    __syncthreads();   // every wave has its share before the segments reuse the LDS
  }
  // the share as scalars (uniform over the workgroup)
  auto word = [&](int k) { return __builtin_amdgcn_readfirstlane(sh[k]); };
  if (wg >= word(kShareNumWg)) return;
  const int u_first = word(kShareUFirst), ns_first = word(kShareNsFirst);
  const int fw_first = word(kShareFirstWgFirst), poff_first = word(kSharePoffFirst);
  const int u_last = word(kShareULast), ns_last = word(kShareNsLast);
  const int fw_last = word(kShareFirstWgLast), poff_last = word(kSharePoffLast);
  const int rs = a.row_split;
  const int end = word(kShareEnd);
  int pos = word(kSharePos);
  int u = u_first;
  int unit_start = word(kShareStartFirst), nb = word(kShareNbFirst);
  while (pos < end) {
    const int b = u / rs, g = u - b * rs;
    const int blk_lo = pos - unit_start, blk_hi = min(end - unit_start, nb);
    int slot = -1;
    if (u == u_first) {
      if (ns_first > 1) slot = poff_first + (wg - fw_first);
    } else if (u == u_last) {
      if (ns_last > 1) slot = poff_last + (wg - fw_last);
    }
    if constexpr (NRT == 4 && !SPARSE) decode_segment_cols(a, lds, b, g * a.rows_per_wg, blk_lo, blk_hi, slot);
    else decode_segment_wide<NRT, SPARSE>(a, lds, b, g * a.rows_per_wg, blk_lo, blk_hi, slot);
    pos = unit_start + blk_hi;
    while (pos < end) {              // the next unit with blocks
      ++u;
      nb = plan_blocks(a, u / rs);
      if (nb > 0) break;
    }
    unit_start = pos;
  }
}

// ===== kernel ==========================================================================
// NRT = 32-row tiles per workgroup (1, 2 or 4).  REPLAN: the launch plans for itself (a
// plan made with plan_in_decode); each form is its own kernel, so that neither carries the
// other's code (a smaller binary to fetch at the start of every workgroup).
template <int NRT, bool SPARSE, bool REPLAN>
__global__ __launch_bounds__(256, 1) void mla_decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[kLdsBytes];
  MLA_LDS uint8_t* lds = (MLA_LDS uint8_t*)lds_raw;
  const bool planned = a.meta != nullptr;
  MetaView v = meta_view(a.meta, a.batch, a.row_split);
  // XCD-aware numbering: workgroups are dealt round-robin to the 8 XCDs, so logical
  // neighbours (the splits of one sequence) are made to share an XCD and its L2.
  int wg = blockIdx.x;
  if (planned && (gridDim.x & 7) == 0) wg = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if constexpr (REPLAN) {   // the host launches this form only with a plan (meta set)
    decode_replanned<NRT, SPARSE>(a, lds, v, wg);
    return;
  }
  int pos = 0, end = 1;                       // unsplit: one segment, the whole sequence
  int first_seq = -1;
  if (planned) {
    if (wg >= ld_const(v.hdr, kHdrNumWg)) return;
    pos = ld_const(v.wg_begin, wg);
    end = ld_const(v.wg_begin, wg + 1);
    first_seq = ld_const(meta_wg_seq(v, gridDim.x), wg);   // the plan's grid is the launch grid
  }
  const int rs = a.row_split;
  while (pos < end) {
    int b, g, blk_lo, blk_hi, slot;
    if (planned) {
      // sequence holding global position pos: the largest b with rs * cu_blocks[b] <= pos,
      // given by the plan for the workgroup's first segment
      if (first_seq >= 0) {
        b = first_seq;
        first_seq = -1;
      } else {
        int lo = 0, hi = a.batch - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (rs * ld_const(v.cu_blocks, mid) <= pos) lo = mid; else hi = mid - 1;
        }
        b = lo;
      }
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
    if constexpr (NRT == 4 && !SPARSE) decode_segment_cols(a, lds, b, g * a.rows_per_wg, blk_lo, blk_hi, slot);
    else decode_segment_wide<NRT, SPARSE>(a, lds, b, g * a.rows_per_wg, blk_lo, blk_hi, slot);
  }
}

}  // namespace mla

namespace {
// One launch of the decode kernel: a plain launch, or with events bound to the kernel's own
// start and end (hipExtLaunchKernelGGL), which adds no timing packet between launches.
template <int NRT, bool SPARSE, bool REPLAN>
void launch_decode_form(const mla::DecodeArgs& args, dim3 g, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (start || stop)
    hipExtLaunchKernelGGL((mla::mla_decode_bf16_kernel<NRT, SPARSE, REPLAN>), g, dim3(256), 0, stream, start, stop, 0,
                          args);
  else
    hipLaunchKernelGGL((mla::mla_decode_bf16_kernel<NRT, SPARSE, REPLAN>), g, dim3(256), 0, stream, args);
}
template <int NRT, bool SPARSE>
void launch_decode(const mla::DecodeArgs& args, dim3 g, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (args.meta && args.plan_in_decode) launch_decode_form<NRT, SPARSE, true>(args, g, stream, start, stop);
  else launch_decode_form<NRT, SPARSE, false>(args, g, stream, start, stop);
}
}  // namespace

extern "C" MLA_INTERNAL hipError_t mla_launch_decode_bf16(const mla::DecodeArgs* args, int grid, hipStream_t stream,
                                                       hipEvent_t start, hipEvent_t stop) {
  const int rpw = args->rows_per_wg;
  const bool sp = args->sparse_rows != nullptr;
  const dim3 g(grid);
  if (rpw > 64) {
    if (sp) launch_decode<4, true>(*args, g, stream, start, stop);
    else launch_decode<4, false>(*args, g, stream, start, stop);
  } else if (rpw > 32) {
    if (sp) launch_decode<2, true>(*args, g, stream, start, stop);
    else launch_decode<2, false>(*args, g, stream, start, stop);
  } else {
    if (sp) launch_decode<1, true>(*args, g, stream, start, stop);
    else launch_decode<1, false>(*args, g, stream, start, stop);
  }
  return hipGetLastError();
}

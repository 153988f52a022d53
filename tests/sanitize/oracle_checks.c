/* The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (built by
 * tests/test_sanitize_cpu.py with gcc): small seeded paged cases through every path of
 * mla_oracle_decode (fp32 and bf16 inputs, causal rows, attention sinks, sparse lists with
 * unused entries, a row subset, an empty sequence) and its refusals (bad arguments, a page
 * index outside the pool).  Prints "ALL OK" and exits 0 when every result is as expected. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mla_oracle_decode(const void* q, const void* kv, int32_t dtype, const int32_t* block_table, int64_t bt_stride,
                      const int32_t* cache_seqlens, int32_t batch, int32_t q_len, int32_t heads, int64_t num_pages,
                      int32_t page, int32_t d_qk, int32_t d_v, int32_t causal, double scale, const double* sinks,
                      const int32_t* indices, int32_t topk, const int64_t* rows, int64_t n_rows, double* out,
                      double* lse, int32_t n_threads);

static int failures = 0;
#define EXPECT(c)                                                     \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c);         \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint64_t st = 7;
static double unif(void) { /* xorshift64*, [0, 1) */
  st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
  return (double)((st * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}
static uint16_t bf16_of(float x) { uint32_t u; memcpy(&u, &x, 4); return (uint16_t)(u >> 16); }

enum { B = 3, T = 2, H = 4, PAGE = 8, DQK = 24, DV = 16, PAGES = 9, BLK = 3 };

int main(void) {
  const int32_t lens[B] = {20, 1, 0};
  int32_t bt[B * BLK];
  for (int i = 0; i < B * BLK; ++i) bt[i] = (i * 4 + 1) % PAGES;           /* a permutation of pages */
  float qf[B * T * H * DQK], kvf[PAGES * PAGE * DQK];
  uint16_t qb[B * T * H * DQK], kvb[PAGES * PAGE * DQK];
  for (int i = 0; i < B * T * H * DQK; ++i) { qf[i] = (float)(2 * unif() - 1); qb[i] = bf16_of(qf[i]); }
  for (int i = 0; i < PAGES * PAGE * DQK; ++i) { kvf[i] = (float)(2 * unif() - 1); kvb[i] = bf16_of(kvf[i]); }
  const int64_t rows = (int64_t)B * T * H;
  double* out = (double*)malloc(sizeof(double) * rows * DV);
  double* lse = (double*)malloc(sizeof(double) * rows);
  const double sinks[H] = {0.5, -1.0, -INFINITY, 2.0};
  for (int dtype = 0; dtype < 2; ++dtype) {
    const void* q = dtype ? (const void*)qb : (const void*)qf;
    const void* kv = dtype ? (const void*)kvb : (const void*)kvf;
    for (int causal = 0; causal < 2; ++causal)
      for (int sk = 0; sk < 2; ++sk) {
        EXPECT(mla_oracle_decode(q, kv, dtype, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, causal, 0.3,
                                 sk ? sinks : NULL, NULL, 0, NULL, 0, out, lse, 2) == 0);
        for (int64_t r = 0; r < rows; ++r) {
          const int b = (int)(r / (T * H));
          const int empty = !sk && (lens[b] == 0 || (causal && lens[b] - T + 1 + (int)((r / H) % T) <= 0));
          EXPECT(empty ? (isinf(lse[r]) && lse[r] < 0) : isfinite(lse[r]) || (sk && isinf(lse[r])));
          for (int d = 0; d < DV; ++d) EXPECT(isfinite(out[r * DV + d]));
        }
      }
    /* sparse lists: -1 entries skipped, positions in any order */
    int32_t idx[B * T * 5];
    for (int i = 0; i < B * T * 5; ++i) idx[i] = -1;
    idx[0] = 3; idx[1] = 19; idx[3] = 0; idx[5] = 7; idx[10] = 0;
    EXPECT(mla_oracle_decode(q, kv, dtype, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, 0, 0.3, NULL, idx, 5, NULL,
                             0, out, lse, 1) == 0);
    idx[1] = 20;   /* at the sequence's length: an input fault */
    EXPECT(mla_oracle_decode(q, kv, dtype, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, 0, 0.3, NULL, idx, 5, NULL,
                             0, out, lse, 1) == 2);
    /* a row subset */
    const int64_t some[3] = {rows - 1, 0, 5};
    EXPECT(mla_oracle_decode(q, kv, dtype, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, 1, 0.3, NULL, NULL, 0, some,
                             3, out, lse, 2) == 0);
    const int64_t outside[1] = {rows};
    EXPECT(mla_oracle_decode(q, kv, dtype, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, 1, 0.3, NULL, NULL, 0,
                             outside, 1, out, lse, 1) == 1);
  }
  /* a page index outside the pool, and refused arguments */
  int32_t badbt[B * BLK];
  memcpy(badbt, bt, sizeof bt);
  badbt[1] = PAGES;
  EXPECT(mla_oracle_decode(qf, kvf, 0, badbt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, 0, 0.3, NULL, NULL, 0, NULL, 0,
                           out, lse, 2) == 2);
  EXPECT(mla_oracle_decode(NULL, kvf, 0, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, 0, 0.3, NULL, NULL, 0, NULL, 0,
                           out, lse, 1) == 1);
  EXPECT(mla_oracle_decode(qf, kvf, 5, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DV, 0, 0.3, NULL, NULL, 0, NULL, 0,
                           out, lse, 1) == 1);
  EXPECT(mla_oracle_decode(qf, kvf, 0, bt, BLK, lens, B, T, H, PAGES, PAGE, DQK, DQK + 1, 0, 0.3, NULL, NULL, 0, NULL,
                           0, out, lse, 1) == 1);
  free(out);
  free(lse);
  if (failures == 0) printf("ALL OK\n");
  return failures == 0 ? 0 : 1;
}

// Host-side checks of libmla under AddressSanitizer and UndefinedBehaviorSanitizer (built by
// tests/test_sanitize_cpu.py with the sanitizers on the host pass only).  Everything here
// returns before any device work: status strings, the size queries over a sweep of problem
// shapes and planner options (extreme values included, for integer overflow), and every
// argument check the entry points make before they touch a stream.  Prints "ALL OK" and
// exits 0 when every status is the expected one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include "mla.h"

static int failures = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);      \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static mla_problem_t problem(int32_t batch = 4, int32_t q_len = 1, int32_t heads = 128) {
  mla_problem_t p;
  std::memset(&p, 0, sizeof(p));
  p.batch = batch;
  p.q_len = q_len;
  p.num_heads = heads;
  p.num_pages = 64;
  p.block_table_stride = 16;
  p.max_blocks_per_seq = 16;
  p.dtype = MLA_DTYPE_BF16;
  return p;
}

// A counter-based stream of picks (SplitMix64), so the sweep is the same on every run.
static uint64_t mix(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
template <size_t N>
static int32_t pick(uint64_t& s, const int32_t (&v)[N]) { return v[mix(s) % N]; }

int main() {
  for (int32_t c = -3; c < 20; ++c) EXPECT(mla_status_string(c) != nullptr && std::strlen(mla_status_string(c)) > 0);
  EXPECT(std::strcmp(mla_status_string(MLA_OK), "ok") == 0);

  // ---- size queries: never crash, never overflow, 0 for what the decode refuses ----------
  const int32_t big = INT32_MAX;
  const int32_t batches[] = {0, 1, 3, 64, 4200, 1 << 20, big, -1};
  const int32_t qlens[] = {1, 2, 4, 128, big, 0, -3};
  const int32_t heads[] = {1, 16, 32, 64, 128, 129, big, 0};
  const int32_t causal[] = {0, 1, 2};
  const int32_t pages[] = {1, 64, 1 << 20, big, 0, -1};
  const int32_t strides[] = {1, 16, 513, 1 << 16, big, 0};
  const int32_t blocks[] = {1, 16, 512, 1 << 16, big, 0};
  const int32_t dtypes[] = {MLA_DTYPE_F32, MLA_DTYPE_BF16, 7};
  const int32_t topks[] = {0, 0, 0, 8, 100, 2048, big, -1};
  const int32_t wgs[] = {0, 0, 1, 3, 256, 100000, big, -5};
  const int32_t mins[] = {0, 0, 1, 7, big, -1};
  const int32_t rsplit[] = {0, 0, 1, 2, 4, 3, -1};
  const int32_t fixed[] = {0, 0, 0, 1, 5, 4096, big, -2};
  const int32_t rules[] = {0, 0, 1, 2, 3, -1};
  const int32_t seg[] = {0, 0, 1, 64, big, -1};
  const int32_t cus[] = {1, 80, 256, 304, 1 << 16, big};
  uint64_t s = 12345;
  size_t nonzero = 0;
  for (int it = 0; it < 200000; ++it) {
    // a valid problem with up to four fields replaced by picks from the lists above
    mla_problem_t p = problem();
    mla_plan_options_t o;
    std::memset(&o, 0, sizeof(o));
    const int nmut = (int)(mix(s) % 5);
    for (int k = 0; k < nmut; ++k) {
      switch (mix(s) % 15) {
        case 0: p.batch = pick(s, batches); break;
        case 1: p.q_len = pick(s, qlens); break;
        case 2: p.num_heads = pick(s, heads); break;
        case 3: p.causal = pick(s, causal); break;
        case 4: p.num_pages = pick(s, pages); break;
        case 5: p.block_table_stride = pick(s, strides); break;
        case 6: p.max_blocks_per_seq = pick(s, blocks); break;
        case 7: p.dtype = pick(s, dtypes); break;
        case 8: p.topk = pick(s, topks); break;
        case 9: o.num_workgroups = pick(s, wgs); break;
        case 10: o.min_blocks_per_wg = pick(s, mins); break;
        case 11: o.row_split = pick(s, rsplit); break;
        case 12: o.fixed_split_blocks = pick(s, fixed); break;
        case 13: o.split_rule = pick(s, rules); break;
        default: o.segment_cost = pick(s, seg); break;
      }
    }
    const int32_t n = pick(s, cus);
    const bool use_o = (mix(s) & 1) != 0;
    const size_t mb = mla_metadata_bytes(&p, use_o ? &o : nullptr, n);
    const size_t wb = mla_workspace_bytes(&p, use_o ? &o : nullptr, n);
    EXPECT((mb == 0) == (wb == 0) || p.batch == 0);
    nonzero += mb != 0;
  }
  EXPECT(nonzero > 1000);   // the sweep reaches valid problems too

  // ---- argument checks before any launch (fake, never dereferenced pointers) --------------
  void* a = reinterpret_cast<void*>(0x10000);
  float* af = reinterpret_cast<float*>(0x10000);
  const int32_t* ai = reinterpret_cast<const int32_t*>(0x10000);
  mla_problem_t p = problem();
  EXPECT(mla_decode(nullptr, a, a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) == MLA_ERR_NULL);
  EXPECT(mla_decode(&p, nullptr, a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) == MLA_ERR_NULL);
  EXPECT(mla_decode(&p, reinterpret_cast<void*>(0x10008), a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) ==
         MLA_ERR_ALIGN);
  for (float bad : {0.f, -0.5f, INFINITY, NAN, 3e38f}) {
    mla_plan_t plan;
    std::memset(&plan, 0, sizeof(plan));
    plan.metadata = a;
    plan.metadata_bytes = mla_metadata_bytes(&p, nullptr, 256);
    plan.grid_wg = 256;
    plan.row_split = 1;
    plan.rows_per_wg = 128;
    plan.max_partials = 260;
    plan.batch = 4;
    plan.rows = 128;
    EXPECT(mla_decode(&p, a, a, ai, ai, bad, a, af, &plan, a, mla_workspace_bytes(&p, nullptr, 256), nullptr) ==
           MLA_ERR_SHAPE);
  }
  {
    mla_problem_t bad = problem(4, 1, 129);
    EXPECT(mla_decode(&bad, a, a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) == MLA_ERR_SHAPE);
    bad = problem();
    bad.dtype = 7;
    EXPECT(mla_decode(&bad, a, a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) == MLA_ERR_DTYPE);
    mla_problem_t zero = problem(0);
    EXPECT(mla_decode(&zero, nullptr, nullptr, nullptr, nullptr, 1.f, nullptr, nullptr, nullptr, nullptr, 0,
                      nullptr) == MLA_OK);
  }
  {
    const size_t mb = mla_metadata_bytes(&p, nullptr, 256);
    mla_plan_t plan;
    std::memset(&plan, 0, sizeof(plan));
    plan.metadata = a;
    plan.metadata_bytes = mb - 4;
    EXPECT(mla_get_metadata(&p, ai, nullptr, 256, &plan, nullptr) == MLA_ERR_WORKSPACE);
    plan.metadata = nullptr;
    plan.metadata_bytes = mb;
    EXPECT(mla_get_metadata(&p, ai, nullptr, 256, &plan, nullptr) == MLA_ERR_NULL);
    plan.metadata = reinterpret_cast<void*>(0x10004);
    EXPECT(mla_get_metadata(&p, ai, nullptr, 256, &plan, nullptr) == MLA_ERR_ALIGN);
    EXPECT(mla_get_metadata(nullptr, ai, nullptr, 256, &plan, nullptr) == MLA_ERR_NULL);
  }
  {
    mla_variant_t v;
    v.sinks = reinterpret_cast<const float*>(0x10002);
    v.indices = nullptr;
    EXPECT(mla_decode_ex(&p, &v, a, a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) == MLA_ERR_ALIGN);
    mla_problem_t sp = problem(4, 2, 128);
    sp.topk = 100;
    EXPECT(mla_decode(&sp, a, a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) == MLA_ERR_NULL);
    v.sinks = nullptr;
    v.indices = reinterpret_cast<const int32_t*>(0x10002);
    EXPECT(mla_decode_ex(&sp, &v, a, a, ai, ai, 1.f, a, af, nullptr, nullptr, 0, nullptr) == MLA_ERR_ALIGN);
  }
  EXPECT(mla_plan_error(nullptr, nullptr) == MLA_ERR_NULL);
  {
    uint32_t* sink = reinterpret_cast<uint32_t*>(0x200000);
    const size_t mib = 1 << 20;
    EXPECT(mla_hbm_read_probe(nullptr, mib, 0, 4, sink, nullptr) == MLA_ERR_NULL);
    EXPECT(mla_hbm_read_probe(a, mib, 2, 4, sink, nullptr) == MLA_ERR_UNSUPPORTED);
    EXPECT(mla_hbm_read_probe(a, 0, 0, 4, sink, nullptr) == MLA_ERR_SHAPE);
    EXPECT(mla_hbm_read_probe(a, (size_t)1 << 33, 0, 2, sink, nullptr) == MLA_ERR_SHAPE);
  }
  {
    EXPECT(mla_decode_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, nullptr, nullptr,
                              nullptr) == MLA_ERR_NULL);
    mla_problem_t bad = problem(4, 1, 129);
    EXPECT(mla_decode_noalloc(&bad, nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, nullptr, nullptr, nullptr) ==
           MLA_ERR_SHAPE);
    mla_problem_t sp = problem();
    sp.topk = 64;
    EXPECT(mla_decode_noalloc(&sp, nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, nullptr, nullptr, nullptr) ==
           MLA_ERR_UNSUPPORTED);
  }
  if (failures == 0) std::printf("ALL OK\n");
  return failures == 0 ? 0 : 1;
}

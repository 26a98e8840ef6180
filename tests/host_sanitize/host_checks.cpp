// Host-side checks of the library's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py builds and runs it on the
// CPU; no GPU is touched). It drives the host code paths that run without a device:
// the CLOCK residency table (random tables and selections, invariants after every
// step, rejected selections leaving the table unchanged), the host record encoder and
// f64 -> f16 rounding on random and special inputs, the size helpers on hostile
// shapes, and the argument checks of every entry point that enqueues device work
// (invalid arguments must be rejected before anything is enqueued).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "kvcache.h"

static int g_failures = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);    \
      ++g_failures;                                                              \
    }                                                                            \
  } while (0)

struct Table {
  std::vector<int32_t> slot_page, page_slot;
  std::vector<uint8_t> ref;
  kv_residency t{};
  Table(int32_t n_slots, int32_t n_pages) : slot_page(n_slots), page_slot(n_pages), ref(n_slots) {
    t.n_slots = n_slots;
    t.n_pages = n_pages;
    t.slot_page = slot_page.data();
    t.page_slot = page_slot.data();
    t.ref = ref.data();
    t.hand = 0;
  }
  bool same(const Table& o) const {
    return slot_page == o.slot_page && page_slot == o.page_slot && ref == o.ref && t.hand == o.t.hand;
  }
  void check_inverse() const {
    int32_t resident = 0;
    for (int32_t s = 0; s < t.n_slots; ++s) {
      const int32_t p = slot_page[s];
      if (p >= 0) {
        CHECK(p < t.n_pages);
        CHECK(page_slot[p] == s);
        ++resident;
      }
    }
    int32_t mapped = 0;
    for (int32_t p = 0; p < t.n_pages; ++p) {
      const int32_t s = page_slot[p];
      if (s >= 0) {
        CHECK(s < t.n_slots);
        CHECK(slot_page[s] == p);
        ++mapped;
      }
    }
    CHECK(resident == mapped);
    CHECK(t.hand >= 0 && t.hand < t.n_slots);
  }
};

static void clock_random(std::mt19937_64& rng) {
  for (int trial = 0; trial < 200; ++trial) {
    const int32_t n_slots = 1 + (int32_t)(rng() % 64);
    const int32_t n_pages = 1 + (int32_t)(rng() % 300);
    Table tb(n_slots, n_pages);
    CHECK(kv_residency_reset(&tb.t) == KV_OK);
    tb.check_inverse();
    for (int step = 0; step < 50; ++step) {
      const int32_t max_sel = n_slots < n_pages ? n_slots : n_pages;
      const int32_t n_sel = (int32_t)(rng() % (max_sel + 1));
      // distinct pages in random order
      std::vector<int32_t> perm(n_pages);
      for (int32_t i = 0; i < n_pages; ++i) perm[i] = i;
      for (int32_t i = n_pages - 1; i > 0; --i) std::swap(perm[i], perm[rng() % (i + 1)]);
      std::vector<int32_t> sel(perm.begin(), perm.begin() + n_sel);
      std::vector<int32_t> out(n_sel + 1, -7), mp(n_sel + 1, -7), ms(n_sel + 1, -7);
      int32_t n_miss = -1;
      std::vector<int32_t> before_slot(n_pages);
      for (int32_t p = 0; p < n_pages; ++p) before_slot[p] = tb.page_slot[p];
      const int r = kv_residency_select(&tb.t, sel.data(), n_sel, out.data(), mp.data(), ms.data(), &n_miss);
      CHECK(r == KV_OK);
      tb.check_inverse();
      int32_t expect_miss = 0;
      for (int32_t i = 0; i < n_sel; ++i) {
        CHECK(out[i] >= 0 && out[i] < n_slots);
        CHECK(tb.slot_page[out[i]] == sel[i]);
        CHECK(tb.ref[out[i]] == 1);
        if (before_slot[sel[i]] < 0) ++expect_miss;
        else CHECK(out[i] == before_slot[sel[i]]);  // a resident page keeps its slot
      }
      CHECK(n_miss == expect_miss);
      for (int32_t i = 0; i < n_miss; ++i) CHECK(tb.page_slot[mp[i]] == ms[i]);
      CHECK(out[n_sel] == -7 && mp[n_sel] == -7 && ms[n_sel] == -7);  // nothing written past n_sel
      // the optional outputs may be NULL
      if (n_sel > 0) {
        Table copy = tb;
        copy.t.slot_page = copy.slot_page.data();
        copy.t.page_slot = copy.page_slot.data();
        copy.t.ref = copy.ref.data();
        CHECK(kv_residency_select(&copy.t, sel.data(), n_sel, out.data(), nullptr, nullptr, nullptr) == KV_OK);
        copy.check_inverse();
      }
    }
  }
}

static void clock_rejects(std::mt19937_64& rng) {
  Table tb(8, 40);
  CHECK(kv_residency_reset(&tb.t) == KV_OK);
  std::vector<int32_t> out(64);
  int32_t warm[5] = {3, 9, 1, 30, 12};
  CHECK(kv_residency_select(&tb.t, warm, 5, out.data(), nullptr, nullptr, nullptr) == KV_OK);
  const Table saved = tb;
  auto unchanged = [&]() { return tb.same(saved); };
  int32_t dup[3] = {4, 5, 4};
  CHECK(kv_residency_select(&tb.t, dup, 3, out.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(unchanged());
  int32_t oob[2] = {4, 40};
  CHECK(kv_residency_select(&tb.t, oob, 2, out.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(unchanged());
  int32_t neg[2] = {-1, 3};
  CHECK(kv_residency_select(&tb.t, neg, 2, out.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(unchanged());
  std::vector<int32_t> many(9);
  for (int i = 0; i < 9; ++i) many[i] = i;
  CHECK(kv_residency_select(&tb.t, many.data(), 9, out.data(), nullptr, nullptr, nullptr) == KV_ENOSLOTS);
  CHECK(unchanged());
  CHECK(kv_residency_select(&tb.t, nullptr, 2, out.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(kv_residency_select(&tb.t, warm, 2, nullptr, nullptr, nullptr, nullptr) < 0);
  CHECK(kv_residency_select(nullptr, warm, 2, out.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(kv_residency_select(&tb.t, warm, -1, out.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(unchanged());
  // a table whose own fields are inconsistent
  Table bad(4, 10);
  CHECK(kv_residency_reset(&bad.t) == KV_OK);
  bad.t.hand = 7;
  CHECK(kv_residency_select(&bad.t, warm, 1, out.data(), nullptr, nullptr, nullptr) < 0);
  bad.t.hand = 0;
  bad.t.n_slots = 0;
  CHECK(kv_residency_select(&bad.t, warm, 1, out.data(), nullptr, nullptr, nullptr) < 0);
  bad.t.n_slots = -3;
  CHECK(kv_residency_reset(&bad.t) < 0);
  kv_residency nulls{};
  nulls.n_slots = 4;
  nulls.n_pages = 4;
  CHECK(kv_residency_reset(&nulls) < 0);
  (void)rng;
}

static uint16_t rand_f16(std::mt19937_64& rng) {
  // mostly finite values of every exponent, some specials
  const uint32_t r = (uint32_t)rng();
  if (r % 97 == 0) return 0x7C00u | (r & 0x8000u);            // +-inf
  if (r % 89 == 0) return 0x7E00u;                              // NaN
  if (r % 83 == 0) return (uint16_t)(r & 0x83FFu);               // subnormal or zero
  uint16_t h = (uint16_t)(r & 0xFFFFu);
  if ((h & 0x7C00u) == 0x7C00u) h ^= 0x4000u;                    // keep it finite
  return h;
}

static void host_encoder(std::mt19937_64& rng) {
  std::vector<uint16_t> x(256);
  std::vector<uint8_t> codes(256);
  std::vector<uint16_t> scales(8);
  for (int trial = 0; trial < 400; ++trial) {
    const int mode = trial % 4;
    for (int i = 0; i < 256; ++i) {
      if (mode == 0) x[i] = rand_f16(rng);
      else if (mode == 1) x[i] = (uint16_t)(0x3C00u + (rng() % 0x400u)) | (uint16_t)((rng() & 1) << 15);
      else if (mode == 2) x[i] = (uint16_t)(rng() % 0x400u);     // tiny
      else x[i] = (uint16_t)((i == trial % 256) ? 0x7BFFu : 0u);  // one large element
    }
    for (int32_t kind = 0; kind < 4; ++kind) {
      std::memset(codes.data(), 0xAB, codes.size());
      const int r = kv_host_encode_vector(kind, x.data(), codes.data(), scales.data());
      CHECK(r == KV_OK);
      if (kind == 1 || kind == 2)
        for (int i = 0; i < 256; ++i) CHECK(codes[i] <= 15);
    }
  }
  CHECK(kv_host_encode_vector(7, x.data(), codes.data(), scales.data()) < 0);
  CHECK(kv_host_encode_vector(-1, x.data(), codes.data(), scales.data()) < 0);
  CHECK(kv_host_encode_vector(0, nullptr, codes.data(), scales.data()) < 0);
  CHECK(kv_host_encode_vector(0, x.data(), nullptr, scales.data()) < 0);
  CHECK(kv_host_encode_vector(0, x.data(), codes.data(), nullptr) < 0);
  // f64 -> f16 over random bit patterns and the special values
  for (int i = 0; i < 200000; ++i) {
    uint64_t b = rng();
    double d;
    std::memcpy(&d, &b, sizeof d);
    (void)kv_host_f64_to_f16(d);
  }
  const double specials[] = {0.0, -0.0, 65504.0, 65520.0, -65520.0, 1e300, -1e300, 5.96e-8, 2.98e-8, 2.99e-8,
                             std::numeric_limits<double>::denorm_min(), std::numeric_limits<double>::infinity(),
                             -std::numeric_limits<double>::infinity(), std::numeric_limits<double>::quiet_NaN()};
  for (double d : specials) (void)kv_host_f64_to_f16(d);
  CHECK(kv_host_f64_to_f16(1.0) == 0x3C00u);
  CHECK(kv_host_f64_to_f16(65520.0) == 0x7C00u);
}

static void size_helpers(std::mt19937_64& rng) {
  const int32_t odd[] = {0, 1, -1, 3, 256, 255, 257, 8, 24, 4, 64, 1 << 30, -(1 << 30),
                         std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::min()};
  const int64_t lens[] = {0, 1, -1, 255, 256, 1 << 20, (int64_t)1 << 40, std::numeric_limits<int64_t>::max(),
                          std::numeric_limits<int64_t>::min()};
  for (int trial = 0; trial < 3000; ++trial) {
    kv_shape s;
    s.n_q_heads = odd[rng() % (sizeof odd / sizeof odd[0])];
    s.n_kv_heads = odd[rng() % (sizeof odd / sizeof odd[0])];
    s.head_dim = (rng() & 1) ? 256 : odd[rng() % (sizeof odd / sizeof odd[0])];
    s.page_tokens = (rng() & 1) ? 256 : odd[rng() % (sizeof odd / sizeof odd[0])];
    s.format = (int32_t)(rng() % 7) - 1;
    const int32_t batch = odd[rng() % (sizeof odd / sizeof odd[0])];
    const int64_t ctx = lens[rng() % (sizeof lens / sizeof lens[0])];
    const int32_t pps = odd[rng() % (sizeof odd / sizeof odd[0])];
    (void)kv_page_bytes(&s);
    (void)kv_decode_workspace_bytes(&s, batch, ctx, pps);
    (void)kv_decode_mq_workspace_bytes(&s, batch, 1 + (int32_t)(rng() % 9), ctx, pps);
    (void)kv_decode_split_pages(&s, batch, ctx, ctx);
    (void)kv_select_workspace_bytes(ctx, batch);
  }
  (void)kv_page_bytes(nullptr);
  CHECK(kv_decode_workspace_bytes(nullptr, 1, 256, 0) == 0);
  kv_shape q4{24, 4, 256, 256, KV_FMT_Q4_0};
  CHECK(kv_page_bytes(&q4) == 294912);
  CHECK(kv_decode_split_pages(&q4, 1, 131072, 131072) >= 1);
}

// Entry points that enqueue device work, called with arguments they must reject on
// the host. Pointers here are never valid device memory; an accepted call would be a
// failure of the checks (it would try to enqueue work).
static void argument_checks() {
  kv_shape s{24, 4, 256, 256, KV_FMT_Q4_0};
  kv_shape bad_fmt{24, 4, 256, 256, 9};
  kv_shape bad_dim{24, 4, 128, 256, KV_FMT_Q4_0};
  kv_shape bad_group{20, 4, 256, 256, KV_FMT_Q4_0};  // 5 query heads per KV head is fine; 20/3 is not
  bad_group.n_kv_heads = 3;
  alignas(16) static uint8_t buf[4096];
  void* a = buf;
  void* mis = buf + 2;
  float* of = reinterpret_cast<float*>(buf + 1024);
  int32_t st = 0;
  const int32_t* bt = reinterpret_cast<const int32_t*>(buf);
  const int32_t* ctx = reinterpret_cast<const int32_t*>(buf + 256);

  CHECK(kv_append_quantize(nullptr, a, a, 1, 0, bt, 1, a, 1, nullptr, nullptr) < 0);
  CHECK(kv_append_quantize(&bad_fmt, a, a, 1, 0, bt, 1, a, 1, nullptr, nullptr) < 0);
  CHECK(kv_append_quantize(&bad_dim, a, a, 1, 0, bt, 1, a, 1, nullptr, nullptr) < 0);
  CHECK(kv_append_quantize(&s, a, a, -1, 0, bt, 1, a, 1, nullptr, nullptr) < 0);
  CHECK(kv_append_quantize(&s, a, a, 1, -5, bt, 1, a, 1, nullptr, nullptr) < 0);
  CHECK(kv_append_quantize(&s, a, a, 300, 0, bt, 1, a, 1, nullptr, nullptr) < 0);  // beyond the table
  CHECK(kv_append_quantize(&s, mis, a, 1, 0, bt, 1, a, 1, nullptr, nullptr) < 0);
  CHECK(kv_append_quantize(&s, nullptr, a, 1, 0, bt, 1, a, 1, nullptr, nullptr) < 0);

  CHECK(kv_decode_attention(nullptr, a, 1, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 4096, 0, nullptr) < 0);
  CHECK(kv_decode_attention(&bad_group, a, 1, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 4096, 0, nullptr) < 0);
  CHECK(kv_decode_attention(&s, a, -1, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 4096, 0, nullptr) < 0);
  CHECK(kv_decode_attention(&s, a, 1, a, 1, bt, 1, ctx, -3, 0.0625f, of, a, 4096, 0, nullptr) < 0);
  CHECK(kv_decode_attention(&s, a, 1, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 8, 0, nullptr) < 0);  // workspace too small
  CHECK(kv_decode_attention(&s, mis, 1, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 4096, 0, nullptr) < 0);
  CHECK(kv_decode_attention(&s, a, 1, a, 1, bt, 1, ctx, 256, std::nanf(""), of, a, 4096, 0, nullptr) < 0);
  CHECK(kv_decode_attention(&s, a, 1, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 4096, -2, nullptr) < 0);
  CHECK(kv_decode_attention_noalloc(&s, a, 1, a, 1, bt, 1, ctx, 256, 0.0625f, of, nullptr, 0, nullptr) < 0);
  CHECK(kv_decode_attention_noalloc(&s, a, 1 << 30, a, 1, bt, 1, ctx, 256, 0.0625f, of, &st, 0, nullptr) < 0);
  CHECK(kv_decode_attention_mq(&s, a, 1, 0, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 4096, 0, nullptr) < 0);
  CHECK(kv_append_decode(&s, a, a, a, 1, a, 1, bt, 1, ctx, -1, 0.0625f, of, a, 4096, 0, nullptr, nullptr, nullptr) < 0);
  CHECK(kv_append_decode(nullptr, a, a, a, 1, a, 1, bt, 1, ctx, 256, 0.0625f, of, a, 4096, 0, nullptr, nullptr, nullptr) < 0);

  Table tb(4, 10);
  CHECK(kv_residency_reset(&tb.t) == KV_OK);
  const Table saved = tb;
  int32_t sel[2] = {1, 2};
  int32_t miss = 0;
  CHECK(kv_gather_pages(&s, &tb.t, sel, 2, nullptr, a, reinterpret_cast<int32_t*>(a), &miss, nullptr) < 0);
  CHECK(kv_gather_pages(&s, &tb.t, sel, 2, mis, a, reinterpret_cast<int32_t*>(a), &miss, nullptr) < 0);
  CHECK(kv_gather_pages(&bad_fmt, &tb.t, sel, 2, a, a, reinterpret_cast<int32_t*>(a), &miss, nullptr) < 0);
  CHECK(tb.same(saved));
  CHECK(kv_gather_pages_layers(&s, -1, &tb.t, sel, 2, nullptr, nullptr, nullptr, nullptr, nullptr) < 0);
  CHECK(kv_gather_pages_layers(&s, 1, nullptr, sel, 2, nullptr, nullptr, nullptr, nullptr, nullptr) < 0);
  CHECK(tb.same(saved));

  int64_t* sums = reinterpret_cast<int64_t*>(a);
  CHECK(kv_page_key_sums(&s, a, -1, 0, sums, a, 4, nullptr) < 0);
  CHECK(kv_page_key_sums(&s, a, 10, 2000, sums, a, 4, nullptr) < 0);  // pages beyond the capacity
  CHECK(kv_page_key_sums(&s, a, 10, 0, sums, nullptr, 4, nullptr) < 0);  // no representatives
  CHECK(kv_select_pages(&s, a, a, 4, 8, 2, 1, reinterpret_cast<int32_t*>(a), a, 16, nullptr) < 0);  // reps_pages < n_pages
  CHECK(kv_select_pages(&s, a, a, 8, 8, 0, 1, reinterpret_cast<int32_t*>(a), a, 4096, nullptr) < 0);
  CHECK(kv_select_pages(&s, a, a, 8, 8, 300, 1, reinterpret_cast<int32_t*>(a), a, 4096, nullptr) < 0);
  CHECK(kv_select_pages(&s, a, static_cast<char*>(a) + 2, 8, 8, 2, 1, reinterpret_cast<int32_t*>(a), a, 4096, nullptr) < 0);  // reps not 16-B aligned

  // every rejected call left a message
  CHECK(kv_last_error() != nullptr && std::strlen(kv_last_error()) > 0);
}

int main() {
  std::mt19937_64 rng(20260512ull);
  clock_random(rng);
  clock_rejects(rng);
  host_encoder(rng);
  size_helpers(rng);
  argument_checks();
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}

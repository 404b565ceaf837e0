// Seeded fuzz of libdpnorm's host layer (argument checks, workspace plans,
// launch sequences) built with AddressSanitizer and UndefinedBehaviorSanitizer
// against the host-side HIP stand-in in fake_hip.cpp (test infrastructure).
//
// Every entry point is called with random sizes (valid and invalid: zero,
// negative, misaligned widths, budgets out of range, sizes whose products
// overflow), random layer counts up to 2^20 with and without shared inputs,
// and fake device addresses that are never dereferenced. Checked:
//   * a call with a workspace of the queried size returns the query's status
//     (every check runs on the host before anything is enqueued);
//   * with one byte less it returns DPNORM_ERR_WORKSPACE, with a misaligned
//     output DPNORM_ERR_ALIGN, with an output overlapping an input
//     DPNORM_ERR_VALUE;
//   * every launch has a valid configuration (the stand-in counts bad ones);
//   * the sanitizers report nothing (they abort the run on any finding).
// Usage: fuzz_plan [iterations] [seed]; exit status 0 when every check held.
#include <algorithm>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "dpnorm.h"

extern "C" long long dpnorm_fake_launches, dpnorm_fake_bad_launches;

namespace {

std::mt19937_64 rng;
long long g_failures = 0, g_calls = 0, g_ok = 0;

int64_t pick(std::initializer_list<int64_t> v) { return v.begin()[rng() % v.size()]; }
int64_t uni(int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); }

// Fake device regions, 2^40 bytes apart, 256-byte aligned.
const void* region(int r) { return (const void*)(uintptr_t)(0x100000000000ull + ((uint64_t)r << 40)); }

#define CHECK(cond, ...)                                          \
  do {                                                            \
    if (!(cond)) {                                                \
      ++g_failures;                                               \
      std::fprintf(stderr, "FAIL line %d: ", __LINE__);           \
      std::fprintf(stderr, __VA_ARGS__);                          \
      std::fprintf(stderr, "\n");                                 \
    }                                                             \
  } while (0)

int64_t width(dpnorm_dtype dt) {
  const int64_t g = dt == DPNORM_BF16 ? 8 : 4;
  switch (rng() % 8) {
    case 0: return pick({0, -8, 3, 12, 20}); // invalid or misaligned for bf16
    case 1: return g;
    case 2: return g * uni(1, 4);
    case 3: return pick({512, 2048, 8192});
    case 4: return g * uni(1, 1 << 13);
    default: return g * uni(1, 300);
  }
}
int64_t tokens() {
  switch (rng() % 6) {
    case 0: return pick({0, -1, 1, 2, 31, 33});
    case 1: return pick({4096, 32768, 131072});
    case 2: return uni(1, 1 << 22);
    default: return uni(1, 1200);
  }
}
int64_t batch() {
  switch (rng() % 6) {
    case 0: return pick({0, -3, 1});
    case 1: return uni(1, 1 << 12);
    case 2: return pick({(int64_t)1 << 40, (int64_t)1 << 62});
    default: return uni(1, 9);
  }
}
dpnorm_dtype dtype() {
  const int r = (int)(rng() % 10);
  return r == 0 ? (dpnorm_dtype)pick({-1, 2, 7}) : (r < 6 ? DPNORM_BF16 : DPNORM_F32);
}

// A tensor of B x T x w elements fits in its fake region (2^40 bytes apart,
// layers of a grouped call 2^20 apart inside it) without reaching the next.
bool fits(int64_t B, int64_t T, int64_t w) {
  return B > 0 && T > 0 && w > 0 && (double)B * (double)T * (double)w * 4.0 < (double)((int64_t)1 << 38);
}

// With tensors that fit their regions the call must return the query's
// status; larger fake tensors overlap the outputs, which the call rightly
// reports as DPNORM_ERR_VALUE.
bool expect_same(const char* what, dpnorm_status q, dpnorm_status c, size_t ws, bool tensors_fit) {
  ++g_calls;
  if (q == DPNORM_OK) ++g_ok;
  if (tensors_fit) CHECK(q == c, "%s: query status %d, call status %d (ws %zu)", what, (int)q, (int)c, ws);
  return tensors_fit && q == DPNORM_OK;
}

void fuzz_hutch() {
  const dpnorm_dtype dt = dtype();
  const int64_t B = batch(), T = tokens(), d = width(dt), p = width(dt), k = pick({0, -1, 1, 16, 32, 33, 64, 65});
  size_t ws = 0;
  const dpnorm_status q = dpnorm_hutch_workspace(dt, B, T, d, p, k, &ws);
  float* n = (float*)region(3);
  const dpnorm_status c = dpnorm_hutch(region(0), region(1), region(2), dt, B, T, d, p, k, n, (int)(rng() % 2),
                                       (void*)region(4), ws, nullptr);
  if (!expect_same("hutch", q, c, ws, fits(B, T, d) && fits(B, T, p))) return;
  if (ws > 0)
    CHECK(dpnorm_hutch(region(0), region(1), region(2), dt, B, T, d, p, k, n, 0, (void*)region(4), ws - 1,
                       nullptr) == DPNORM_ERR_WORKSPACE, "hutch short workspace");
  CHECK(dpnorm_hutch(region(0), region(1), region(2), dt, B, T, d, p, k, (float*)((char*)n + 2), 0,
                     (void*)region(4), ws, nullptr) == DPNORM_ERR_ALIGN, "hutch misaligned n");
  CHECK(dpnorm_hutch(region(0), region(1), region(2), dt, B, T, d, p, k, (float*)region(1), 0, (void*)region(4), ws,
                     nullptr) == DPNORM_ERR_VALUE, "hutch n overlaps G");
  CHECK(dpnorm_hutch_sign(region(0), region(1), (const uint32_t*)region(2), dt, B, T, d, p, k, n, 0,
                          (void*)region(4), ws, nullptr) == DPNORM_OK, "hutch_sign with the Hutchinson workspace");
}

void fuzz_grouped_layers(dpnorm_dtype dt, int64_t B, int64_t T, int64_t k, int64_t L);

void fuzz_grouped() {
  const dpnorm_dtype dt = dtype();
  const int64_t B = batch(), T = tokens(), k = pick({1, 8, 16, 32, 40, 64, 0, 65});
  const int r = (int)(rng() % 20);
  const int64_t L = r == 0 ? pick({1 << 10, 1 << 13, 1 << 16}) : (r == 1 ? pick({0, -1}) : uni(1, 12));
  fuzz_grouped_layers(dt, B, T, k, L);
}

void fuzz_grouped_layers(dpnorm_dtype dt, int64_t B, int64_t T, int64_t k, int64_t L) {
  std::vector<dpnorm_layer> layers((size_t)std::max<int64_t>(L, 1));
  for (int64_t l = 0; l < (int64_t)layers.size(); ++l) {
    const bool share = l > 0 && rng() % 3 == 0;
    dpnorm_layer& y = layers[(size_t)l];
    y.A = share ? layers[(size_t)l - 1].A : (const void*)((const char*)region(10) + (uint64_t)l * ((uint64_t)1 << 20));
    y.G = (const void*)((const char*)region(11) + (uint64_t)l * ((uint64_t)1 << 20));
    y.P = (const void*)((const char*)region(12) + (uint64_t)l * 4096);
    y.d = share ? layers[(size_t)l - 1].d : (L > 1000 ? pick({8, 16, 64}) : width(dt));
    y.p = L > 1000 ? pick({8, 32, 128}) : width(dt);
  }
  size_t ws = 0, ws_plain = 0;
  const dpnorm_status q = dpnorm_hutch_grouped_workspace(layers.data(), L, dt, B, T, k, &ws);
  std::vector<dpnorm_layer> anon = layers;
  for (auto& y : anon) y.A = y.G = y.P = nullptr;
  const dpnorm_status qp = dpnorm_hutch_grouped_workspace(anon.data(), L, dt, B, T, k, &ws_plain);
  CHECK(q == qp, "grouped query with and without pointers: %d vs %d", (int)q, (int)qp);
  float* n = (float*)region(13);
  float* c = rng() % 2 ? (float*)region(14) : nullptr;
  const float C = (float)pick({1, 0, -1, 3});
  const dpnorm_status st = dpnorm_hutch_grouped(layers.data(), L, dt, B, T, k, n, (int)(rng() % 2), c, C,
                                                (void*)region(15), ws, nullptr);
  const dpnorm_status want = (q == DPNORM_OK && c && !(C > 0)) ? DPNORM_ERR_VALUE : q;
  bool all_fit = true;
  for (const dpnorm_layer& y : layers) all_fit = all_fit && fits(B, T, y.d) && fits(B, T, y.p);
  if (expect_same("grouped", want, st, ws, all_fit)) {
    // a workspace sized without the pointers runs the call without sharing
    CHECK(dpnorm_hutch_grouped(layers.data(), L, dt, B, T, k, n, 0, c, C, (void*)region(15), ws_plain, nullptr) ==
              DPNORM_OK, "grouped with the plain workspace");
    CHECK(dpnorm_hutch_sign_grouped(layers.data(), L, dt, B, T, k, n, 0, c, C, (void*)region(15), ws, nullptr) ==
              DPNORM_OK, "sign grouped");
    size_t wsr = 0;
    if (dpnorm_norms_routed_workspace(layers.data(), L, dt, B, T, k, &wsr) == DPNORM_OK) {
      std::vector<int32_t> routes((size_t)L);
      CHECK(dpnorm_norms_routed(layers.data(), L, dt, B, T, k, n, 0, c, C, routes.data(), (void*)region(15), wsr,
                                nullptr) == DPNORM_OK, "routed");
      for (int64_t l = 0; l < L; ++l) {
        const bool ex = std::min(layers[(size_t)l].d, layers[(size_t)l].p) <= k;
        CHECK(routes[(size_t)l] == (ex ? 1 : 0), "route of layer %" PRId64, l);
      }
    }
    // traced, with too few and with enough events
    std::vector<hipEvent_t> evs(64, (hipEvent_t)region(16));
    std::vector<int32_t> kinds(64, 0);
    dpnorm_trace tr{evs.data(), kinds.data(), 2, 0};
    const dpnorm_status t2 = dpnorm_hutch_grouped_traced(layers.data(), L, dt, B, T, k, n, 0, c, C,
                                                         (void*)region(15), ws, nullptr, &tr);
    CHECK(t2 == DPNORM_OK || t2 == DPNORM_ERR_SIZE, "traced with 2 events: %d", (int)t2);
    if (L <= 160) {
      tr.capacity = 64;
      tr.count = 0;
      CHECK(dpnorm_hutch_grouped_traced(layers.data(), L, dt, B, T, k, n, 0, c, C, (void*)region(15), ws, nullptr,
                                        &tr) == DPNORM_OK && tr.count >= 2 && tr.count <= 64,
            "traced count %" PRId64, tr.count);
    }
    // no caller workspace: fits the static scratch or is refused
    const dpnorm_status na = dpnorm_hutch_grouped_noalloc(layers.data(), L, dt, B, T, k, n, 0, c, C, nullptr);
    CHECK(na == (std::min(ws, ws_plain) <= DPNORM_STATIC_SCRATCH_BYTES ? DPNORM_OK : DPNORM_ERR_WORKSPACE),
          "noalloc status %d for workspace %zu / %zu", (int)na, ws, ws_plain);
  }
}

void fuzz_hutchpp() {
  const dpnorm_dtype dt = dtype();
  const int64_t B = batch(), T = tokens(), d = width(dt), p = width(dt);
  const int64_t k = pick({2, 3, 4, 12, 32, 48, 96, 97, 0});
  size_t ws = 0;
  const dpnorm_status q = dpnorm_hutchpp_workspace(dt, B, T, d, p, k, &ws);
  int64_t ms = 0, mt = 0;
  const dpnorm_status sp = dpnorm_hutchpp_split(k, &ms, &mt);
  if (sp != DPNORM_OK) CHECK(q != DPNORM_OK, "hutchpp query accepts budget %" PRId64, k);
  float* head = rng() % 2 ? (float*)region(24) : nullptr;
  float* tail = rng() % 2 ? (float*)region(25) : nullptr;
  int32_t* rank = rng() % 2 ? (int32_t*)region(26) : nullptr;
  float* resid = rng() % 2 ? (float*)region(27) : nullptr;
  const dpnorm_status c = dpnorm_hutchpp(region(20), region(21), region(22), region(23), dt, B, T, d, p, k,
                                         (float*)region(28), 0, head, tail, rank, resid, (void*)region(29), ws, nullptr);
  if (expect_same("hutchpp", q, c, ws, fits(B, T, d) && fits(B, T, p)) && resid)
    CHECK(dpnorm_hutchpp(region(20), region(21), region(22), region(23), dt, B, T, d, p, k, (float*)region(28), 0,
                         head, tail, rank, (float*)region(28), (void*)region(29), ws, nullptr) == DPNORM_ERR_VALUE,
          "hutchpp resid overlapping n");
}

void fuzz_exact() {
  const dpnorm_dtype dt = dtype();
  const int64_t B = batch(), T = tokens(), d = width(dt), p = width(dt);
  const dpnorm_route r = (dpnorm_route)pick({0, 1, 2, 3});
  size_t ws = 0;
  const dpnorm_status q = dpnorm_exact_workspace(dt, B, T, d, p, r, &ws);
  const dpnorm_status c = dpnorm_exact(region(30), region(31), dt, B, T, d, p, r, (float*)region(32), 0,
                                       (void*)region(33), ws, nullptr);
  expect_same("exact", q, c, ws, fits(B, T, d) && fits(B, T, p));
}

void fuzz_small() {
  const int64_t B = batch();
  const float C = (float)pick({1, 0, -2, 5});
  const dpnorm_status c = dpnorm_clip_factors((const float*)region(40), B, C, (float*)region(40), nullptr);
  const bool ok = B >= 1 && B <= ((int64_t)1 << 30) && C > 0;
  CHECK((c == DPNORM_OK) == ok, "clip factors B %" PRId64 " C %g: %d", B, (double)C, (int)c);
  const int64_t bytes = pick({0, 16384, 16384 * 3, 100, (int64_t)1 << 44, ((int64_t)1 << 44) + 16384});
  const dpnorm_status rp = dpnorm_read_probe(region(41), bytes, nullptr);
  CHECK((rp == DPNORM_OK) == (bytes > 0 && bytes % 16384 == 0 && bytes <= ((int64_t)1 << 44)),
        "read probe %" PRId64 ": %d", bytes, (int)rp);
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 4000;
  const unsigned long long seed = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 12345;
  rng.seed(seed);
  // one call over 2^20 layers (with shared inputs) besides the random ones
  fuzz_grouped_layers(DPNORM_BF16, 2, 64, 32, (int64_t)1 << 20);
  for (long it = 0; it < iters; ++it) {
    switch (it % 5) {
      case 0: fuzz_hutch(); break;
      case 1: fuzz_grouped(); break;
      case 2: fuzz_hutchpp(); break;
      case 3: fuzz_exact(); break;
      default: fuzz_small();
    }
  }
  std::printf("fuzz_plan: %ld iterations, %lld paired calls (%lld valid), %lld launches, %lld bad launches, "
              "%lld failures\n", iters, g_calls, g_ok, dpnorm_fake_launches, dpnorm_fake_bad_launches, g_failures);
  return (g_failures == 0 && dpnorm_fake_bad_launches == 0) ? 0 : 1;
}

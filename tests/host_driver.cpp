// Host-side driver for the C ABI, built against a host-only, sanitizer-
// instrumented build of the library (AddressSanitizer + UndefinedBehavior-
// Sanitizer on the host code; no device code, no GPU). It drives every entry
// point that does host work only: status strings, workspace and plan sizes,
// the cu_seqlens checker, the schedule model, the batcher and the argument
// validation of every device entry point, including seeded random inputs.
// Invariants are checked here too; the sanitizers report any out-of-bounds
// access, overflow or undefined shift on the way. Prints "host driver ok" and
// exits 0 when every check passes.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <tuple>
#include <vector>

#include "esm_attn.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

// splitmix64: a small seeded generator for the random cases
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int32_t below(int32_t n) { return n <= 0 ? 0 : (int32_t)(next() % (uint64_t)n); }
};

static std::vector<int32_t> cu_of(const std::vector<int32_t>& L) {
  std::vector<int32_t> cu(L.size() + 1, 0);
  for (size_t b = 0; b < L.size(); ++b) cu[b + 1] = cu[b] + L[b];
  return cu;
}

static void strings_and_sizes() {
  CHECK(esm_attn_abi_version() == ESM_ATTN_ABI_VERSION);
  for (int s = -3; s < 10; ++s) CHECK(esm_attn_status_string(s) != nullptr);
  const int32_t dims[] = {16, 32, 64, 128, 0, 48, 256, -64};
  const int32_t Ts[] = {0, 1, 1000, 1 << 20, 1 << 30, -1};
  for (int32_t d : dims)
    for (int32_t T : Ts)
      for (int32_t H : {1, 20, 40, 1 << 16, 0})
        for (int32_t maxL : {0, 1, 1024, 65536, 65537, -1}) {
          const size_t f = esm_attn_fwd_workspace_bytes(4, T, maxL, H, d);
          const size_t b = esm_attn_bwd_workspace_bytes(4, T, maxL, H, d);
          const size_t p = esm_attn_plan_bytes(4, T, maxL, H, d);
          const bool legal = (d == 16 || d == 32 || d == 64 || d == 128) && T >= 0 && H >= 1 &&
                             maxL >= 0 && maxL <= 65536 &&
                             (int64_t)T * H * d < ((int64_t)1 << 31);
          if (!legal) {
            CHECK(f == 0 && b == 0 && p == 0);
          } else {
            CHECK(b >= f && f >= p && p > 0);
          }
        }
}

static void cu_checker() {
  const int32_t good[] = {0, 3, 3, 10};
  CHECK(esm_attn_check_cu_seqlens_host(good, 3, 10, 7) == ESM_ATTN_OK);
  CHECK(esm_attn_check_cu_seqlens_host(good, 3, 10, 6) == ESM_ATTN_ERR_INVALID_ARGUMENT);
  CHECK(esm_attn_check_cu_seqlens_host(good, 3, 11, 7) == ESM_ATTN_ERR_INVALID_ARGUMENT);
  const int32_t dec[] = {0, 5, 4, 10};
  CHECK(esm_attn_check_cu_seqlens_host(dec, 3, 10, 10) == ESM_ATTN_ERR_INVALID_ARGUMENT);
  const int32_t off[] = {1, 5, 10};
  CHECK(esm_attn_check_cu_seqlens_host(off, 2, 10, 10) == ESM_ATTN_ERR_INVALID_ARGUMENT);
  const int32_t huge[] = {0, 2147483647};
  CHECK(esm_attn_check_cu_seqlens_host(huge, 1, 2147483647, 65536) ==
        ESM_ATTN_ERR_INVALID_ARGUMENT);
  CHECK(esm_attn_check_cu_seqlens_host(nullptr, 1, 0, 0) == ESM_ATTN_ERR_INVALID_ARGUMENT);
  CHECK(esm_attn_check_cu_seqlens_host(good, 0, 0, 0) == ESM_ATTN_ERR_INVALID_ARGUMENT);
}

// every item of every (sequence, head) exactly once, idle slots all -1, the
// blocks of one (sequence, head) on one residue of the slot index mod 8
static void check_schedule(const std::vector<int32_t>& L, int32_t H, int32_t block) {
  const std::vector<int32_t> cu = cu_of(L);
  const int32_t B = (int32_t)L.size(), T = cu[B];
  int32_t maxL = 0;
  for (int32_t x : L) maxL = x > maxL ? x : maxL;
  int32_t n = -1;
  int32_t dummy[4];
  // too small a capacity is rejected
  CHECK(esm_attn_schedule_host(cu.data(), B, T, maxL, H, block, dummy, 0, &n) ==
            ESM_ATTN_ERR_INVALID_ARGUMENT || T == 0);
  const int32_t cap = 8 * (maxL / block + 2) + H * (B * (maxL / block + 1) + T / block + B) + 64;
  std::vector<int32_t> items(4 * (size_t)cap, 7);
  CHECK(esm_attn_schedule_host(cu.data(), B, T, maxL, H, block, items.data(), cap, &n) ==
        ESM_ATTN_OK);
  CHECK(n >= 0 && n <= cap);
  std::set<std::tuple<int32_t, int32_t, int32_t, int32_t>> seen;
  std::vector<int> residue((size_t)B * H, -1);
  std::vector<int32_t> seq_of(T + 1, -1);
  for (int32_t b = 0; b < B; ++b) seq_of[cu[b]] = b;
  for (int32_t s = 0; s < n; ++s) {
    const int32_t* it = &items[4 * (size_t)s];
    if (it[1] <= 0) {
      CHECK(it[0] == -1 && it[1] == -1 && it[2] == -1 && it[3] == -1);
      continue;
    }
    CHECK(it[0] >= 0 && it[0] < T && it[2] >= 0 && it[2] < H && it[3] >= 0);
    const int32_t b = seq_of[it[0]];
    CHECK(b >= 0 && L[b] == it[1] && it[3] * block < it[1]);
    CHECK(seen.insert(std::make_tuple(it[0], it[1], it[2], it[3])).second);
    int& r = residue[(size_t)b * H + it[2]];
    CHECK(r < 0 || r == s % 8);
    r = s % 8;
  }
  size_t want = 0;
  for (int32_t x : L) want += (size_t)H * ((x + block - 1) / block);
  CHECK(seen.size() == want);
}

static void schedules(Rng& rng) {
  check_schedule({0, 0, 5, 0}, 3, 128);
  check_schedule({128, 129, 127, 0, 256}, 7, 64);
  check_schedule({65536}, 1, 128);
  check_schedule(std::vector<int32_t>(300, 1), 2, 128);
  for (int trial = 0; trial < 200; ++trial) {
    const int32_t B = 1 + rng.below(40), H = 1 + rng.below(6);
    const int32_t cap_len = 1 + rng.below(trial % 4 == 0 ? 3000 : 300);
    std::vector<int32_t> L(B);
    for (auto& x : L) x = rng.below(5) == 0 ? 0 : rng.below(cap_len + 1);
    check_schedule(L, H, trial % 2 ? 64 : 128);
  }
  int32_t n;
  int32_t items[4];
  const int32_t cu[] = {0, 4};
  CHECK(esm_attn_schedule_host(cu, 1, 4, 4, 1, 8, items, 1, &n) == ESM_ATTN_ERR_INVALID_ARGUMENT);
  CHECK(esm_attn_schedule_host(cu, 1, 4, 65537, 1, 128, items, 1, &n) ==
        ESM_ATTN_ERR_INVALID_ARGUMENT);
  CHECK(esm_attn_schedule_host(nullptr, 1, 4, 4, 1, 128, items, 1, &n) ==
        ESM_ATTN_ERR_INVALID_ARGUMENT);
}

// batches partition the input; in each bucket, batches keep input order and
// stay within the budget unless a single sequence exceeds it
static void batching(Rng& rng) {
  for (int trial = 0; trial < 300; ++trial) {
    const int32_t n = rng.below(200);
    std::vector<int32_t> len(n);
    for (auto& x : len) x = rng.below(2000);
    std::vector<int32_t> bounds;
    for (int32_t v = 1 + rng.below(300); v < 2000 && bounds.size() < 6; v += 1 + rng.below(600))
      bounds.push_back(v);
    const int64_t budget = 1 + rng.below(8000);
    const int32_t padded = rng.below(2);
    std::vector<int32_t> order(n + 1, -5), offs(n + 2, -5);
    int32_t nb = -1;
    CHECK(esm_attn_bucket_batches(len.data(), n, bounds.data(), (int32_t)bounds.size(), budget,
                                  padded, order.data(), offs.data(), n, &nb) == ESM_ATTN_OK);
    CHECK(nb >= 0 && nb <= n && order[n] == -5);
    if (nb < 0 || nb > n) continue;
    CHECK(offs[0] == 0 && offs[nb] == n);
    std::vector<int> hit(n, 0);
    for (int32_t b = 0; b < nb; ++b) {
      CHECK(offs[b] < offs[b + 1]);
      int64_t sum = 0, mx = 0, cnt = 0;
      for (int32_t i = offs[b]; i < offs[b + 1]; ++i) {
        const int32_t s = order[i];
        CHECK(s >= 0 && s < n);
        if (s < 0 || s >= n) continue;
        ++hit[s];
        if (i > offs[b]) CHECK(order[i - 1] < s);
        sum += len[s];
        mx = len[s] > mx ? len[s] : mx;
        ++cnt;
      }
      const int64_t cost = padded ? cnt * mx : sum;
      CHECK(cost <= budget || cnt == 1);
    }
    for (int32_t s = 0; s < n; ++s) CHECK(hit[s] == 1);
    // a capacity one short of the count is rejected
    if (nb > 0) {
      int32_t nb2 = -1;
      CHECK(esm_attn_bucket_batches(len.data(), n, bounds.data(), (int32_t)bounds.size(), budget,
                                    padded, order.data(), offs.data(), nb - 1, &nb2) ==
            ESM_ATTN_ERR_INVALID_ARGUMENT);
    }
  }
  const int32_t neg[] = {3, -1};
  int32_t order[2], offs[3], nb;
  CHECK(esm_attn_bucket_batches(neg, 2, nullptr, 0, 10, 0, order, offs, 2, &nb) ==
        ESM_ATTN_ERR_INVALID_ARGUMENT);
  const int32_t ok[] = {3, 1}, dec[] = {5, 5};
  CHECK(esm_attn_bucket_batches(ok, 2, dec, 2, 10, 0, order, offs, 2, &nb) ==
        ESM_ATTN_ERR_INVALID_ARGUMENT);
  CHECK(esm_attn_bucket_batches(ok, 2, nullptr, 0, 0, 0, order, offs, 2, &nb) ==
        ESM_ATTN_ERR_INVALID_ARGUMENT);
  CHECK(esm_attn_bucket_batches(ok, 2, nullptr, 0, 10, 2, order, offs, 2, &nb) ==
        ESM_ATTN_ERR_INVALID_ARGUMENT);
}

// argument validation of the device entry points: each case is rejected on
// the host, before any HIP call (fake, aligned pointers are never touched)
static void validation() {
  alignas(256) static uint16_t buf[64];
  uint16_t* p = buf;
  const int32_t* cu = reinterpret_cast<const int32_t*>(buf);
  float* f = reinterpret_cast<float*>(buf);
  uint8_t* b8 = reinterpret_cast<uint8_t*>(buf);
  const size_t big = (size_t)1 << 40;
  const float nan = std::nanf(""), inf = INFINITY;
  const int INV = ESM_ATTN_ERR_INVALID_ARGUMENT, UNS = ESM_ATTN_ERR_UNSUPPORTED,
            WS = ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  CHECK(esm_attn_fwd(nullptr, p, p, cu, 1, 8, 8, 1, 64, 0.1f, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p + 1, p, p, cu, 1, 8, 8, 1, 64, 0.1f, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 0, 8, 8, 1, 64, 0.1f, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, -1, 8, 1, 64, 0.1f, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 65537, 1, 64, 0.1f, 1e4f, p, f, p, big, nullptr) == UNS);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 0, 64, 0.1f, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 1, 48, 0.1f, 1e4f, p, f, p, big, nullptr) == UNS);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 1 << 24, 8, 1 << 4, 128, 0.1f, 1e4f, p, f, p, big,
                     nullptr) == UNS);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 1, 64, nan, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 1, 64, inf, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 1, 64, 3e38f, 1e4f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 1, 64, 0.1f, -1.f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 1, 64, 0.1f, inf, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd(p, p, p, cu, 1, 8, 8, 1, 64, 0.1f, 1e4f, p, f, p, 16, nullptr) == WS);
  CHECK(esm_attn_bwd(p, p, p, p, p, f, cu, 1, 8, 8, 1, 64, 0.1f, 1e4f, p, p, nullptr, p, big,
                     nullptr) == INV);
  CHECK(esm_attn_bwd(p, p, p, p, p, f, cu, 1, 8, 8, 1, 64, 0.1f, 1e4f, p, p, p, p,
                     esm_attn_fwd_workspace_bytes(1, 8, 8, 1, 64), nullptr) == WS);
  CHECK(esm_attn_plan(cu, 1, 8, 8, 1, 64, 1e4f, p, 16, nullptr) == WS);
  CHECK(esm_attn_plan(cu, 1, 8, 8, 1, 64, nan, p, big, nullptr) == INV);
  CHECK(esm_attn_rotate_planned(p, p, 63, 1, 8, 8, 1, 64, 0.125f, 1e4f, p, p, 64, p, big,
                                nullptr) == INV);
  CHECK(esm_attn_rotate_planned(p, p, 64, 1, 8, 8, 1, 64, 3e38f, 1e4f, p, p, 64, p, big,
                                nullptr) == INV);  // softmax_scale * log2(e) overflows
  // in place (both outputs on their inputs) needs one stride for both sides
  CHECK(esm_attn_rotate_planned(p, p + 32, 64, 1, 8, 8, 1, 64, 0.125f, 1e4f, p, p + 32, 72, p,
                                big, nullptr) == INV);
  CHECK(esm_attn_fwd_planned(p, p, p, 60, 1, 8, 8, 1, 64, 0.1f, p, f, p, big, nullptr) == INV);
  CHECK(esm_attn_fwd_planned(p, p, p, 1 << 20, 1, 1 << 11, 8, 1, 64, 0.1f, p, f, p, big,
                             nullptr) == UNS);  // total_tokens * stride >= 2^31
  CHECK(esm_attn_fwd_split_planned(p, p, p, 64, 1, 8, 8, 1, 64, 0.1f, 0, f, f, p, f, p, big,
                                   nullptr) == INV);
  CHECK(esm_attn_fwd_split_planned(p, p, p, 64, 1, 8, 8, 1, 64, 0.1f, 65, f, f, p, f, p, big,
                                   nullptr) == INV);
  CHECK(esm_attn_quantize_fp8_planned(p, p, 64, 1, 8, 8, 1, 64, 1e4f, 0.f, 1.f, b8, b8, p, big,
                                      nullptr) == INV);
  CHECK(esm_attn_quantize_fp8_planned(p, p, 64, 1, 8, 8, 1, 32, 1e4f, 1.f, 1.f, b8, b8, p, big,
                                      nullptr) == UNS);
  CHECK(esm_attn_fwd_fp8_planned(b8, b8, p, 64, 1, 8, 8, 1, 64, 0.1f, 1e-45f, 1.f, p, f, p, big,
                                 nullptr) == INV);
  CHECK(esm_attn_fwd_fp8_planned(b8, b8, p, 64, 1, 8, 8, 1, 64, 1e20f, 1e20f, 1.f, p, f, p, big,
                                 nullptr) == INV);  // scale product overflows fp32
  CHECK(esm_attn_merge_partials(f, f, 0, 8, 1, 64, p, f, nullptr) == INV);
  CHECK(esm_attn_merge_partials(f, f, 2, 8, 1, 48, p, f, nullptr) == UNS);
  CHECK(esm_attn_bwd_planned(p, p, p, 64, p, p, f, 1, 8, 8, 1, 64, 0.1f, 1e4f, p, p, p, 64, f,
                             0, p, big, nullptr) == INV);
  CHECK(esm_attn_bwd_planned(p, p, p, 64, p, p, f, 1, 8, 8, 1, 64, 0.1f, 1e4f, p, p, p, 56, f,
                             3, p, big, nullptr) == INV);
  // empty batches return OK without touching anything
  CHECK(esm_attn_fwd(nullptr, nullptr, nullptr, nullptr, 1, 0, 0, 1, 64, 0.1f, 1e4f, nullptr,
                     nullptr, nullptr, 0, nullptr) == ESM_ATTN_OK);
  CHECK(esm_attn_merge_partials(nullptr, nullptr, 1, 0, 1, 64, nullptr, nullptr, nullptr) ==
        ESM_ATTN_OK);
}

int main() {
  Rng rng{0x5EEDull};
  strings_and_sizes();
  cu_checker();
  schedules(rng);
  batching(rng);
  validation();
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host driver ok\n");
  return 0;
}

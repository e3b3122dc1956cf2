// Host planner fuzz, built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_host_sanitizers.py: random and adversarial call shapes through
// the same host code the library exports as mla_plan_host /
// mla_plan_groups_host, checking that every piece stays inside its unit, that
// the pieces add up to every unit's entries, and that bad input is refused,
// not read out of bounds.
#include <stdint.h>
#include <stdio.h>

#include <random>
#include <vector>

#include "mla_plan_host.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int seed) {
  if (!ok) {
    ++failures;
    if (failures < 20) fprintf(stderr, "seed %d: %s\n", seed, what);
  }
}

std::vector<int32_t> indptr(const std::vector<int>& v) {
  std::vector<int32_t> p(v.size() + 1, 0);
  for (size_t i = 0; i < v.size(); ++i) p[i + 1] = p[i] + v[i];
  return p;
}

// Runs one planner twice (count, then fill) and checks the pieces.
template <class F>
void check(F plan, int64_t stream_rows, int seed) {  // stream_rows: entries of all units
  const int64_t n = plan(nullptr, 0);
  expect(n >= 0, "planner refused valid input", seed);
  if (n < 0) return;
  std::vector<int64_t> out(8 * (n + 1), -7);
  const int64_t n2 = plan(out.data(), n);
  expect(n2 == n, "count changed between calls", seed);
  expect(out[8 * n] == -7, "wrote past out_cap", seed);
  int64_t total = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t* r = &out[8 * i];
    expect(0 <= r[3] && r[3] < r[4] && r[4] <= r[5], "piece outside its unit", seed);
    expect((r[7] == 1) == (r[6] == -1), "slot / completeness mismatch", seed);
    total += r[4] - r[3];
  }
  expect(total == stream_rows, "pieces do not add up to the entries", seed);
}

}  // namespace

int main() {
  std::mt19937 rng(1234);
  for (int seed = 0; seed < 3000; ++seed) {
    auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    const int B = U(1, 48);
    const int G = U(1, 6);
    const int H = 16 * G;
    const int nw = U(1, 300);
    const int cps = U(1, 8), cpr = U(0, cps - 1);
    const bool dcp = U(0, 2) == 0;
    const int causal = U(0, 3) ? 1 : 0;
    std::vector<int> lens(B), full(B), qlens(B);
    for (int b = 0; b < B; ++b) {
      qlens[b] = U(1, 4);
      full[b] = U(0, 5) == 0 ? U(0, 9) : U(0, 6000);
      lens[b] = dcp ? (full[b] > cpr ? (full[b] - cpr + cps - 1) / cps : 0) : full[b];
    }
    const auto qo = indptr(qlens), kv = indptr(lens), gkv = indptr(full);
    const int32_t* g = dcp ? gkv.data() : nullptr;
    const int w_cp = dcp ? cps : 1, r_cp = dcp ? cpr : 0;
    // Expected stream lengths from the planner's own request view.
    mla::ReqSource src{qo.data(), kv.data(), g, kv[B], qo[B], 1, w_cp, r_cp, nullptr, 0, -1};
    int64_t W = 0, Wg = 0;
    for (int b = 0; b < B; ++b) W += (int64_t)G * mla::request_rows(mla::load_req(src, b));
    src.causal = causal;
    // Group mode: the pieces hold every unit's entries, not the leading stream
    // rows that charge each non-empty unit's start.  Its rows are packed, so
    // any head count is allowed there.
    const int Hg = (seed & 1) ? H : U(1, 100);
    for (int b = 0; b < B; ++b) {
      const mla::Req r = mla::load_req(src, b);
      for (int u = 0; u < mla::group_units(r, Hg); ++u) Wg += mla::group_unit_len(r, Hg, u);
    }
    check([&](int64_t* o, int64_t cap) {
      return mla::plan_pieces_host(qo.data(), kv.data(), g, B, H, nw, w_cp, r_cp, o, cap);
    }, W, seed);
    check([&](int64_t* o, int64_t cap) {
      return mla::plan_group_pieces_host(qo.data(), kv.data(), g, B, Hg, nw, causal, w_cp, r_cp, o,
                                         cap);
    }, Wg, seed);
  }
  // Adversarial indptr: decreasing, negative and oversized entries are
  // clamped to the buffers (no out-of-bounds read), negative totals refused.
  {
    std::vector<int32_t> qo = {0, 3, 1, 4}, kv = {0, 900, 100, 1000};
    int64_t out[8 * 512];
    expect(mla::plan_pieces_host(qo.data(), kv.data(), nullptr, 3, 16, 64, 1, 0, out, 512) >= 0,
           "non-monotone indptr", -1);
    std::vector<int32_t> neg = {0, -5, 7, -2};
    expect(mla::plan_pieces_host(qo.data(), neg.data(), nullptr, 3, 16, 64, 1, 0, out, 512) == -1,
           "negative total accepted", -2);
    std::vector<int32_t> big = {0, 2000000000, 5, 100};
    expect(mla::plan_group_pieces_host(qo.data(), big.data(), nullptr, 3, 96, 64, 1, 1, 0, out,
                                       512) >= 0,
           "oversized entry", -3);
    expect(mla::plan_pieces_host(qo.data(), kv.data(), nullptr, 3, 16, 64, 8, 8, out, 512) == -1,
           "bad rank accepted", -4);
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}

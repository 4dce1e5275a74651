// Drives the host-side LRU of the expert-slot cache (LruCore) through random
// steps, miss splits, failed fills and resizes, for a build under AddressSanitizer
// and UndefinedBehaviorSanitizer (host code only), checking its invariants after
// every operation: each resident key in one slot, slot tables and fills inside the
// slot range and distinct within a wave, at most S accesses per wave.  Prints "ok"
// and exits 0; any sanitizer report aborts the run.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "cache_core.hpp"

static uint64_t rs = 0xD1B54A32D192ED03ull;
static uint32_t rnd() {
  rs ^= rs >> 12; rs ^= rs << 25; rs ^= rs >> 27;
  return (uint32_t)((rs * 0x2545F4914F6CDD1Dull) >> 32);
}
static int rint_in(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                        \
    }                                                                      \
  } while (0)

static void check_state(const moe::LruCore& c) {
  const int S = c.n_slots();
  std::vector<int64_t> key(S), tick(S);
  c.state(key.data(), tick.data());
  std::set<int64_t> seen;
  for (int s = 0; s < S; ++s) {
    CHECK(key[s] >= -1 && key[s] < (int64_t)c.n_layers() * c.n_experts());
    if (key[s] >= 0) CHECK(seen.insert(key[s]).second);
  }
}

static void run(int S, int L, int E, int steps) {
  moe::LruCore c(S, L, E);
  std::vector<int32_t> counts(E), table(E);
  std::vector<moe::PlannedFill> fills;
  for (int st = 0; st < steps; ++st) {
    const int dens = rint_in(0, 3);
    for (int e = 0; e < E; ++e) counts[e] = (int)(rnd() % 4) < dens ? rint_in(1, 9) : 0;
    const int den = rint_in(1, 4);
    c.set_fill_fraction(rint_in(0, den), den);
    c.begin_step(rint_in(0, L - 1), counts.data());
    const moe::StepStats ss = c.step_stats();
    CHECK(ss.hits + ss.misses == ss.accesses && ss.inplace >= 0 && ss.inplace <= ss.misses);
    CHECK((int64_t)c.inplace().size() == ss.inplace);
    for (int e : c.inplace()) CHECK(e >= 0 && e < E && counts[e] > 0);
    bool failed = false;
    // as the library's lookups do: wave 0 is planned and committed even when the
    // step has no accesses, which closes it
    for (int w = 0; w < (ss.n_waves > 0 ? ss.n_waves : 1); ++w) {
      const int n = c.plan_wave(w, table.data(), fills);
      CHECK(n >= (ss.n_waves > 0 ? 1 : 0) && n <= c.n_slots());
      std::set<int32_t> slots;
      int in_wave = 0;
      for (int e = 0; e < E; ++e)
        if (table[e] >= 0) {
          CHECK(table[e] < c.n_slots() && slots.insert(table[e]).second);
          ++in_wave;
        }
      CHECK(in_wave == n);
      std::set<int32_t> fs;
      for (const auto& f : fills) {
        CHECK(f.slot >= 0 && f.slot < c.n_slots() && fs.insert(f.slot).second);
        CHECK(f.expert >= 0 && f.expert < E && table[f.expert] == f.slot);
      }
      if (!fills.empty() && rnd() % 10 == 0) {  // a failed fill: forget the touched slots
        std::vector<int32_t> bad;
        for (const auto& f : fills) bad.push_back(f.slot);
        c.invalidate(bad);
        CHECK(!c.step_open());
        failed = true;
        break;
      }
      c.commit_wave(w);
      check_state(c);
    }
    if (!failed) CHECK(!c.step_open());
    if (rnd() % 7 == 0) {
      const int nS = rint_in(1, 2 * c.n_slots() + 1);
      std::vector<int32_t> moved;
      c.plan_resize(nS, moved);
      CHECK((int)moved.size() == nS);
      for (int32_t m : moved) CHECK(m >= -1 && m < c.n_slots());
      c.commit_resize(nS, moved);
      CHECK(c.n_slots() == nS);
      check_state(c);
    }
  }
}

int main() {
  for (int rep = 0; rep < 40; ++rep) run(rint_in(1, 16), rint_in(1, 4), rint_in(1, 40), 80);
  run(1, 1, 1, 20);
  run(256, 2, 256, 40);
  std::printf("ok\n");
  return 0;
}

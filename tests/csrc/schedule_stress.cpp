// Stand-alone stress driver of the host state machine (schedule.hpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by the CPU tests.  It
// runs many pseudo-random configurations -- PR-Sink with and without a
// static sink, retrieval, reference frames, context-relative positions, a
// FIFO bank and displacements resolved late; ConvKV with one to four memory
// frames -- through long streams, and checks after every call that slots
// are in range and never shared, counts are consistent and every conv tap
// names a staged slot.  Exit status 0: no violation (the sanitizers abort on
// their own findings).
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <set>
#include <vector>

#include "schedule.hpp"

using bkv::Schedule;

static int fails = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                          \
    }                                                                   \
  } while (0)

static unsigned rng_state = 12345u;
static unsigned rnd(unsigned n) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return (rng_state >> 8) % n;
}

static void check_open(const Schedule& s) {
  std::set<int> used;
  for (const auto& g : s.segments()) {
    if (g.kind == bkv::SEG_DYNAMIC) {
      CHECK(g.slot == -1 && g.dyn >= 0 && g.dyn < s.n_dynamic());
      continue;
    }
    if (g.kind == bkv::SEG_MEMORY || g.kind == bkv::SEG_REFERENCE) {
      CHECK(g.slot == -1);
      continue;
    }
    CHECK(g.slot >= 0 && g.slot < s.n_slots());
    CHECK(used.insert(g.slot).second);
  }
  for (const auto& b : s.bank()) {
    CHECK(b.second >= 0 && b.second < s.n_slots());
    CHECK(used.insert(b.second).second);
  }
  CHECK((int)used.size() + s.free_slots() <= s.n_slots());
  CHECK(s.cur_slot() == s.segments().back().slot);
  CHECK(s.context_tokens() <= s.max_context_tokens());
  CHECK((int)s.segments().size() <= s.max_segments());
}

static void prsink_case(int it) {
  Schedule::Shape sh{};
  sh.convkv = false;
  sh.layers = 1 + (int)rnd(3);
  sh.frames = 1 + (int)rnd(3);
  sh.tokens_per_frame = 1 + (int)rnd(40);
  sh.window = 1 + (int)rnd(8);
  sh.statics = (int)rnd(2);
  sh.k = (int)rnd(9);
  sh.bank = (int)rnd(20);
  sh.kernel = 1;
  sh.memory_frames = 0;
  sh.ref_frames = (int)rnd(3);
  sh.relative = rnd(2) == 1;
  const bool deferred = sh.bank > 0 && rnd(2) == 1;
  sh.spare = deferred ? 2 : 0;
  Schedule s(sh);
  std::deque<int64_t> pending;                       // displaced members not yet resolved
  const int blocks = 20 + (int)rnd(200);
  for (int m = 0; m < blocks; ++m) {
    while (!pending.empty() && (s.free_slots() == 0 || rnd(3) == 0)) {
      CHECK(s.resolve_displaced(pending.front()));
      pending.pop_front();
    }
    CHECK(s.open());
    CHECK(!s.open());                                // already open
    check_open(s);
    for (int l = 0; l < sh.layers; ++l) CHECK(s.mark_attended(l));
    CHECK(!s.mark_attended(sh.layers));
    std::vector<bkv::ConvTap> taps;
    int displace = -1;
    const auto ev = s.pending_eviction();
    // a deferred-policy bank displaces whenever it is full; the other mixes
    // FIFO drops with displacements named at once
    if (ev.first >= 0 && s.bank_full() && sh.bank > 0 && (deferred || rnd(2) == 1)) {
      // some present member (not one already displaced)
      std::vector<int64_t> members;
      for (const auto& b : s.bank()) {
        bool gone = false;
        for (int64_t p : pending) gone |= p == b.first;
        if (!gone) members.push_back(b.first);
      }
      CHECK(!members.empty());
      if (deferred) {
        displace = Schedule::kDisplaceDeferred;
        pending.push_back(members[rnd((unsigned)members.size())]);
      } else if (pending.empty()) {
        displace = (int)rnd((unsigned)s.bank().size());
      }
    }
    CHECK(s.commit(&taps, displace));
    CHECK(taps.empty());
    CHECK(s.bank_count() <= sh.bank);
  }
  (void)it;
}

static void convkv_case(int it) {
  Schedule::Shape sh{};
  sh.convkv = true;
  sh.layers = 1 + (int)rnd(2);
  sh.frames = 1 + (int)rnd(4);
  sh.tokens_per_frame = 1 + (int)rnd(30);
  sh.window = 1 + (int)rnd(8);
  sh.kernel = 1 + (int)rnd(8);
  sh.memory_frames = 1 + (int)rnd(4);
  if (sh.kernel * sh.memory_frames > 32) sh.memory_frames = 32 / sh.kernel;
  Schedule s(sh);
  const int blocks = 20 + (int)rnd(150);
  for (int m = 0; m < blocks; ++m) {
    CHECK(s.open());
    check_open(s);
    for (int l = 0; l < sh.layers; ++l) CHECK(s.mark_attended(l));
    std::vector<bkv::ConvTap> taps;
    CHECK(s.commit(&taps));
    CHECK(taps.size() % (size_t)sh.kernel == 0);
    CHECK((int)taps.size() <= sh.kernel * sh.memory_frames);
    for (const auto& t : taps) {
      CHECK(t.slot >= 0 && t.slot < s.n_slots());
      CHECK(t.frame >= 0 && t.frame < sh.frames);
    }
  }
  (void)it;
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 400;
  for (int it = 0; it < n; ++it) {
    prsink_case(it);
    convkv_case(it);
  }
  if (fails) std::fprintf(stderr, "%d checks failed\n", fails);
  else std::printf("schedule stress: %d configurations of each mode, no violation\n", n);
  return fails ? 1 : 0;
}

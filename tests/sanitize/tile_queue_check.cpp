// The ragged-K tile-queue protocol (csrc/tile_queue.h) on host threads: the
// same take / finish code the kernels run, over std::atomic words.  Checks
// that every tile of a launch is handed out exactly once whatever an earlier
// user left in the slot (a launch that died part-way, a finished launch, a
// replay with the same epoch), that exactly the last finisher is told to
// zero the slot, and the host's epoch and slot numbering.
#include <atomic>
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <thread>
#include <vector>

#include "tile_queue.h"

using namespace moe;

static int g_failed = 0, g_checks = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    ++g_checks;                                                   \
    if (!(c)) {                                                   \
      ++g_failed;                                                 \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c); \
    }                                                             \
  } while (0)

struct HostWord {
  std::atomic<uint32_t>* p;
  uint32_t add1() { return p->fetch_add(1u); }
  uint32_t cas(uint32_t expected, uint32_t desired) {
    p->compare_exchange_strong(expected, desired);
    return expected;   // the old word, whether or not the swap happened
  }
};

struct Slot {
  std::atomic<uint32_t> w[tq::kWords];
};

// One launch on `slot`: `workers` threads take tiles from nq queues of
// `ntiles[q]` tiles each, as the kernels do (own queue first, then the
// others); a worker with `die_after` >= 0 stops after that many takes and
// never finishes.  Returns per queue how often each tile was taken.
static std::vector<std::vector<int>> run_launch(Slot& slot, uint32_t epoch, uint32_t next, int workers, int nq,
                                                const std::vector<int>& ntiles, int die_after,
                                                int* finishers_told) {
  std::vector<std::vector<std::atomic<int>>> hits(nq);
  for (int q = 0; q < nq; ++q) hits[q] = std::vector<std::atomic<int>>(ntiles[q]);
  std::atomic<int> told{0};
  std::vector<std::thread> th;
  for (int b = 0; b < workers; ++b) {
    th.emplace_back([&, b] {
      int takes = 0;
      for (int qq = 0; qq < nq; ++qq) {
        const int q = (b % nq + qq) % nq;
        HostWord hw{&slot.w[q]};
        for (;;) {
          if (die_after >= 0 && takes == die_after) return;   // died part-way
          const uint32_t t = tq::take(hw, epoch);
          ++takes;
          if (t >= (uint32_t)ntiles[q]) break;
          hits[q][t].fetch_add(1);
        }
      }
      HostWord done{&slot.w[tq::kQueues]};
      if (tq::finish(done, epoch, (uint32_t)workers)) {
        told.fetch_add(1);
        for (auto& w : slot.w) w.store(tq::word(next, 0u));
      }
    });
  }
  for (auto& t : th) t.join();
  if (finishers_told) *finishers_told = told.load();
  std::vector<std::vector<int>> out(nq);
  for (int q = 0; q < nq; ++q)
    for (auto& h : hits[q]) out[q].push_back(h.load());
  return out;
}

static bool each_once(const std::vector<std::vector<int>>& hits) {
  for (auto& q : hits)
    for (int h : q)
      if (h != 1) return false;
  return true;
}

int main() {
  // host numbering: slot n % 64, epochs 1..255 in turn, the slot's next
  // launch kSlots later, with a different epoch for 254 launches on a slot
  CHECK(tq::launch_epoch(0) == 1u);
  CHECK(tq::launch_epoch(254) == 255u);
  CHECK(tq::launch_epoch(255) == 1u);
  CHECK(tq::launch_slot(0) == 0 && tq::launch_slot(65) == 1);
  for (uint64_t n : {0ull, 5ull, 63ull, 64ull, 254ull, 255ull, 0xFFFFFFFFull, 12345678901ull}) {
    CHECK(tq::launch_epoch(n) >= 1u && tq::launch_epoch(n) <= 255u);
    CHECK(tq::launch_slot(n) == tq::launch_slot(n + tq::kSlots));
    CHECK(tq::slot_next_epoch(n) == tq::launch_epoch(n + tq::kSlots));
    bool distinct = true;
    for (uint64_t j = 1; j < tq::kEpochs; ++j) distinct &= tq::launch_epoch(n + j * tq::kSlots) != tq::launch_epoch(n);
    CHECK(distinct);
    CHECK(tq::launch_epoch(n + tq::kEpochs * tq::kSlots) == tq::launch_epoch(n));
  }
  // counts stay below the epoch bits: a launch's tiles plus one failed take
  // per workgroup and queue, and a stale count plus the adds that meet it
  CHECK(tq::kMaxTiles + 2 * 4096 * tq::kQueues < (int64_t)tq::kCountMask);

  // the word rules
  CHECK(tq::count_for(tq::word(5, 17), 5) == 17u);
  CHECK(tq::count_for(tq::word(4, 17), 5) == 0u);
  CHECK(tq::count_for(0, 5) == 0u);
  CHECK(tq::after_take(tq::word(4, 17), 5) == tq::word(5, 1));
  CHECK(tq::after_take(tq::word(5, 17), 5) == tq::word(5, 18));

  const std::vector<int> tiles = {3000, 1, 0, 2500, 17, 900, 4000, 64};
  const int nq = tq::kQueues, workers = 16;

  // a fresh slot
  {
    Slot s{};
    int told = 0;
    CHECK(each_once(run_launch(s, 9, 73, workers, nq, tiles, -1, &told)));
    CHECK(told == 1);
    for (auto& w : s.w) CHECK(w.load() == tq::word(73, 0u));   // preset by the last finisher
    // the slot's next launch finds its own epoch at count 0
    CHECK(each_once(run_launch(s, 73, 137, workers, nq, tiles, -1, &told)));
    CHECK(told == 1);
  }
  // left behind by a launch that died part-way: counts of another epoch,
  // some below the tile counts, some above, the finish count part-way
  {
    Slot s{};
    int told = -1;
    (void)run_launch(s, 41, 105, workers, nq, tiles, 37, &told);
    CHECK(told == 0);
    bool dirty = false;
    for (auto& w : s.w) dirty |= w.load() != 0u;
    CHECK(dirty);
    CHECK(each_once(run_launch(s, 42, 106, workers, nq, tiles, -1, &told)));
    CHECK(told == 1);
    for (auto& w : s.w) CHECK(w.load() == tq::word(106, 0u));
    s.w[2].store(tq::word(41, 0xFFFF00u));        // a huge stale count
    s.w[tq::kQueues].store(tq::word(41, 15u));    // a stale finish count one short
    CHECK(each_once(run_launch(s, 43, 107, workers, nq, tiles, -1, &told)));
    CHECK(told == 1);
  }
  // replays with the same epoch (a captured graph) after a finished launch
  {
    Slot s{};
    int told = 0;
    for (int r = 0; r < 3; ++r) {
      CHECK(each_once(run_launch(s, 77, 141, workers, nq, tiles, -1, &told)));
      CHECK(told == 1);
    }
  }
  // a stream of launches through the slots as the host numbers them (past
  // one wrap of the epochs on every slot), every fifth one dying part-way
  {
    // as the library loads them: slot s preset for launch s
    constexpr tq::Slots init = tq::initial_slots();
    std::vector<Slot> slots(tq::kSlots);
    for (int i = 0; i < tq::kSlots; ++i)
      for (int q = 0; q < tq::kWords; ++q) {
        CHECK(init.w[i][q] == tq::word(tq::launch_epoch((uint64_t)i), 0u));
        slots[i].w[q].store(init.w[i][q]);
      }
    int ok = 0, runs = 0;
    std::vector<uint64_t> seq;
    for (uint64_t n = 0; n < 512; ++n) seq.push_back(n);                        // in turn
    for (uint64_t j = 8; j < 600; ++j) seq.push_back(j * tq::kSlots);             // one slot, epochs wrap
    for (uint64_t n = 40000; n < 60000; n += 37) seq.push_back(n);               // slots out of turn
    for (const uint64_t n : seq) {
      Slot& s = slots[tq::launch_slot(n)];
      const std::vector<int> t = {int(n % 97) * 13, 5, int(n % 7), 300, 0, 1, 2, int(n % 11) * 40};
      int told = 0;
      const bool dies = n % 5 == 4;
      auto hits = run_launch(s, tq::launch_epoch(n), tq::slot_next_epoch(n), 1 + int(n % 9), nq, t,
                             dies ? int(n % 13) : -1, &told);
      if (!dies) {
        ++runs;
        ok += each_once(hits) && told == 1;
      }
    }
    CHECK(runs > 1000);
    CHECK(ok == runs);
  }
  // contention on one word from a stale epoch: 32 threads, one install
  {
    std::atomic<uint32_t> w{tq::word(3, 1000)};
    std::vector<std::atomic<int>> hits(32 * 50);
    std::vector<std::thread> th;
    for (int b = 0; b < 32; ++b)
      th.emplace_back([&] {
        HostWord hw{&w};
        for (int i = 0; i < 50; ++i) {
          const uint32_t t = tq::take(hw, 4);
          if (t < hits.size()) hits[t].fetch_add(1);
        }
      });
    for (auto& t : th) t.join();
    bool once = true;
    for (auto& h : hits) once &= h.load() == 1;
    CHECK(once);
    CHECK(w.load() == tq::word(4, 32 * 50));
  }
  std::printf("ok: %d checks failed of %d\n", g_failed, g_checks);
  return g_failed ? 1 : 0;
}

// Tile queues of the ragged-K (weight-gradient) grouped GEMMs: the counter
// words and the rules that read them, as plain functions that the host
// compiler can run too.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 1: Grouped GEMM": one launch covers every
// expert's product, so its workgroups share out the tiles of all groups.
//
// A launch owns one slot of kQueues + 1 words: kQueues tile counters and one
// count of workgroups that have finished.  A 32-bit word holds an epoch
// (1..255, handed out by the host in turn; 0 marks a word no launch owns) in
// its top 8 bits and a count in its low 24.  A word that carries another
// epoch counts as zero, so whatever an earlier user of the slot left there
// (a launch that ended part-way included) is never taken for this launch's
// count.  The last workgroup to finish writes (the epoch of the slot's next
// launch, 0) to every word: that launch then finds its own epoch and takes
// with plain adds, and any other launch, a graph replay whose epoch is the
// one recorded at capture included, finds another epoch, which counts as
// zero.  A slot's epochs repeat only after 255 launches on it.  A launch
// has at most kMaxTiles tiles, so its counts, and those it finds left by
// another launch plus the adds that meet them, stay below 2^24 and never
// reach the epoch bits.
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

namespace moe {
namespace tq {

constexpr int kQueues = 8;           // tile counters per launch
constexpr int kWords = kQueues + 1;  // and the finished-workgroup count
constexpr int kSlots = 64;           // launches that can be in flight at once
constexpr uint32_t kEpochs = 255;
constexpr uint32_t kCountMask = (1u << 24) - 1u;
constexpr int64_t kMaxTiles = int64_t(1) << 22;

constexpr uint32_t word(uint32_t epoch, uint32_t count) { return (epoch << 24) | count; }
constexpr uint32_t epoch_of_word(uint32_t w) { return w >> 24; }

// the count that a launch of `epoch` reads from the word `seen`
constexpr uint32_t count_for(uint32_t seen, uint32_t epoch) {
  return epoch_of_word(seen) == epoch ? (seen & kCountMask) : 0u;
}
// the word that a take leaves behind when it finds `seen`
constexpr uint32_t after_take(uint32_t seen, uint32_t epoch) { return word(epoch, count_for(seen, epoch) + 1u); }

// Takes the next count of one word for the launch of `epoch`, through a
// word type with add1() (a fetch-and-add of 1, returning the old word) and
// cas(expected, desired) (returning the old word).  Fast path: one add,
// whose old word carries this launch's epoch.  A word from another epoch is
// replaced by (epoch, 1) with a compare-and-swap, which returns 0 to the one
// that installs it; the others see the installed word and go back to adds.
// Every count is handed out once: all takes are atomic read-modify-writes
// of the one word, and an add that met another epoch's word takes nothing
// (its increment is overwritten by the install).
template <class Word>
__host__ __device__ inline uint32_t take(Word& w, uint32_t epoch) {
  uint32_t old = w.add1();
  for (;;) {
    if (epoch_of_word(old) == epoch) return old & kCountMask;
    const uint32_t seen = old + 1u;   // the word as that add left it
    const uint32_t prev = w.cas(seen, word(epoch, 1u));
    if (prev == seen) return 0u;
    old = epoch_of_word(prev) == epoch ? w.add1() : prev - 1u;
  }
}

// Called once per workgroup after its last take, with the launch's
// workgroup count: true for the last one to arrive, which then writes
// word(the slot's next epoch, 0) to the launch's words.  Every other
// workgroup has made its last take by then, so no take of this launch
// follows.
template <class Word>
__host__ __device__ inline bool finish(Word& done, uint32_t epoch, uint32_t workgroups) {
  return take(done, epoch) == workgroups - 1u;
}

// host: the n-th launch (n from 0) runs in slot n % kSlots with epoch
// n % 255 + 1; the slot's next launch is launch n + kSlots
constexpr uint32_t launch_epoch(uint64_t n) { return (uint32_t)(n % kEpochs) + 1u; }
constexpr int launch_slot(uint64_t n) { return (int)(n % kSlots); }
constexpr uint32_t slot_next_epoch(uint64_t n) { return launch_epoch(n + kSlots); }

// The words of all slots, as the library loads them: slot s preset for its
// first launch, launch s, so a process's first launches take with adds too.
struct Slots {
  uint32_t w[kSlots][kWords];
};
constexpr Slots initial_slots() {
  Slots t{};
  for (int s = 0; s < kSlots; ++s)
    for (int i = 0; i < kWords; ++i) t.w[s][i] = word(launch_epoch((uint64_t)s), 0u);
  return t;
}

}  // namespace tq
}  // namespace moe

// cache_core.hpp -- host-side global LRU of the expert-slot cache (no HIP calls).
//
// Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
// on a Single Workstation GPU" (MarkTechPost), "Three mechanisms": in decode, one
// least-recently-used cache keyed over all MoE layers keeps the experts the router
// selects; nothing is cached when serving begins.
//
// Policy (the pages leave the details open; this is the reading implemented):
//  - keys are (layer, expert) -> layer*E + expert, one LRU over all layers;
//  - a step's active experts are accessed hits first, then misses, each in
//    ascending expert id, hit/miss judged against the state before the step;
//  - a miss takes the lowest-index free slot, else the least recently used key's;
//  - more active experts than slots -> consecutive waves of n_slots accesses;
//  - miss split (fill fraction num/den, default 1): of the step's m misses the
//    first floor(m num / den + 1/2) (ascending id) are accessed and filled, the
//    others are computed in place from host memory and not accessed at all.
//
// Data structures: key -> slot array over all keys, an intrusive doubly linked
// recency list over slots (head = least recent) with a strictly increasing tick,
// and an ordered set of free slots.  A wave is first planned without mutation
// (victims = free slots ascending, then the list from its head skipping the
// wave's own hits), the caller issues the fills, and only then is the wave
// committed; on a failed fill the caller invalidates the touched slots instead.
#pragma once

#include <stdint.h>

#include <set>
#include <vector>

namespace moe {

struct PlannedFill {
  int32_t slot;
  int32_t expert;
  int64_t old_key;  // key evicted from the slot, -1 if the slot was free
};

struct StepStats {
  int64_t accesses = 0, hits = 0, misses = 0, cold_misses = 0, inplace = 0;
  int32_t n_waves = 0;
};

class LruCore {
 public:
  LruCore(int n_slots, int n_layers, int n_experts);

  int n_slots() const { return S_; }
  int n_layers() const { return L_; }
  int n_experts() const { return E_; }

  // Fill fraction of the miss split (0 <= num <= den, den >= 1); between steps.
  void set_fill_fraction(int num, int den) {
    fill_num_ = num;
    fill_den_ = den;
  }
  // Start a step for `layer`: builds the access order from counts (host, [E]).
  void begin_step(int layer, const int32_t* counts);
  // Misses of the open (or last) step computed in place, ascending id.
  const std::vector<int32_t>& inplace() const { return inplace_; }
  int layer() const { return layer_; }
  bool step_open() const { return step_open_; }
  int next_wave() const { return next_wave_; }
  const StepStats& step_stats() const { return stats_; }

  // Plan wave `w` of the open step without changing the cache.  slot_table gets
  // [E] entries (slot of each expert of the wave, -1 otherwise); fills gets the
  // misses of the wave in access order.  Returns the number of accesses.
  int plan_wave(int w, int32_t* slot_table, std::vector<PlannedFill>& fills) const;
  // Apply the planned wave (accesses in order) and advance to the next wave.
  void commit_wave(int w);
  // After a failed fill: forget the keys of these slots and free them, and close
  // the step (the caller restarts with wave 0).
  void invalidate(const std::vector<int32_t>& slots);
  void abort_step() { step_open_ = false; }

  // Snapshot for comparison: key per slot (-1 empty) and last-use tick.
  void state(int64_t* key_of_slot, int64_t* tick_of_slot) const;

  // Elastic resize between steps: keep the min(new_S, resident) most recently used
  // keys, most recent first in new slots 0, 1, ...; moved_from[s] is the old slot
  // of new slot s (-1 empty).  plan_resize does not change the cache.
  void plan_resize(int new_S, std::vector<int32_t>& moved_from) const;
  void commit_resize(int new_S, const std::vector<int32_t>& moved_from);

 private:
  void unlink(int s);
  void push_tail(int s);
  int access(int64_t key);  // one sequential LRU access, returns the slot

  int S_, L_, E_;
  int64_t clock_ = 0;
  std::vector<int64_t> key_of_slot_, tick_of_slot_;
  std::vector<int32_t> prev_, next_;
  int head_ = -1, tail_ = -1;
  std::vector<int32_t> slot_of_key_;
  std::vector<uint8_t> seen_;
  std::set<int32_t> free_;

  // open step
  bool step_open_ = false;
  int layer_ = 0;
  int next_wave_ = 0;
  std::vector<int32_t> order_;  // experts in access order
  std::vector<int32_t> inplace_;
  StepStats stats_;
  int fill_num_ = 1, fill_den_ = 1;
};

}  // namespace moe

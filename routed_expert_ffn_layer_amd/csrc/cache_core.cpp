// cache_core.cpp -- global LRU of the expert-slot cache (policy in cache_core.hpp).
#include "cache_core.hpp"

#include <algorithm>

namespace moe {

LruCore::LruCore(int n_slots, int n_layers, int n_experts)
    : S_(n_slots),
      L_(n_layers),
      E_(n_experts),
      key_of_slot_(n_slots, -1),
      tick_of_slot_(n_slots, -1),
      prev_(n_slots, -1),
      next_(n_slots, -1),
      slot_of_key_((size_t)n_layers * n_experts, -1),
      seen_((size_t)n_layers * n_experts, 0) {
  for (int s = 0; s < n_slots; ++s) free_.insert(s);
}

void LruCore::unlink(int s) {
  const int p = prev_[s], n = next_[s];
  if (p >= 0) next_[p] = n; else head_ = n;
  if (n >= 0) prev_[n] = p; else tail_ = p;
  prev_[s] = next_[s] = -1;
}

void LruCore::push_tail(int s) {
  prev_[s] = tail_;
  next_[s] = -1;
  if (tail_ >= 0) next_[tail_] = s; else head_ = s;
  tail_ = s;
}

int LruCore::access(int64_t key) {
  int s = slot_of_key_[key];
  if (s >= 0) {
    unlink(s);
  } else if (!free_.empty()) {
    s = *free_.begin();
    free_.erase(free_.begin());
  } else {
    s = head_;
    unlink(s);
    slot_of_key_[key_of_slot_[s]] = -1;
  }
  key_of_slot_[s] = key;
  slot_of_key_[key] = s;
  tick_of_slot_[s] = ++clock_;
  push_tail(s);
  return s;
}

void LruCore::begin_step(int layer, const int32_t* counts) {
  layer_ = layer;
  order_.clear();
  stats_ = StepStats();
  const int64_t base = (int64_t)layer * E_;
  for (int e = 0; e < E_; ++e)
    if (counts[e] > 0 && slot_of_key_[base + e] >= 0) order_.push_back(e);
  stats_.hits = (int64_t)order_.size();
  inplace_.clear();
  int64_t m = 0;
  for (int e = 0; e < E_; ++e)
    if (counts[e] > 0 && slot_of_key_[base + e] < 0) ++m;
  const int64_t q = (2 * m * fill_num_ + fill_den_) / (2 * (int64_t)fill_den_);
  int64_t i = 0;
  for (int e = 0; e < E_; ++e)
    if (counts[e] > 0 && slot_of_key_[base + e] < 0) {
      if (i++ < q)
        order_.push_back(e);
      else
        inplace_.push_back(e);
      stats_.cold_misses += seen_[base + e] ? 0 : 1;
    }
  stats_.misses = m;
  stats_.inplace = m - q;
  stats_.accesses = stats_.hits + m;
  stats_.n_waves = order_.empty() ? 0 : (int32_t)((order_.size() - 1) / S_ + 1);
  next_wave_ = 0;
  step_open_ = true;
}

int LruCore::plan_wave(int w, int32_t* slot_table, std::vector<PlannedFill>& fills) const {
  fills.clear();
  for (int e = 0; e < E_; ++e) slot_table[e] = -1;
  const int64_t base = (int64_t)layer_ * E_;
  const size_t a0 = (size_t)w * S_;
  const size_t a1 = std::min(order_.size(), a0 + (size_t)S_);
  if (a0 >= a1) return 0;
  // keys refreshed by this wave (its hits) are never victims of its misses
  std::vector<int32_t> hit_slots;
  for (size_t a = a0; a < a1; ++a) {
    const int s = slot_of_key_[base + order_[a]];
    if (s >= 0) hit_slots.push_back(s);
  }
  std::sort(hit_slots.begin(), hit_slots.end());
  auto free_it = free_.begin();
  int victim = head_;
  for (size_t a = a0; a < a1; ++a) {
    const int e = order_[a];
    int s = slot_of_key_[base + e];
    if (s < 0) {
      PlannedFill f;
      f.expert = e;
      if (free_it != free_.end()) {
        s = *free_it++;
        f.old_key = -1;
      } else {
        while (victim >= 0 && std::binary_search(hit_slots.begin(), hit_slots.end(), victim)) victim = next_[victim];
        s = victim;  // the wave never exceeds the capacity, so a victim exists
        f.old_key = key_of_slot_[s];
        victim = next_[victim];
      }
      f.slot = s;
      fills.push_back(f);
    }
    slot_table[e] = s;
  }
  return (int)(a1 - a0);
}

void LruCore::commit_wave(int w) {
  const int64_t base = (int64_t)layer_ * E_;
  const size_t a0 = (size_t)w * S_;
  const size_t a1 = std::min(order_.size(), a0 + (size_t)S_);
  for (size_t a = a0; a < a1; ++a) {
    const int64_t key = base + order_[a];
    seen_[key] = 1;
    access(key);
  }
  next_wave_ = w + 1;
  if (next_wave_ >= stats_.n_waves) step_open_ = false;
}

void LruCore::invalidate(const std::vector<int32_t>& slots) {
  for (int s : slots) {
    if (key_of_slot_[s] >= 0) {
      slot_of_key_[key_of_slot_[s]] = -1;
      key_of_slot_[s] = -1;
      tick_of_slot_[s] = -1;
      unlink(s);
      free_.insert(s);
    }
  }
  step_open_ = false;
}

void LruCore::state(int64_t* key_of_slot, int64_t* tick_of_slot) const {
  for (int s = 0; s < S_; ++s) {
    key_of_slot[s] = key_of_slot_[s];
    tick_of_slot[s] = tick_of_slot_[s];
  }
}

void LruCore::plan_resize(int new_S, std::vector<int32_t>& moved_from) const {
  std::vector<int32_t> resident;
  for (int q = 0; q < S_; ++q)
    if (key_of_slot_[q] >= 0) resident.push_back(q);
  std::sort(resident.begin(), resident.end(),
            [&](int32_t x, int32_t y) { return tick_of_slot_[x] > tick_of_slot_[y]; });
  moved_from.assign(new_S, -1);
  const int keep = (int)std::min<size_t>((size_t)new_S, resident.size());
  for (int q = 0; q < keep; ++q) moved_from[q] = resident[q];
}

void LruCore::commit_resize(int new_S, const std::vector<int32_t>& moved_from) {
  std::vector<int64_t> key2(new_S, -1), tick2(new_S, -1);
  for (int q = 0; q < S_; ++q)
    if (key_of_slot_[q] >= 0) slot_of_key_[key_of_slot_[q]] = -1;
  int keep = 0;
  for (int q = 0; q < new_S; ++q) {
    if (moved_from[q] < 0) continue;
    key2[q] = key_of_slot_[moved_from[q]];
    tick2[q] = tick_of_slot_[moved_from[q]];
    slot_of_key_[key2[q]] = q;
    keep = q + 1;
  }
  S_ = new_S;
  key_of_slot_.swap(key2);
  tick_of_slot_.swap(tick2);
  prev_.assign(new_S, -1);
  next_.assign(new_S, -1);
  head_ = tail_ = -1;
  for (int q = keep - 1; q >= 0; --q) push_tail(q);  // least recent (highest slot) first
  free_.clear();
  for (int q = keep; q < new_S; ++q) free_.insert(q);
}

}  // namespace moe

#include "lfu.hpp"

#include <algorithm>

namespace moe {

void LfuPolicy::prefetch(const int32_t* experts, int n, int32_t* slot_out, int32_t* evicted_out) {
  const int ns = (int)slots.size();
  std::vector<char> pinned(ns, 0);
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) {
    order[i] = i;
    slot_out[i] = evicted_out[i] = -1;
  }
  std::sort(order.begin(), order.end(), [&](int a, int b) { return experts[a] < experts[b]; });
  for (int i : order) {
    if (find(experts[i]) >= 0) continue;
    int victim = -1;
    for (int s = 0; s < ns && victim < 0; ++s)
      if (slots[s].expert < 0) victim = s;
    if (victim < 0) {
      for (int s = 0; s < ns; ++s) {
        if (pinned[s] || (slots[s].tick == now && !slots[s].fetched_ahead)) continue;  // last call's working set
        const Slot& a = slots[s];
        if (victim < 0 || a.count < slots[victim].count ||
            (a.count == slots[victim].count && a.tick < slots[victim].tick))
          victim = s;
      }
      if (victim < 0) continue;  // every slot holds this prefetch's entries
      ++evictions;
      evicted_out[i] = slots[victim].expert;
    }
    slots[victim] = Slot{experts[i], 0, now, true};
    pinned[victim] = 1;
    ++prefetches;
    slot_out[i] = victim;
  }
}

int LfuPolicy::find(int32_t expert) const {
  for (size_t s = 0; s < slots.size(); ++s)
    if (slots[s].expert == expert) return (int)s;
  return -1;
}

void LfuPolicy::clear_contents() {
  for (auto& s : slots) s = Slot{};
}

bool LfuPolicy::step(const int32_t* chosen, int n, int32_t* slot_out, int32_t* miss_out, int32_t* evicted_out) {
  const int ns = (int)slots.size();
  if (n > ns) return false;
  ++now;
  std::vector<char> pinned(ns, 0);
  std::vector<int> miss_idx;
  // hits first
  for (int i = 0; i < n; ++i) {
    int s = find(chosen[i]);
    ++accesses;
    if (s >= 0) {
      ++hits;
      if (slots[s].fetched_ahead) ++prefetch_used;
      slots[s].fetched_ahead = false;
      slots[s].count += 1;
      slots[s].tick = now;
      pinned[s] = 1;
      slot_out[i] = s;
      miss_out[i] = 0;
      if (evicted_out) evicted_out[i] = -1;
    } else {
      miss_idx.push_back(i);
    }
  }
  // misses in ascending expert order
  std::sort(miss_idx.begin(), miss_idx.end(), [&](int a, int b) { return chosen[a] < chosen[b]; });
  for (int i : miss_idx) {
    int victim = -1;
    for (int s = 0; s < ns; ++s)
      if (slots[s].expert < 0) {
        victim = s;
        break;
      }
    if (victim < 0) {
      for (int s = 0; s < ns; ++s) {
        if (pinned[s]) continue;
        if (victim < 0) {
          victim = s;
          continue;
        }
        const Slot &a = slots[s], &v = slots[victim];
        if (a.count < v.count || (a.count == v.count && a.tick < v.tick)) victim = s;
      }
      ++evictions;
    }
    if (evicted_out) evicted_out[i] = slots[victim].expert;
    slots[victim].expert = chosen[i];
    slots[victim].count = 1;
    slots[victim].tick = now;
    slots[victim].fetched_ahead = false;
    pinned[victim] = 1;
    ++misses;
    slot_out[i] = victim;
    miss_out[i] = 1;
  }
  return true;
}

}  // namespace moe

namespace moe {

int LruPool::find(int32_t layer, int32_t expert) const {
  for (size_t s = 0; s < slots.size(); ++s)
    if (slots[s].layer == layer && slots[s].expert == expert) return (int)s;
  return -1;
}

void LruPool::drop_layer(int32_t layer) {
  for (auto& s : slots)
    if (s.layer == layer) s = Slot{};
}

bool LruPool::step(int32_t layer, const int32_t* chosen, int n, int32_t* slot_out, int32_t* miss_out,
                   int32_t* ev_layer, int32_t* ev_expert) {
  const int ns = (int)slots.size();
  if (n > ns) return false;
  ++now;
  std::vector<char> pinned(ns, 0);
  std::vector<int> miss_idx;
  for (int i = 0; i < n; ++i) {  // hits first
    const int s = find(layer, chosen[i]);
    ++accesses;
    ev_layer[i] = ev_expert[i] = -1;
    if (s >= 0) {
      ++hits;
      slots[s].tick = now;
      pinned[s] = 1;
      slot_out[i] = s;
      miss_out[i] = 0;
    } else {
      miss_idx.push_back(i);
    }
  }
  std::sort(miss_idx.begin(), miss_idx.end(), [&](int a, int b) { return chosen[a] < chosen[b]; });
  for (int i : miss_idx) {
    int victim = -1;
    for (int s = 0; s < ns && victim < 0; ++s)
      if (slots[s].expert < 0) victim = s;
    if (victim < 0) {
      for (int s = 0; s < ns; ++s)
        if (!pinned[s] && (victim < 0 || slots[s].tick < slots[victim].tick)) victim = s;
      ++evictions;
      ev_layer[i] = slots[victim].layer;
      ev_expert[i] = slots[victim].expert;
    }
    slots[victim] = Slot{layer, chosen[i], now};
    pinned[victim] = 1;
    ++misses;
    slot_out[i] = victim;
    miss_out[i] = 1;
  }
  return true;
}

}  // namespace moe

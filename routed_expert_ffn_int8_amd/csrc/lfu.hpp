// Per-layer expert-cache policy: LFU with an LRU tie-break and pinning of the
// experts chosen by the current call.  Pure host C++ (no HIP), so it can be
// exercised without a GPU.
//
// Rockchip-NPU MoE streaming plan (cnblogs): §6.2.2 gives the cache entry
// (expert, use count, last-used tick) and a fixed array of slots per layer;
// §6.2.3's cache increments the count on a hit, fills an empty slot first,
// otherwise evicts the entry with the smallest count, and starts a new entry
// at count 1; §9.5 item 1 prefers LFU over LRU for MoE.  Where the plan is
// silent: ties on the count go to the older last-used tick, then the lower
// slot; entries chosen by the current call are never its victims; counts are
// never aged; hits are applied before misses and misses are placed in
// ascending expert order.
#pragma once
#include <cstdint>
#include <vector>

namespace moe {

struct LfuPolicy {
  struct Slot {
    int32_t expert = -1;
    uint32_t count = 0;
    uint64_t tick = 0;
    bool fetched_ahead = false;  // placed by prefetch and not yet used by a call
  };
  std::vector<Slot> slots;
  uint64_t now = 0;
  uint64_t accesses = 0, hits = 0, misses = 0, evictions = 0;
  uint64_t prefetches = 0, prefetch_used = 0;

  explicit LfuPolicy(int n_slots) : slots(n_slots) {}

  // Fetch ahead (Rockchip-NPU plan §8 readahead, §9.5 item 2): place the
  // experts of `experts` that are absent, in ascending id order, without
  // counting an access.  Each takes the lowest empty slot, else evicts as a
  // miss would, but never an entry placed by the same prefetch nor one the
  // last call used (the working set, BigMoeOnEdge: the working set in use is
  // protected); with no such slot left the guess is dropped.  A new entry
  // starts at count 0 with the last call's tick, so a guess that no call
  // uses is the first to go; a call's hit on it counts as prefetch_used.
  // slot_out[i] / evicted_out[i] for experts[i]: -1 where it was present.
  void prefetch(const int32_t* experts, int n, int32_t* slot_out, int32_t* evicted_out);

  // Decide where each chosen expert lives for this call.  `chosen` holds n
  // distinct ids.  slot_out[i] / miss_out[i] describe chosen[i]; for a miss,
  // evicted_out[i] is the expert that slot held before (-1 if it was empty).
  // Returns false (and changes nothing) if n exceeds the slot count.
  bool step(const int32_t* chosen, int n, int32_t* slot_out, int32_t* miss_out, int32_t* evicted_out);

  // Look where an expert is without counting an access (-1 if absent).
  int find(int32_t expert) const;
  void clear_contents();
  void clear_counters() { accesses = hits = misses = evictions = prefetches = prefetch_used = 0; }
};

}  // namespace moe

namespace moe {

// Expert cache shared by several layers under one byte budget, LRU.
//
// BigMoeOnEdge, "the cache manages the expert working set": entries are
// keyed by (layer, expert), the budget covers expert weights only, least
// recently used entries go first, and the working set in use is protected
// (the page lets residency exceed the budget for it; here every slot has
// the size of one expert, and a call needing more slots than the budget
// holds is refused).  Readings where the page is silent: an empty slot is
// taken first (lowest index); among the other slots, entries chosen by the
// current call are never its victims, the oldest last-use goes first, then
// the lower slot; hits are applied before misses, misses in ascending
// expert order; one access per (call, chosen expert).
struct LruPool {
  struct Slot {
    int32_t layer = -1, expert = -1;
    uint64_t tick = 0;
  };
  std::vector<Slot> slots;
  uint64_t now = 0;
  uint64_t accesses = 0, hits = 0, misses = 0, evictions = 0;

  explicit LruPool(int n_slots) : slots(n_slots) {}

  // Place the n distinct experts `chosen` of `layer` for one call.
  // slot_out[i] / miss_out[i] describe chosen[i]; for a miss that evicted an
  // entry, ev_layer[i] / ev_expert[i] name it (-1 if the slot was empty).
  // Returns false (and changes nothing) if n exceeds the slot count.
  bool step(int32_t layer, const int32_t* chosen, int n, int32_t* slot_out, int32_t* miss_out, int32_t* ev_layer,
            int32_t* ev_expert);
  int find(int32_t layer, int32_t expert) const;
  void drop_layer(int32_t layer);  // empty every slot of `layer`
  void clear_counters() { accesses = hits = misses = evictions = 0; }
};

}  // namespace moe

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
  };
  std::vector<Slot> slots;
  uint64_t now = 0;
  uint64_t accesses = 0, hits = 0, misses = 0, evictions = 0;

  explicit LfuPolicy(int n_slots) : slots(n_slots) {}

  // Decide where each chosen expert lives for this call.  `chosen` holds n
  // distinct ids.  slot_out[i] / miss_out[i] describe chosen[i]; for a miss,
  // evicted_out[i] is the expert that slot held before (-1 if it was empty).
  // Returns false (and changes nothing) if n exceeds the slot count.
  bool step(const int32_t* chosen, int n, int32_t* slot_out, int32_t* miss_out, int32_t* evicted_out);

  // Look where an expert is without counting an access (-1 if absent).
  int find(int32_t expert) const;
  void clear_contents();
  void clear_counters() { accesses = hits = misses = evictions = 0; }
};

}  // namespace moe

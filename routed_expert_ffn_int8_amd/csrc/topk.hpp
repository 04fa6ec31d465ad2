// Softmax top-K of one token by one wavefront, shared by the decode and
// prefill kernels.
//
// Gating (BigMoeOnEdge, section "re-routing at every token and layer"; the
// Rockchip-NPU plan, section 2.1): order the experts by logit, descending,
// lower index first on ties; keep the first K; their coefficients are a
// softmax over the chosen logits, which equals a softmax over all experts
// renormalised to the chosen ones.  Chosen experts are reported in ascending
// index order.
#pragma once
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Orderable 32-bit key of a logit: larger logit -> larger key (-0 == +0).
__device__ __forceinline__ uint32_t order_key(float l) {
  uint32_t u = __float_as_uint(l + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Radix search for the K-th largest key over the wavefront's NE keys per lane:
// returns a value P with at least K keys >= P and, below every key >= P that
// is not equal to P, fewer than K keys.  Bits are decided from the top; the
// search stops as soon as exactly K keys are >= P (then any key >= P is chosen
// and ties cannot cross P), which for distinct logits happens after a few
// bits instead of all 32.
template <int NE>
__device__ __forceinline__ uint32_t kth_prefix(const uint32_t (&key)[NE], int K) {
  uint32_t prefix = 0;
  int c = 64 * NE;  // keys >= prefix
  for (int bit = 31; bit >= 0 && c != K; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NE; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= K) {
      prefix = cand;
      c = cnt;
    }
  }
  return prefix;
}

// Coefficients of a chosen set held in LDS (`scratch`: ids ascending in
// [0, K), their logits in [K, 2K)), by one wavefront: lane k < K takes the
// k-th chosen expert; the maximum and the denominator are whole-wavefront
// reductions in a fixed order (DPP), so every lane holds the same bits and
// every kernel that fills scratch alike gets the same coefficients.
__device__ __forceinline__ void topk_finish(int K, const uint32_t* scratch, int* id_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  const int my_id = lane < K ? (int)scratch[lane] : 0;
  const float my_l = lane < K ? __uint_as_float(scratch[K + lane]) : -INFINITY;
  const uint32_t km = wave_max_u32(lane < K ? order_key(my_l) : 0u);  // the largest chosen key, as a float:
  const float mx = __uint_as_float((km & 0x80000000u) ? (km & 0x7FFFFFFFu) : ~km);
  const float v = lane < K ? expf(my_l - mx) : 0.f;
  const float den = wave_sum_f32(v);
  *id_out = my_id;
  *w_out = v / den;
}

// Softmax top-K of token t by one wavefront (lane = threadIdx.x & 63).
// Selection order: logit descending, expert index ascending on ties.  The
// K-th largest key is found by a radix search over the 32 key bits with
// wavefront ballots (no cross-lane data movement), ties at that key are
// taken in index order, and the chosen experts are compacted in ascending
// index order.  Weights: softmax over the chosen set, i.e. a softmax over
// all experts renormalised to the chosen ones.  On return lane k < K holds
// the k-th chosen expert (ascending) in *id and its weight in *w.
// `scratch` is LDS space for 2*K words private to this wavefront.
// NE = logits held per lane (E <= 64 * NE), a compile-time constant so the
// radix loop has no per-slice branches.
template <int NE>
__device__ void topk_wave(const LayerArgs& a, int t, const float* lt, int* id_out, float* w_out, uint32_t* scratch) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.K;
  int my_id = 0;
  float my_l = -INFINITY;
  if (a.forced) {
    if (lane < K) {
      my_id = a.forced[(size_t)t * K + lane];
      if (my_id < 0 || my_id >= E) {
        atomicOr(a.err, kErrBadForcedId);
        my_id = 0;
      }
      my_l = lt[my_id];
    }
    int rank = 0;
    for (int j = 0; j < K; ++j) {  // ascending order, unique rank even for repeated ids
      const int o = __shfl(my_id, j, 64);
      rank += (o < my_id || (o == my_id && j < lane)) ? 1 : 0;
    }
    if (lane < K) {
      scratch[rank] = (uint32_t)my_id;
      scratch[K + rank] = __float_as_uint(my_l);
    }
  } else if (K <= 16) {
    // K rounds of: the wavefront maximum of the remaining keys (DPP), the
    // lowest expert index holding it (ballots), which leaves the pool.  Then
    // the chosen entries are compacted in ascending index order.
    uint32_t key[NE];
    float lv[NE];
    bool sel[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E;
      lv[i] = ok ? lt[e] : -INFINITY;
      key[i] = ok ? order_key(lv[i]) : 0u;
      sel[i] = false;
    }
    for (int k = 0; k < K; ++k) {
      uint32_t lm = key[0];
#pragma unroll
      for (int i = 1; i < NE; ++i) lm = max(lm, key[i]);
      const uint32_t m = wave_max_u32(lm);
      int slot = -1, at = 0;
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const uint64_t b = __ballot(key[i] == m);
        if (slot < 0 && b != 0) {
          slot = i;
          at = (int)__builtin_ctzll(b);
        }
      }
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (i == slot && lane == at) {
          key[i] = 0u;
          sel[i] = true;
        }
    }
    int pos_base = 0;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const uint64_t sm = __ballot(sel[i]);
      if (sel[i]) {
        const int pos = pos_base + lanes_below(sm);
        scratch[pos] = (uint32_t)(lane + 64 * i);
        scratch[K + pos] = __float_as_uint(lv[i]);
      }
      pos_base += __popcll(sm);
    }
  } else {
    uint32_t key[NE];
    float lv[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E;
      lv[i] = ok ? lt[e] : -INFINITY;
      key[i] = ok ? order_key(lv[i]) : 0u;
    }
    const uint32_t prefix = kth_prefix<NE>(key, K);
    int gt = 0;
#pragma unroll
    for (int i = 0; i < NE; ++i) gt += __popcll(__ballot(key[i] > prefix));
    const int need = K - gt;
    int eq_before = 0, pos_base = 0;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      {
        const int e = lane + 64 * i;
        const bool valid = e < E;
        const uint64_t eqm = __ballot(valid && key[i] == prefix);
        const bool take_eq = valid && key[i] == prefix && (eq_before + lanes_below(eqm)) < need;
        eq_before += __popcll(eqm);
        const bool sel = key[i] > prefix || take_eq;
        const uint64_t sm = __ballot(sel);
        if (sel) {
          const int pos = pos_base + lanes_below(sm);
          scratch[pos] = (uint32_t)e;
          scratch[K + pos] = __float_as_uint(lv[i]);
        }
        pos_base += __popcll(sm);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses complete in order
  topk_finish(K, scratch, id_out, w_out);
}

// The k-th chosen expert of token t (ascending order), uniform across the
// calling wavefront: the same radix search as topk_wave, then the lane whose
// compacted position is k is located with a ballot; no data leaves a lane.
template <int NE>
__device__ int topk_kth(const LayerArgs& a, int t, const float* lt, int k) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.K;
  if (a.forced) {
    int my_id = 0;
    if (lane < K) {  // an out-of-range id is replaced by 0 (and flagged by topk_wave)
      const int v = a.forced[(size_t)t * K + lane];
      my_id = (v < 0 || v >= E) ? 0 : v;
    }
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int o = __shfl(my_id, j, 64);
      rank += (o < my_id || (o == my_id && j < lane)) ? 1 : 0;
    }
    const uint64_t m = __ballot(lane < K && rank == k);
    return __shfl(my_id, (int)__builtin_ctzll(m), 64);
  }
  uint32_t key[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? order_key(lt[e]) : 0u;
  }
  const uint32_t prefix = kth_prefix<NE>(key, K);
  int gt = 0;
#pragma unroll
  for (int i = 0; i < NE; ++i) gt += __popcll(__ballot(key[i] > prefix));
  const int need = K - gt;
  int eq_before = 0, pos_base = 0, found = 0;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    {
      const int e = lane + 64 * i;
      const bool valid = e < E;
      const uint64_t eqm = __ballot(valid && key[i] == prefix);
      const bool take_eq = valid && key[i] == prefix && (eq_before + lanes_below(eqm)) < need;
      eq_before += __popcll(eqm);
      const bool sel = key[i] > prefix || take_eq;
      const uint64_t sm = __ballot(sel);
      const uint64_t hit = __ballot(sel && pos_base + lanes_below(sm) == k);
      if (hit) found = (int)__builtin_ctzll(hit) + 64 * i;
      pos_base += __popcll(sm);
    }
  }
  return found;
}

// Publish the routing of token t (lane k < K holds the k-th chosen expert).
__device__ __forceinline__ void publish_routing(const LayerArgs& a, int t, int lane, int id, float w) {
  if (lane < a.K) {
    const size_t o = (size_t)t * a.K + lane;
    if (a.ids != a.forced)  // reusing the stored sets: they stay as they are
      __hip_atomic_store(a.ids + o, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // read by the prefill sort
    a.wts[o] = w;
    a.sel_addr[o] = a.expert_addr[id];
    if (a.ids_out) a.ids_out[o] = id;
    if (a.w_out) a.w_out[o] = w;
  }
}

}  // namespace
}  // namespace moe

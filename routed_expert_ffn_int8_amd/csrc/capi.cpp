// C ABI of the MoE FFN library: descriptor validation, weight repack and
// upload, workspace management, kernel launch sequencing, the streamed expert
// cache and the stack driver.  No PyTorch types cross this boundary.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <string>
#include <thread>
#include <vector>

#include "../../include/moe.h"
#include "kernels.hpp"
#include "layout.hpp"
#include "lfu.hpp"

namespace moe {
size_t decode_lds_bytes_x(int d);
size_t decode_arep_bytes(int F);
size_t decode_lds_bytes_down(int F, int NI, int K, int act);
size_t prefill_workspace_bytes(int T, int d, int E, int K, int f, int fs);
void prefill_carve(PrefillArgs& p, char* ws, int T, int d, int E, int K, int f, int fs);
}  // namespace moe

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_OK(expr)                                                                                   \
  do {                                                                                                 \
    hipError_t e_ = (expr);                                                                            \
    if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));     \
  } while (0)

template <class T>
hipError_t dalloc(T** p, size_t bytes) {
  return hipMalloc(reinterpret_cast<void**>(p), bytes ? bytes : 16);
}

// Brackets kernel launches with pooled HIP events; durations are read back
// (after a device sync) by moe_layer_profile_read.
struct EventProfiler : Profiler {
  struct Rec {
    int kernel;
    hipEvent_t a, b;
  };
  std::vector<hipEvent_t> pool;
  std::vector<Rec> recs;
  hipError_t err = hipSuccess;
  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) err = r;
    return e;
  }
  void pair(int kernel, hipEvent_t* a, hipEvent_t* b) override {
    *a = take();
    *b = take();
    if (*a && *b) recs.push_back(Rec{kernel, *a, *b});
  }
  ~EventProfiler() override {
    for (auto& r : recs) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

}  // namespace

struct moe_layer {
  int dev = 0;
  int d = 0, E = 0, K = 0, f = 0, fs = 0, act = 0, max_tokens = 0, residency = 0;
  BlobLayout rl, sl;
  BlobOffsets ro{}, so{};
  // device weights
  uint8_t* d_experts = nullptr;  // resident: E blobs at stride rl.stride
  uint8_t* d_shared = nullptr;
  uint8_t* d_zero = nullptr;  // one all-zero routed blob
  int8_t* d_router_w = nullptr;
  uint16_t* d_router_scale = nullptr;
  float* d_router_bias = nullptr;
  uint64_t* d_expert_addr = nullptr;  // [E]
  // decode workspace
  float* d_logits = nullptr;
  int32_t* d_ids = nullptr;
  uint64_t* d_sel = nullptr;  // [T][K] blob address per chosen expert
  float* d_wts = nullptr;
  uint32_t* d_counter = nullptr;
  void* d_abuf = nullptr;
  void* d_arep = nullptr;  // the fused kernel's activation copies
  int32_t* d_err = nullptr;
  // prefill workspace
  char* d_prefill = nullptr;
  size_t prefill_bytes = 0;
  // previous call (for reuse_previous)
  int prev_T = -1;
  int default_path = MOE_PATH_AUTO;  // what a call passing MOE_PATH_AUTO runs
  int fused_ok = -1;  // whether the single-launch decode kernel serves this layer here (-1: not yet known)
  // streamed experts
  uint8_t* h_store = nullptr;  // pinned, E blobs
  const uint8_t* d_store = nullptr;  // its device view
  uint8_t* d_slots = nullptr;
  int n_slots = 0;
  std::unique_ptr<LfuPolicy> lfu;
  moe_cache_pool* pool = nullptr;  // or a cache shared with other layers
  int pool_id = -1;                // this layer's key in it
  hipStream_t side = nullptr;
  bool own_side = false;
  hipEvent_t ev_fill = nullptr, ev_fill_start = nullptr;
  bool fill_pending = false;
  hipEvent_t ev_ahead = nullptr;  // after the last prefetch's copies
  bool ahead_pending = false;
  std::vector<uint32_t> hist;     // calls that chose each expert (the prefetch predictor)
  uint64_t* h_addr = nullptr;  // pinned mirror of d_expert_addr
  bool addr_dirty = false;     // h_addr changed since d_expert_addr was last uploaded
  int32_t* h_ids = nullptr;    // pinned, coherent routing copy [max_tokens*K], then a sequence word
  void* d_host_ids = nullptr;  // its device view
  uint32_t host_seq = 0;       // sequence number of the last one-token routing written by the GPU
  bool h_ids_last = false;     // h_ids holds the routing of this layer's last call (a one-token streamed call)
  int64_t host_wait_us = 2000000;  // how long the host spins for that routing before it waits for the stream
  int32_t* h_pf = nullptr;     // prefill through the cache: pinned counts [E], then group tile lists
  int32_t* d_pf_tiles = nullptr;  // the group tile lists on the device
  size_t pf_ints = 0;          // capacity of both lists, in ints
  uint64_t* h_pf_addr = nullptr;  // pinned snapshots of the expert table, one per group of a chunk
  size_t pf_groups = 0;           // their count
  std::vector<char> fail_expert;
  moe_cache_stats stats{};
  uint64_t device_bytes = 0;
  std::unique_ptr<EventProfiler> prof;
};

moe_status launch_prefill_path(moe_layer* L, const LayerArgs& a, const moe_fwd_opts* o, hipStream_t s);

struct moe_stack {
  std::vector<moe_layer*> layers;
  float eps = 1e-6f;
  int prefetch_depth = 0;
  // One synchronisation area and one set of activation copies per layer
  // shape (E, K, d_ff, d_ff_shared), shared by the fused launches of every
  // layer of that shape.  The layers run one after another, so one area's
  // launch count serves them all (its tag just keeps counting), and the area
  // stays in cache instead of each layer touching its own cold one.  Layers
  // of another shape need their own: a stage counter grows by the number of
  // that stage's workgroups per launch, which depends on the shape, and the
  // activation copies are laid out for one vector length.
  int dev = 0;
  std::vector<uint32_t*> d_counter;  // per shape
  std::vector<void*> d_arep;         // per shape
  std::vector<int> area_of;          // per layer: index of its shape's area
};

struct moe_lfu {
  LfuPolicy policy;
  explicit moe_lfu(int n) : policy(n) {}
};

struct moe_lru {
  LruPool policy;
  explicit moe_lru(int n) : policy(n) {}
};

// One expert cache for many streamed layers: slots of one expert blob each,
// as many as the byte budget holds, LRU over (layer, expert).
struct moe_cache_pool {
  int dev = 0;
  uint64_t expert_bytes = 0;
  int n_slots = 0;
  uint8_t* d_slots = nullptr;
  std::unique_ptr<LruPool> policy;
  std::vector<moe_layer*> members;  // by key; null once a layer has left
  moe_cache_stats stats{};
};

namespace {

moe_status validate(const moe_layer_desc* D) {
  if (!D) return fail(MOE_ERR_INVALID, "descriptor is NULL");
  if (D->d_model <= 0 || D->d_model % 64 || D->d_model > 8192)
    return fail(MOE_ERR_INVALID, "d_model=%d must be a positive multiple of 64 and <= 8192", D->d_model);
  if (D->n_experts < 1 || D->n_experts > 1024) return fail(MOE_ERR_INVALID, "n_experts=%d not in 1..1024", D->n_experts);
  if (D->top_k < 1 || D->top_k > D->n_experts || D->top_k > 64)
    return fail(MOE_ERR_INVALID, "top_k=%d must be in 1..min(E,64)", D->top_k);
  if (D->d_ff <= 0 || D->d_ff % 64) return fail(MOE_ERR_INVALID, "d_ff=%d must be a positive multiple of 64", D->d_ff);
  if (D->d_ff_shared < 0 || D->d_ff_shared % 64)
    return fail(MOE_ERR_INVALID, "d_ff_shared=%d must be a multiple of 64 (or 0)", D->d_ff_shared);
  if (D->act_dtype != MOE_ACT_F32 && D->act_dtype != MOE_ACT_BF16)
    return fail(MOE_ERR_INVALID, "act_dtype=%d unknown", D->act_dtype);
  if (D->max_tokens < 1 || D->max_tokens > 65536) return fail(MOE_ERR_INVALID, "max_tokens=%d not in 1..65536", D->max_tokens);
  if (D->residency != MOE_RESIDENT && D->residency != MOE_STREAMED)
    return fail(MOE_ERR_INVALID, "residency=%d unknown", D->residency);
  if (!D->router_w || !D->router_scale || !D->gate_q || !D->gate_s || !D->gate_b || !D->up_q || !D->up_s ||
      !D->up_b || !D->down_q || !D->down_s || !D->down_b)
    return fail(MOE_ERR_INVALID, "a routed weight pointer is NULL");
  if (D->d_ff_shared > 0 && (!D->sh_gate_q || !D->sh_gate_s || !D->sh_gate_b || !D->sh_up_q || !D->sh_up_s ||
                             !D->sh_up_b || !D->sh_down_q || !D->sh_down_s || !D->sh_down_b))
    return fail(MOE_ERR_INVALID, "a shared-expert weight pointer is NULL");
  const int F = D->d_ff_shared + D->top_k * D->d_ff;
  const int NI = D->d_ff_shared / 64 + D->top_k * (D->d_ff / 64);
  if (decode_lds_bytes_down(F, NI, D->top_k, D->act_dtype) > 64 * 1024)
    return fail(MOE_ERR_INVALID, "d_ff_shared + top_k*d_ff = %d too large for the decode combine kernel", F);
  return MOE_OK;
}

BlobOffsets offsets_of(const BlobLayout& L) {
  return BlobOffsets{(uint32_t)L.gate.q_off, (uint32_t)L.gate.sb_off, (uint32_t)L.up.q_off,
                     (uint32_t)L.up.sb_off,  (uint32_t)L.down.q_off, (uint32_t)L.down.sb_off};
}

// Repack experts [e0, e1) of the canonical arrays into consecutive blobs.
void pack_experts(const moe_layer_desc* D, const BlobLayout& L, int e0, int e1, uint8_t* dst) {
  const size_t gu_w = (size_t)D->d_ff * D->d_model / 8, gu_g = (size_t)D->d_ff * D->d_model / 64;
  for (int e = e0; e < e1; ++e) {
    uint8_t* blob = dst + (size_t)(e - e0) * L.stride;
    std::memset(blob, 0, L.stride);
    pack_matrix(L.gate, D->gate_q + e * gu_w, D->gate_s + e * gu_g, D->gate_b + e * gu_g, blob);
    pack_matrix(L.up, D->up_q + e * gu_w, D->up_s + e * gu_g, D->up_b + e * gu_g, blob);
    pack_matrix(L.down, D->down_q + e * gu_w, D->down_s + e * gu_g, D->down_b + e * gu_g, blob);
  }
}

void pack_parallel(const moe_layer_desc* D, const BlobLayout& L, uint8_t* dst) {
  const int E = D->n_experts;
  const int nt = std::max(1, std::min<int>(E, (int)std::thread::hardware_concurrency()));
  std::vector<std::thread> th;
  for (int i = 0; i < nt; ++i) {
    const int e0 = E * i / nt, e1 = E * (i + 1) / nt;
    th.emplace_back([=] { pack_experts(D, L, e0, e1, dst + (size_t)e0 * L.stride); });
  }
  for (auto& t : th) t.join();
}

// Take a layer out of its shared cache: its entries become empty slots.
void leave_pool(moe_layer* L) {
  if (!L->pool) return;
  L->pool->policy->drop_layer(L->pool_id);
  L->pool->members[L->pool_id] = nullptr;
  L->pool = nullptr;
  L->pool_id = -1;
}

void free_layer(moe_layer* L) {
  if (!L) return;
  (void)hipDeviceSynchronize();
  leave_pool(L);
  (void)hipFree(L->d_experts);
  (void)hipFree(L->d_shared);
  (void)hipFree(L->d_zero);
  (void)hipFree(L->d_router_w);
  (void)hipFree(L->d_router_scale);
  (void)hipFree(L->d_router_bias);
  (void)hipFree(L->d_expert_addr);
  (void)hipFree(L->d_logits);
  (void)hipFree(L->d_ids);
  (void)hipFree(L->d_sel);
  (void)hipFree(L->d_wts);
  (void)hipFree(L->d_counter);
  (void)hipFree(L->d_abuf);
  (void)hipFree(L->d_arep);
  (void)hipFree(L->d_err);
  (void)hipFree(L->d_prefill);
  (void)hipFree(L->d_slots);
  if (L->h_store) (void)hipHostFree(L->h_store);
  if (L->h_addr) (void)hipHostFree(L->h_addr);
  if (L->h_ids) (void)hipHostFree(L->h_ids);
  if (L->h_pf) (void)hipHostFree(L->h_pf);
  if (L->h_pf_addr) (void)hipHostFree(L->h_pf_addr);
  (void)hipFree(L->d_pf_tiles);
  if (L->ev_fill) (void)hipEventDestroy(L->ev_fill);
  if (L->ev_fill_start) (void)hipEventDestroy(L->ev_fill_start);
  if (L->ev_ahead) (void)hipEventDestroy(L->ev_ahead);
  if (L->own_side && L->side) (void)hipStreamDestroy(L->side);
  delete L;
}

moe_status create_impl(const moe_layer_desc* D, moe_layer* L) {
  HIP_OK(hipGetDevice(&L->dev));
  L->d = D->d_model;
  L->E = D->n_experts;
  L->K = D->top_k;
  L->f = D->d_ff;
  L->fs = D->d_ff_shared;
  L->act = D->act_dtype;
  L->max_tokens = D->max_tokens;
  L->residency = D->residency;
  L->rl = make_blob_layout(L->d, L->f);
  L->ro = offsets_of(L->rl);
  if (L->fs > 0) {
    L->sl = make_blob_layout(L->d, L->fs);
    L->so = offsets_of(L->sl);
  }
  const size_t E = L->E, stride = L->rl.stride;
  uint64_t dev_bytes = 0;
  // routed experts
  std::vector<uint64_t> addr(E, 0);
  if (L->residency == MOE_RESIDENT) {
    if (dalloc(&L->d_experts, E * stride) != hipSuccess)
      return fail(MOE_ERR_NOMEM, "hipMalloc of %zu bytes of expert weights failed", E * stride);
    dev_bytes += E * stride;
    std::vector<uint8_t> host(E * stride);
    pack_parallel(D, L->rl, host.data());
    HIP_OK(hipMemcpy(L->d_experts, host.data(), E * stride, hipMemcpyHostToDevice));
    for (size_t e = 0; e < E; ++e) addr[e] = reinterpret_cast<uint64_t>(L->d_experts + e * stride);
  } else {
    if (hipHostMalloc(reinterpret_cast<void**>(&L->h_store), E * stride, hipHostMallocDefault) != hipSuccess)
      return fail(MOE_ERR_NOMEM, "pinned host store of %zu bytes failed", E * stride);
    pack_parallel(D, L->rl, L->h_store);
    void* dv = nullptr;  // the fill kernel reads the store through its device view
    HIP_OK(hipHostGetDevicePointer(&dv, L->h_store, 0));
    L->d_store = static_cast<const uint8_t*>(dv);
    // pinned mirror of the device expert table [E]
    if (hipHostMalloc(reinterpret_cast<void**>(&L->h_addr), E * 8, hipHostMallocDefault) != hipSuccess)
      return fail(MOE_ERR_NOMEM, "pinned expert table failed");
    std::memset(L->h_addr, 0, E * 8);
    L->fail_expert.assign(E, 0);
  }
  if (dalloc(&L->d_zero, stride) != hipSuccess) return fail(MOE_ERR_NOMEM, "zero blob alloc failed");
  HIP_OK(hipMemset(L->d_zero, 0, stride));
  // shared expert
  if (L->fs > 0) {
    std::vector<uint8_t> blob(L->sl.stride, 0);
    pack_matrix(L->sl.gate, D->sh_gate_q, D->sh_gate_s, D->sh_gate_b, blob.data());
    pack_matrix(L->sl.up, D->sh_up_q, D->sh_up_s, D->sh_up_b, blob.data());
    pack_matrix(L->sl.down, D->sh_down_q, D->sh_down_s, D->sh_down_b, blob.data());
    if (dalloc(&L->d_shared, blob.size()) != hipSuccess) return fail(MOE_ERR_NOMEM, "shared expert alloc failed");
    HIP_OK(hipMemcpy(L->d_shared, blob.data(), blob.size(), hipMemcpyHostToDevice));
    dev_bytes += blob.size();
  }
  // router
  if (dalloc(&L->d_router_w, E * L->d) != hipSuccess || dalloc(&L->d_router_scale, E * 2) != hipSuccess)
    return fail(MOE_ERR_NOMEM, "router alloc failed");
  HIP_OK(hipMemcpy(L->d_router_w, D->router_w, E * L->d, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(L->d_router_scale, D->router_scale, E * 2, hipMemcpyHostToDevice));
  dev_bytes += E * L->d + E * 2;
  if (D->router_bias) {
    if (dalloc(&L->d_router_bias, E * 4) != hipSuccess) return fail(MOE_ERR_NOMEM, "router bias alloc failed");
    HIP_OK(hipMemcpy(L->d_router_bias, D->router_bias, E * 4, hipMemcpyHostToDevice));
    dev_bytes += E * 4;
  }
  if (dalloc(&L->d_expert_addr, E * 8) != hipSuccess) return fail(MOE_ERR_NOMEM, "expert table alloc failed");
  HIP_OK(hipMemcpy(L->d_expert_addr, addr.data(), E * 8, hipMemcpyHostToDevice));
  // decode workspace
  const size_t T = L->max_tokens, K = L->K;
  const size_t F = L->fs + K * L->f;
  if (dalloc(&L->d_logits, T * E * 4) != hipSuccess || dalloc(&L->d_ids, T * K * 4) != hipSuccess ||
      dalloc(&L->d_wts, T * K * 4) != hipSuccess || dalloc(&L->d_sel, T * K * 8) != hipSuccess || dalloc(&L->d_counter, decode_sync_bytes(L->E)) != hipSuccess ||
      dalloc(&L->d_abuf, T * F * 4) != hipSuccess || dalloc(&L->d_arep, decode_arep_bytes((int)F)) != hipSuccess ||
      dalloc(&L->d_err, 64) != hipSuccess)
    return fail(MOE_ERR_NOMEM, "decode workspace alloc failed");
  HIP_OK(hipMemset(L->d_ids, 0, T * K * 4));
  HIP_OK(hipMemset(L->d_wts, 0, T * K * 4));
  {  // a valid address in every slot until the first routing
    std::vector<uint64_t> z(T * K, reinterpret_cast<uint64_t>(L->d_zero));
    HIP_OK(hipMemcpy(L->d_sel, z.data(), T * K * 8, hipMemcpyHostToDevice));
  }
  HIP_OK(hipMemset(L->d_counter, 0, decode_sync_bytes(L->E)));
  HIP_OK(hipMemset(L->d_err, 0, 64));
  HIP_OK(hipMemset(L->d_arep, 0, decode_arep_bytes((int)F)));  // parity 0: older than any launch
  // prefill workspace (bf16 only)
  if (L->act == MOE_ACT_BF16 && L->max_tokens > 1) {
    L->prefill_bytes = prefill_workspace_bytes((int)T, L->d, L->E, L->K, L->f, L->fs);
    if (dalloc(&L->d_prefill, L->prefill_bytes) != hipSuccess) return fail(MOE_ERR_NOMEM, "prefill workspace alloc failed");
    HIP_OK(hipMemset(L->d_prefill, 0, L->prefill_bytes));
  }
  L->device_bytes = dev_bytes;
  HIP_OK(hipDeviceSynchronize());
  return MOE_OK;
}

LayerArgs base_args(moe_layer* L, const void* x, void* out, int T) {
  LayerArgs a{};
  a.d = L->d; a.E = L->E; a.K = L->K; a.f = L->f; a.fs = L->fs; a.T = T;
  a.act = L->act;
  a.rms = 0;
  a.eps = 1e-6f;
  a.x = x;
  a.router_w = L->d_router_w;
  a.router_scale = L->d_router_scale;
  a.router_bias = L->d_router_bias;
  a.expert_addr = L->d_expert_addr;
  a.expert_base = L->d_experts;
  a.expert_stride = L->rl.stride;
  a.shared_blob = L->d_shared;
  a.zero_blob = L->d_zero;
  a.ro = L->ro;
  a.so = L->so;
  a.logits = L->d_logits;
  a.ids = L->d_ids;
  a.sel_addr = L->d_sel;
  a.wts = L->d_wts;
  a.counter = L->d_counter;
  a.abuf = L->d_abuf;
  a.arep = L->d_arep;
  a.err = L->d_err;
  a.out = out;
  a.prof = L->prof.get();
  return a;
}

// Place experts ahead of use in L's own cache and copy them on its side
// stream (after `after`, if given: the current layer's demand fills go
// first); L's next call waits for them.  Everything earlier on the stream
// L's calls use must be complete.
moe_status prefetch_impl(moe_layer* L, const int32_t* experts, int n, hipEvent_t after) {
  std::vector<int32_t> want;
  for (int i = 0; i < n; ++i) {
    const int32_t e = experts[i];
    if (e < 0 || e >= L->E) return fail(MOE_ERR_INVALID, "expert %d out of range", e);
    if (!L->fail_expert[e]) want.push_back(e);
  }
  if (want.empty()) return MOE_OK;
  std::vector<int32_t> slot(want.size()), evicted(want.size());
  L->lfu->prefetch(want.data(), (int)want.size(), slot.data(), evicted.data());
  const size_t stride = L->rl.stride;
  bool any = false;
  for (size_t i = 0; i < want.size(); ++i) {
    if (slot[i] < 0) continue;
    if (!any && after) HIP_OK(hipStreamWaitEvent(L->side, after, 0));
    any = true;
    uint8_t* dst = L->d_slots + (size_t)slot[i] * stride;
    HIP_OK(hipMemcpyAsync(dst, L->h_store + (size_t)want[i] * stride, stride, hipMemcpyHostToDevice, L->side));
    if (evicted[i] >= 0) L->h_addr[evicted[i]] = 0;
    L->h_addr[want[i]] = reinterpret_cast<uint64_t>(dst);
    L->addr_dirty = true;
    L->stats.h2d_bytes += stride;
  }
  L->stats.prefetches = L->lfu->prefetches;
  L->stats.evictions = L->lfu->evictions;
  if (any) {
    HIP_OK(hipEventRecord(L->ev_ahead, L->side));
    L->ahead_pending = true;
  }
  return MOE_OK;
}

// Add the last call's fill time to the layer's counters; its events must be
// complete.
void account_fills(moe_layer* L) {
  if (!L->fill_pending) return;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, L->ev_fill_start, L->ev_fill) == hipSuccess) L->stats.h2d_ns += (uint64_t)(ms * 1e6);
  L->fill_pending = false;
}

// Byte offset of the sequence word behind the routing copy in h_ids.
size_t host_flag_offset(const moe_layer* L) { return ((size_t)L->max_tokens * L->K * 4 + 63) / 64 * 64; }

// A one-token call of a streamed layer computes its hits in kernels queued
// before the cache step (the device table marks them); its misses are
// computed after the fill kernel, on the same stream.
struct SlotPlan {
  uint32_t late = 0;  // slots of the missed experts
};

// Spin until the GPU has written `seq` behind the routing in h_ids (at most
// the layer's host_wait_us, 2 s unless a test shortened it); true when it has.
bool wait_host_flag(const moe_layer* L, uint32_t seq) {
  const uint32_t* flag = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(L->h_ids) +
                                                           host_flag_offset(L));
  const auto t0 = std::chrono::steady_clock::now();
  const auto limit = std::chrono::microseconds(L->host_wait_us);
  for (uint32_t i = 1;; ++i) {
    if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == seq) return true;
    if ((i & 4095) == 0 || L->host_wait_us == 0)
      if (std::chrono::steady_clock::now() - t0 >= limit) return false;
    __builtin_ia32_pause();
  }
}

// The prefetch predictor: the `depth` experts the layer's calls chose most
// often (ties to the lower id), among those not in its cache.
std::vector<int32_t> predict_next(const moe_layer* L, int depth) {
  std::vector<int32_t> cand;
  for (int e = 0; e < L->E && !L->hist.empty(); ++e)
    if (L->hist[e] > 0 && L->lfu->find(e) < 0) cand.push_back(e);
  std::sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) {
    return L->hist[a] != L->hist[b] ? L->hist[a] > L->hist[b] : a < b;
  });
  if ((int)cand.size() > depth) cand.resize(depth);
  return cand;
}

// Make every expert chosen by the routing in L->d_ids resident in a slot of
// the layer's cache (its own LFU slots or a shared LRU pool), after the
// router has run on `stream`.  Blocks on the routing copy: once it is back,
// everything queued earlier on `stream` is done, so no slot about to be
// refilled is still being read.  (A one-token call instead spins until the
// routed gate/up's top-K workgroup has published the routing: stream order
// puts every earlier command of the stream behind it, and the call's own
// kernels read only the slots of chosen experts, which the step never
// refills.)
moe_status stream_in(moe_layer* L, int T, hipStream_t stream, moe_layer* next = nullptr, int depth = 0,
                     uint32_t seq = 0, SlotPlan* plan = nullptr, bool ids_known = false) {
  moe_cache_pool* P = L->pool;
  if (!L->lfu && !P) return fail(MOE_ERR_STATE, "streamed layer has no cache: call moe_cache_attach first");
  const size_t n = (size_t)T * L->K;
  if (ids_known) {
    // a one-token call that reuses the previous call's sets: h_ids already
    // holds them (that call waited for them), so the cache step needs
    // nothing from this call's kernels and the host goes on at once; only a
    // fill of the previous call is waited for, to account its time
    if (L->fill_pending) HIP_OK(hipEventSynchronize(L->ev_fill));
  } else if (seq) {  // one token: the top-K kernel writes the ids and then seq into host memory
    if (!wait_host_flag(L, seq)) {  // not within the time limit: the stream's own status decides
      HIP_OK(hipStreamSynchronize(stream));
      if (!wait_host_flag(L, seq)) return fail(MOE_ERR_STATE, "the routing of the call did not reach the host");
    }
  } else {
    HIP_OK(hipMemcpyAsync(L->h_ids, L->d_ids, n * 4, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
  }
  account_fills(L);  // the previous call's (complete by now)
  if (L->ahead_pending) {  // this call may use what was fetched ahead
    HIP_OK(hipStreamWaitEvent(stream, L->ev_ahead, 0));
    L->ahead_pending = false;
  }
  std::vector<int32_t> chosen(L->h_ids, L->h_ids + n);
  std::sort(chosen.begin(), chosen.end());
  chosen.erase(std::unique(chosen.begin(), chosen.end()), chosen.end());
  for (int32_t e : chosen) {
    if (e < 0 || e >= L->E) return fail(MOE_ERR_STATE, "routing produced expert id %d outside 0..%d", e, L->E - 1);
    const bool cached = P ? P->policy->find(L->pool_id, e) >= 0 : L->lfu->find(e) >= 0;
    if (!cached && L->fail_expert[e]) return fail(MOE_ERR_IO, "expert %d could not be read into a cache slot", e);
  }
  const int m = (int)chosen.size();
  const int n_slots = P ? P->n_slots : L->n_slots;
  if (m > n_slots) return fail(MOE_ERR_STATE, "call chose %d distinct experts but the cache has %d slots", m, n_slots);
  std::vector<int32_t> slot(m), miss(m), ev_layer(m, -1), ev_expert(m, -1);
  if (P)
    P->policy->step(L->pool_id, chosen.data(), m, slot.data(), miss.data(), ev_layer.data(), ev_expert.data());
  else
    L->lfu->step(chosen.data(), m, slot.data(), miss.data(), ev_expert.data());
  // One token: slot k holds expert h_ids[k] (chosen[] is those ids sorted,
  // without repeats).  The hits were computed by the kernels queued ahead.
  std::vector<uint32_t> slots_of(m, 0u);
  if (plan) {
    uint32_t hits = 0;
    for (int k = 0; k < L->K; ++k) {
      const int i = (int)(std::lower_bound(chosen.begin(), chosen.end(), L->h_ids[k]) - chosen.begin());
      slots_of[i] |= 1u << k;
      if (!miss[i]) hits |= 1u << k;
    }
    L->stats.ahead_slots += (uint64_t)__builtin_popcount(hits);
    if (P) P->stats.ahead_slots += (uint64_t)__builtin_popcount(hits);
  }
  const size_t stride = L->rl.stride;
  uint8_t* base = P ? P->d_slots : L->d_slots;
  // The misses are filled by copy kernels on `stream` (kMaxFills blobs per
  // launch), which also write the layer's table entries: the expert kernels
  // that follow on the stream see both.
  FillArgs fa{};
  fa.bytes = stride;
  fa.table = L->d_expert_addr;
  bool any = false;
  uint64_t h2d = 0;
  for (int i = 0; i < m; ++i) {
    if (!miss[i]) continue;
    if (!any) HIP_OK(hipEventRecord(L->ev_fill_start, stream));
    any = true;
    uint8_t* dst = base + (size_t)slot[i] * stride;
    moe_layer* owner = nullptr;  // the layer whose entry the fill evicts (another one's, for a pool)
    if (ev_expert[i] >= 0) owner = P ? (ev_layer[i] >= 0 ? P->members[ev_layer[i]] : nullptr) : L;
    if (fa.n == kMaxFills) {
      HIP_OK(launch_fill(fa, stream));
      fa.n = 0;
    }
    fa.src[fa.n] = L->d_store + (size_t)chosen[i] * stride;
    fa.dst[fa.n] = dst;
    fa.expert[fa.n] = chosen[i];
    fa.evicted[fa.n] = owner == L ? ev_expert[i] : -1;
    ++fa.n;
    if (plan) plan->late |= slots_of[i];
    if (owner) {  // the kernel clears this layer's entry; another layer re-uploads its table on its next call
      owner->h_addr[ev_expert[i]] = 0;
      if (owner != L) owner->addr_dirty = true;
    }
    L->h_addr[chosen[i]] = reinterpret_cast<uint64_t>(dst);
    h2d += stride;
  }
  if (P) {  // this layer's share of the pool's counts
    int nm = 0, ne = 0;
    for (int i = 0; i < m; ++i) {
      nm += miss[i] ? 1 : 0;
      ne += (miss[i] && ev_expert[i] >= 0) ? 1 : 0;
    }
    L->stats.accesses += m;
    L->stats.hits += m - nm;
    L->stats.misses += nm;
    L->stats.evictions += ne;
    P->stats.accesses = P->policy->accesses;
    P->stats.hits = P->policy->hits;
    P->stats.misses = P->policy->misses;
    P->stats.evictions = P->policy->evictions;
    P->stats.h2d_bytes += h2d;
  } else {
    L->stats.accesses = L->lfu->accesses;
    L->stats.hits = L->lfu->hits;
    L->stats.misses = L->lfu->misses;
    L->stats.evictions = L->lfu->evictions;
    L->stats.prefetch_used = L->lfu->prefetch_used;
  }
  L->stats.h2d_bytes += h2d;
  if (L->hist.empty()) L->hist.assign(L->E, 0);
  for (int32_t e : chosen) ++L->hist[e];
  if (any) {
    HIP_OK(launch_fill(fa, stream));
    HIP_OK(hipEventRecord(L->ev_fill, stream));
    L->fill_pending = true;
  }
  if (next && depth > 0 && next->lfu) {  // fetch ahead for the next layer, behind this layer's fills
    const std::vector<int32_t> guess = predict_next(next, depth);
    moe_status st = prefetch_impl(next, guess.data(), (int)guess.size(), any ? L->ev_fill : nullptr);
    if (st != MOE_OK) return st;
  }
  // The routed kernel reads each chosen expert's address from the device
  // table; the fill kernels wrote this call's entries, so the table goes up
  // only when a fetch-ahead or another layer's eviction changed it (the
  // stream was synchronised above, so no earlier upload of h_addr is still
  // pending).
  if (L->addr_dirty && !plan) {
    HIP_OK(hipMemcpyAsync(L->d_expert_addr, L->h_addr, (size_t)L->E * 8, hipMemcpyHostToDevice, stream));
    L->addr_dirty = false;
  }
  return MOE_OK;
}

moe_status forward_impl(moe_layer* L, LayerArgs a, const moe_fwd_opts* o, hipStream_t s, moe_layer* next = nullptr,
                        int depth = 0) {
  const int T = a.T;
  if (T == 0) return MOE_OK;
  if (T < 0 || T > L->max_tokens) return fail(MOE_ERR_INVALID, "n_tokens=%d not in 0..%d", T, L->max_tokens);
  HIP_OK(hipSetDevice(L->dev));
  const bool h_ids_last = L->h_ids_last;  // set again below when this call leaves its routing in h_ids
  L->h_ids_last = false;
  if (o) {
    a.ids_out = o->topk_ids;
    a.w_out = o->topk_w;
    a.forced = o->forced_ids;
    if (o->reuse_previous) {
      if (o->forced_ids) return fail(MOE_ERR_INVALID, "forced_ids and reuse_previous are exclusive");
      if (L->prev_T != T) return fail(MOE_ERR_STATE, "reuse_previous needs a previous call with the same n_tokens");
      a.forced = L->d_ids;
    }
    if (o->residual) {
      if (!o->residual_src) return fail(MOE_ERR_INVALID, "residual requested without residual_src");
      a.resid = o->residual_src;
    }
  }
  int path = o ? o->path : MOE_PATH_AUTO;
  if (path == MOE_PATH_AUTO) path = L->default_path;
  const bool resident = L->residency == MOE_RESIDENT;
  if (L->fused_ok < 0) {  // shape, LDS and residency check, once per layer
    LayerArgs one = a;
    one.T = 1;
    L->fused_ok = resident && decode_fused_ok(one) ? 1 : 0;
  }
  const bool fused_ok = L->fused_ok == 1 && T == 1;
  if (path == MOE_PATH_AUTO) {
    if (fused_ok)
      path = MOE_PATH_FUSED;
    else if (L->act == MOE_ACT_BF16 && T >= 16 && L->d_prefill && L->d <= 4096 && (resident || L->lfu) && !a.rms)
      path = MOE_PATH_PREFILL;
    else
      path = MOE_PATH_DECODE;
  }
  if (path == MOE_PATH_FUSED) {
    if (!fused_ok)
      return fail(MOE_ERR_INVALID,
                  "the fused path serves one bf16 token on resident experts, d_model <= 4096, within 64 KB "
                  "of LDS");
    a.fused = 1;
    HIP_OK(launch_decode(a, s));
    L->prev_T = T;
    return MOE_OK;
  }
  if (path == MOE_PATH_PREFILL) {
    if (L->act != MOE_ACT_BF16 || !L->d_prefill)
      return fail(MOE_ERR_INVALID, "the prefill path needs bf16 activations and max_tokens > 1");
    if (L->residency == MOE_STREAMED && !L->lfu)
      return fail(MOE_ERR_INVALID, "prefill of a streamed layer needs its own LFU cache (moe_cache_attach)");
    if (L->d > 4096) return fail(MOE_ERR_INVALID, "the prefill path supports d_model <= 4096");
    if (a.rms) return fail(MOE_ERR_INVALID, "the prefill path takes the layer input directly (no rmsnorm)");
    moe_status st = launch_prefill_path(L, a, o, s);
    if (st == MOE_OK) L->prev_T = T;
    return st;
  }
  if (path != MOE_PATH_DECODE) return fail(MOE_ERR_INVALID, "unknown path %d", path);
  if (L->residency == MOE_STREAMED) {
    LayerArgs a1 = a;
    a1.stages = kStageRouter | kStageShared;
    LayerArgs a2 = a;
    a2.stages = kStageRouted | kStageDown;
    a2.sel_from_table = 1;
    // One token: three launches are queued at once, before the cache step:
    // the router; the routed gate/up, whose first workgroup runs the top-K and
    // hands the routing to the host through host memory, with the shared
    // expert's gate/up in the same launch; the down kernel.  The device table
    // holds exactly the cache's contents (it is brought up to date first), so
    // those kernels compute the hits without waiting for the host.  The host
    // launches each miss behind its own fill and the down kernel again after
    // the last; with no miss it launches nothing more.
    const bool one = T == 1 && L->d_host_ids && L->K <= 32;
    uint32_t seq = 0;
    bool uploaded = false;  // the device table goes up from h_addr in this call
    if (one) {
      seq = ++L->host_seq;
      if (seq >= (1u << 30)) seq = L->host_seq = 1;  // 0 means "no flag"
      a1.stages = kStageRouter;
      a1.topk_in_gate_up = 1;  // no top-K kernel after the router
      if (L->addr_dirty) {  // a fetch-ahead or another layer's eviction changed it since the last upload
        HIP_OK(hipMemcpyAsync(L->d_expert_addr, L->h_addr, (size_t)L->E * 8, hipMemcpyHostToDevice, s));
        L->addr_dirty = false;
        uploaded = true;
      }
    }
    HIP_OK(launch_decode(a1, s));
    if (one) {
      if (L->ahead_pending) {  // fetched-ahead copies land before the expert kernels read their slots
        HIP_OK(hipStreamWaitEvent(s, L->ev_ahead, 0));
        L->ahead_pending = false;
      }
      LayerArgs a3 = a2;
      a3.hits_only = 1;
      a3.shared_in_routed = 1;
      a3.topk_in_gate_up = 1;
      a3.host_ids = static_cast<int32_t*>(L->d_host_ids);
      a3.host_flag = reinterpret_cast<uint32_t*>(static_cast<char*>(L->d_host_ids) + host_flag_offset(L));
      a3.host_seq = seq;
      HIP_OK(launch_decode(a3, s));
    }
    SlotPlan plan;
    // The host may skip the wait for the routing only when it needs nothing
    // from this call's kernels: the sets are reused and known, and no upload
    // of h_addr is in flight (the copy reads host memory when it runs, and
    // the cache step is about to change it).
    const bool known = one && o && o->reuse_previous && h_ids_last && !uploaded;
    moe_status st = stream_in(L, T, s, next, depth, seq, one ? &plan : nullptr, known);
    if (st != MOE_OK) return st;
    L->h_ids_last = one;
    if (!one) {
      HIP_OK(launch_decode(a2, s));
    } else if (plan.late) {  // behind the fill kernel on the stream
      a2.stages = kStageRouted;
      a2.run_mask = plan.late;
      HIP_OK(launch_decode(a2, s));
      a2.stages = kStageDown;
      a2.run_mask = 0;
      HIP_OK(launch_decode(a2, s));
    }
  } else {
    a.topk_in_gate_up = 1;
    HIP_OK(launch_decode(a, s));
  }
  L->prev_T = T;
  return MOE_OK;
}

}  // namespace

// Prefill through the streamed layer's LFU cache (Rockchip-NPU plan §2.5:
// the prefill chunk fetches each chosen expert once for all its rows).  The
// chunk's distinct experts go through the cache in groups of at most n_slots:
// first those already cached (ascending id: hits, used before anything can
// evict them), then the rest least chosen first (ties: lower id), so that
// the cache ends up holding the chunk's most chosen experts.  Each group is
// one cache step (its ids ascending).  A group's fills wait for the previous
// group's GEMMs, whose slots they may reuse.
struct StreamPrefill final : PrefillStreamer {
  moe_layer* L;
  moe_status err = MOE_OK;
  std::vector<std::vector<int32_t>> groups;
  std::vector<size_t> list_at;  // each group's tile list, in ints from d_pf_tiles
  explicit StreamPrefill(moe_layer* l) : L(l) {}

  hipError_t plan(const PrefillArgs& p, int C, hipStream_t s, int* n_groups) override {
    hipError_t e = hipMemcpyAsync(L->h_pf, p.counts, (size_t)L->E * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    if (L->ahead_pending) {  // fetched-ahead copies land before anything reads their slots
      if ((e = hipStreamWaitEvent(s, L->ev_ahead, 0)) != hipSuccess) return e;
      L->ahead_pending = false;
    }
    std::vector<int32_t> order, rest;
    for (int x = 0; x < L->E; ++x)
      if (L->h_pf[x] > 0) (L->lfu->find(x) >= 0 ? order : rest).push_back(x);
    std::stable_sort(rest.begin(), rest.end(), [&](int32_t u, int32_t v) { return L->h_pf[u] < L->h_pf[v]; });
    order.insert(order.end(), rest.begin(), rest.end());
    const int n_slots = L->n_slots;
    groups.clear();
    for (size_t i = 0; i < order.size(); i += n_slots) {
      std::vector<int32_t> g(order.begin() + i, order.begin() + std::min(order.size(), i + n_slots));
      std::sort(g.begin(), g.end());
      groups.push_back(g);
    }
    if (groups.empty()) groups.emplace_back();  // no routed expert: the shared expert still runs
    // tile lists: [n, (expert, tile) x n]; the shared expert's tiles go with group 0
    const int shared_tiles = L->fs > 0 ? (C + 15) / 16 : 0;
    size_t need = groups.size() + 2 * (size_t)shared_tiles;
    for (const auto& g : groups)
      for (int32_t x : g) need += 2 * (size_t)((L->h_pf[x] + 15) / 16);
    if (need > L->pf_ints) return hipErrorInvalidValue;  // cannot happen: sized for the worst case
    int32_t* h = L->h_pf + L->E;
    size_t at = 0;
    list_at.clear();
    for (size_t g = 0; g < groups.size(); ++g) {
      list_at.push_back(at);
      const size_t head = at++;
      int n = 0;
      for (int32_t x : groups[g])
        for (int tt = 0; tt * 16 < L->h_pf[x]; ++tt, ++n) {
          h[at++] = x;
          h[at++] = tt;
        }
      if (g == 0)
        for (int tt = 0; tt < shared_tiles; ++tt, ++n) {
          h[at++] = L->E;
          h[at++] = tt;
        }
      h[head] = n;
    }
    if ((e = hipMemcpyAsync(L->d_pf_tiles, h, at * 4, hipMemcpyHostToDevice, s)) != hipSuccess) return e;
    *n_groups = (int)groups.size();
    return hipSuccess;
  }

  hipError_t group(int gi, hipStream_t s, int32_t** tiles) override {
    const std::vector<int32_t>& chosen = groups[gi];
    const int m = (int)chosen.size();
    for (int32_t x : chosen)
      if (!(L->lfu->find(x) >= 0) && L->fail_expert[x]) {
        err = fail(MOE_ERR_IO, "expert %d could not be read into a cache slot", x);
        return hipErrorUnknown;
      }
    std::vector<int32_t> slot(m), miss(m), ev_expert(m, -1);
    if (m > 0) L->lfu->step(chosen.data(), m, slot.data(), miss.data(), ev_expert.data());
    const size_t stride = L->rl.stride;
    // Fill kernels on the chunk's stream (after the previous group's GEMMs,
    // whose slots they may reuse); they also write the table entries.
    FillArgs fa{};
    fa.bytes = stride;
    fa.table = L->d_expert_addr;
    hipError_t e = hipSuccess;
    for (int i = 0; i < m; ++i) {
      if (!miss[i]) continue;
      if (fa.n == kMaxFills) {
        if ((e = launch_fill(fa, s)) != hipSuccess) return e;
        fa.n = 0;
      }
      uint8_t* dst = L->d_slots + (size_t)slot[i] * stride;
      fa.src[fa.n] = L->d_store + (size_t)chosen[i] * stride;
      fa.dst[fa.n] = dst;
      fa.expert[fa.n] = chosen[i];
      fa.evicted[fa.n] = ev_expert[i];
      ++fa.n;
      if (ev_expert[i] >= 0) L->h_addr[ev_expert[i]] = 0;
      L->h_addr[chosen[i]] = reinterpret_cast<uint64_t>(dst);
      L->stats.h2d_bytes += stride;
    }
    if ((e = launch_fill(fa, s)) != hipSuccess) return e;
    L->stats.accesses = L->lfu->accesses;
    L->stats.hits = L->lfu->hits;
    L->stats.misses = L->lfu->misses;
    L->stats.evictions = L->lfu->evictions;
    L->stats.prefetch_used = L->lfu->prefetch_used;
    if (L->hist.empty()) L->hist.assign(L->E, 0);
    for (int32_t x : chosen) ++L->hist[x];
    if (L->addr_dirty) {  // a fetch-ahead changed it before this chunk
      // from a snapshot of its own: the host takes the next group's step
      // (and changes h_addr) before this copy runs
      if ((size_t)gi >= L->pf_groups) return hipErrorInvalidValue;  // cannot happen: sized for every group
      uint64_t* snap = L->h_pf_addr + (size_t)gi * L->E;
      std::memcpy(snap, L->h_addr, (size_t)L->E * 8);
      e = hipMemcpyAsync(L->d_expert_addr, snap, (size_t)L->E * 8, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return e;
      L->addr_dirty = false;
    }
    *tiles = L->d_pf_tiles + list_at[gi];
    return hipSuccess;
  }

  hipError_t done(int, hipStream_t) override { return hipSuccess; }
};

moe_status launch_prefill_path(moe_layer* L, const LayerArgs& a, const moe_fwd_opts* o, hipStream_t s) {
  PrefillArgs p{};
  p.L = a;
  prefill_carve(p, L->d_prefill, L->max_tokens, L->d, L->E, L->K, L->f, L->fs);  // the layout of every call
  p.sort_offsets_out = o ? o->sort_offsets : nullptr;
  p.sort_perm_out = o ? o->sort_perm : nullptr;
  if (L->residency != MOE_STREAMED) {
    HIP_OK(launch_prefill(p, s));
    return MOE_OK;
  }
  if (!L->lfu) return fail(MOE_ERR_INVALID, "prefill of a streamed layer needs its own LFU cache (moe_cache_attach)");
  if (!L->h_pf) {
    const int C = std::min(L->max_tokens, 128);
    L->pf_ints = (size_t)C * L->K * 2 + (size_t)L->E * 3 + (size_t)(C + 15) / 16 * 2 + 64;
    if (hipHostMalloc(reinterpret_cast<void**>(&L->h_pf), ((size_t)L->E + L->pf_ints) * 4, hipHostMallocDefault) !=
        hipSuccess)
      return fail(MOE_ERR_NOMEM, "pinned prefill lists failed");
    if (dalloc(&L->d_pf_tiles, L->pf_ints * 4) != hipSuccess) return fail(MOE_ERR_NOMEM, "prefill list alloc failed");
    L->pf_groups = (size_t)(L->E + L->n_slots - 1) / L->n_slots + 1;
    if (hipHostMalloc(reinterpret_cast<void**>(&L->h_pf_addr), L->pf_groups * L->E * 8, hipHostMallocDefault) !=
        hipSuccess)
      return fail(MOE_ERR_NOMEM, "pinned table snapshots failed");
  }
  StreamPrefill sp(L);
  p.streamer = &sp;
  const hipError_t e = launch_prefill(p, s);
  if (sp.err != MOE_OK) return sp.err;
  HIP_OK(e);
  return MOE_OK;
}

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_layer_create(const moe_layer_desc* desc, moe_layer** out) {
  if (!out) return fail(MOE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  moe_status st = validate(desc);
  if (st != MOE_OK) return st;
  moe_layer* L = new (std::nothrow) moe_layer();
  if (!L) return fail(MOE_ERR_NOMEM, "host allocation failed");
  st = create_impl(desc, L);
  if (st != MOE_OK) {
    std::string keep = g_err;
    free_layer(L);
    g_err = keep;
    return st;
  }
  *out = L;
  return MOE_OK;
}

moe_status moe_layer_destroy(moe_layer* layer) {
  free_layer(layer);
  return MOE_OK;
}

moe_status moe_layer_forward_ex(const void* x, moe_layer* L, void* out, int32_t n_tokens, const moe_fwd_opts* o,
                                void* stream) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (n_tokens > 0 && (!x || !out)) return fail(MOE_ERR_INVALID, "x/out is NULL");
  if (x == out && n_tokens > 0) return fail(MOE_ERR_INVALID, "x and out may not alias");
  LayerArgs a = base_args(L, x, out, n_tokens);
  return forward_impl(L, a, o, static_cast<hipStream_t>(stream));
}

moe_status moe_layer_forward(const void* x, moe_layer* L, void* out, int32_t n_tokens, void* stream) {
  return moe_layer_forward_ex(x, L, out, n_tokens, nullptr, stream);
}

// Bytes of the allocation-free forward's workspace for T tokens: logits,
// ids, coefficients, chosen blob addresses and the activation vectors.
static size_t noalloc_bytes(const moe_layer* L, size_t T) {
  const size_t K = L->K, F = (size_t)L->fs + K * L->f;
  return align256(T * L->E * 4) + 2 * align256(T * K * 4) + align256(T * K * 8) +
         align256(T * F * (L->act == MOE_ACT_BF16 ? 2 : 4));
}

moe_status moe_layer_forward_noalloc(const void* x, moe_layer* L, void* out, int32_t n_tokens, void* stream) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (n_tokens == 0) return MOE_OK;
  if (n_tokens < 0 || n_tokens > L->max_tokens)
    return fail(MOE_ERR_INVALID, "n_tokens=%d not in 0..%d", n_tokens, L->max_tokens);
  if (!x || !out) return fail(MOE_ERR_INVALID, "x/out is NULL");
  if (x == out) return fail(MOE_ERR_INVALID, "x and out may not alias");
  if (L->residency != MOE_RESIDENT) return fail(MOE_ERR_INVALID, "the allocation-free forward serves resident layers");
  const size_t need = noalloc_bytes(L, (size_t)n_tokens);
  if (need > kNoAllocScratchBytes)
    return fail(MOE_ERR_INVALID, "%d tokens need %zu bytes of workspace; the allocation-free forward has %zu", n_tokens,
                need, kNoAllocScratchBytes);
  HIP_OK(hipSetDevice(L->dev));
  void* base = nullptr;
  HIP_OK(noalloc_scratch(&base));
  LayerArgs a = base_args(L, x, out, n_tokens);
  const size_t T = (size_t)n_tokens, K = L->K;
  char* p = static_cast<char*>(base);
  a.logits = reinterpret_cast<float*>(p);
  p += align256(T * L->E * 4);
  a.ids = reinterpret_cast<int32_t*>(p);
  p += align256(T * K * 4);
  a.wts = reinterpret_cast<float*>(p);
  p += align256(T * K * 4);
  a.sel_addr = reinterpret_cast<uint64_t*>(p);
  p += align256(T * K * 8);
  a.abuf = p;
  a.counter = nullptr;  // the three-kernel path uses neither the fused kernel's counters ...
  a.arep = nullptr;     // ... nor its copies
  a.topk_in_gate_up = 1;
  HIP_OK(launch_decode(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_route(const void* x, moe_layer* L, int32_t* ids, float* w, int32_t n_tokens, void* stream) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (n_tokens == 0) return MOE_OK;
  if (n_tokens < 0 || n_tokens > L->max_tokens)
    return fail(MOE_ERR_INVALID, "n_tokens=%d not in 0..%d", n_tokens, L->max_tokens);
  if (!x || !ids || !w) return fail(MOE_ERR_INVALID, "x/ids/w is NULL");
  HIP_OK(hipSetDevice(L->dev));
  LayerArgs a = base_args(L, x, nullptr, n_tokens);
  a.stages = kStageRouter;
  a.ids_out = ids;
  a.w_out = w;
  L->h_ids_last = false;  // the layer's stored sets become these
  HIP_OK(launch_decode(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_sort(const int32_t* ids, moe_layer* L, int32_t n_tokens, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, void* stream) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (n_tokens < 0 || n_tokens > L->max_tokens)
    return fail(MOE_ERR_INVALID, "n_tokens=%d not in 0..%d", n_tokens, L->max_tokens);
  if (!counts || !offsets || (n_tokens > 0 && (!ids || !perm || !inv)))
    return fail(MOE_ERR_INVALID, "a sort buffer is NULL");
  HIP_OK(hipSetDevice(L->dev));
  if (((size_t)L->E + 1 + (size_t)L->E * ((n_tokens + 31) / 32)) * 4 > 144 * 1024)
    return fail(MOE_ERR_INVALID, "grouping %d tokens over %d experts needs more than 144 KB of LDS", n_tokens, L->E);
  HIP_OK(launch_sort(ids, n_tokens, L->K, L->E, counts, offsets, perm, inv, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_bytes(const moe_layer* L, uint64_t* device_bytes, uint64_t* expert_bytes) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (device_bytes) *device_bytes = L->device_bytes;
  if (expert_bytes) *expert_bytes = L->rl.stride;
  return MOE_OK;
}

moe_status moe_layer_set_default_path(moe_layer* L, int32_t path) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (path < MOE_PATH_AUTO || path > MOE_PATH_FUSED) return fail(MOE_ERR_INVALID, "unknown path %d", path);
  L->default_path = path;
  return MOE_OK;
}

moe_status moe_layer_check_errors(moe_layer* L, int32_t* flags) {
  if (!L || !flags) return fail(MOE_ERR_INVALID, "layer/flags is NULL");
  HIP_OK(hipSetDevice(L->dev));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(flags, L->d_err, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemset(L->d_err, 0, 4));
  return MOE_OK;
}

moe_status moe_debug_dequant(const moe_layer* L, int32_t which, int32_t expert, float* host_out) {
  if (!L || !host_out) return fail(MOE_ERR_INVALID, "layer/host_out is NULL");
  if (which < 0 || which > 2) return fail(MOE_ERR_INVALID, "which=%d not in 0..2 (gate, up, down)", which);
  if (expert < -1 || expert >= L->E) return fail(MOE_ERR_INVALID, "expert %d not in -1..%d", expert, L->E - 1);
  if (expert == -1 && L->fs == 0) return fail(MOE_ERR_INVALID, "the layer has no shared expert");
  HIP_OK(hipSetDevice(L->dev));
  const BlobLayout& B = expert < 0 ? L->sl : L->rl;
  const MatLayout& m = which == 0 ? B.gate : which == 1 ? B.up : B.down;
  const uint8_t* blob = nullptr;
  uint8_t* tmp = nullptr;  // a streamed expert's blob, copied from the pinned store
  if (expert < 0) {
    blob = L->d_shared;
  } else if (L->residency == MOE_RESIDENT) {
    blob = L->d_experts + (size_t)expert * L->rl.stride;
  } else {
    if (dalloc(&tmp, L->rl.stride) != hipSuccess) return fail(MOE_ERR_NOMEM, "blob copy alloc failed");
    blob = tmp;
  }
  float* d_out = nullptr;
  const size_t n = (size_t)m.rows * m.cols;
  if (dalloc(&d_out, n * 4) != hipSuccess) {
    (void)hipFree(tmp);
    return fail(MOE_ERR_NOMEM, "dequant output alloc failed");
  }
  hipError_t e = hipSuccess;
  if (tmp) e = hipMemcpy(tmp, L->h_store + (size_t)expert * L->rl.stride, L->rl.stride, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = launch_dequant(blob, (uint32_t)m.q_off, (uint32_t)m.sb_off, m.rows, m.cols, d_out, nullptr);
  if (e == hipSuccess) e = hipMemcpy(host_out, d_out, n * 4, hipMemcpyDeviceToHost);
  (void)hipFree(d_out);
  (void)hipFree(tmp);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "dequant failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_debug_host_wait(moe_layer* L, int64_t microseconds) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (microseconds < 0) return fail(MOE_ERR_INVALID, "microseconds=%lld is negative", (long long)microseconds);
  L->host_wait_us = microseconds;
  return MOE_OK;
}

moe_status moe_layer_profile(moe_layer* L, int32_t enable) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (enable && !L->prof) L->prof.reset(new EventProfiler());
  if (!enable) {
    if (L->prof) (void)hipDeviceSynchronize();
    L->prof.reset();
  }
  return MOE_OK;
}

moe_status moe_layer_profile_read(moe_layer* L, int64_t* launches, double* total_ms) {
  if (!L || !launches || !total_ms) return fail(MOE_ERR_INVALID, "NULL argument");
  for (int k = 0; k < MOE_N_KERNELS; ++k) {
    launches[k] = 0;
    total_ms[k] = 0.0;
  }
  if (!L->prof) return MOE_OK;
  EventProfiler* P = L->prof.get();
  if (P->err != hipSuccess) return fail(MOE_ERR_HIP, "profiling event failed: %s", hipGetErrorString(P->err));
  HIP_OK(hipSetDevice(L->dev));
  HIP_OK(hipDeviceSynchronize());
  for (auto& r : P->recs) {
    float ms = 0.f;
    HIP_OK(hipEventElapsedTime(&ms, r.a, r.b));
    if (r.kernel >= 0 && r.kernel < MOE_N_KERNELS) {
      launches[r.kernel] += 1;
      total_ms[r.kernel] += ms;
    }
    P->pool.push_back(r.a);
    P->pool.push_back(r.b);
  }
  P->recs.clear();
  return MOE_OK;
}

// ---- cache ----
namespace {
// Routing copy and fill events of a streamed layer that gets a cache.
moe_status cache_common(moe_layer* L) {
  if (!L->h_ids) {  // coherent, so the top-K kernel can write a one-token routing straight into it
    const size_t bytes = host_flag_offset(L) + 64;  // + the sequence word
    if (hipHostMalloc(reinterpret_cast<void**>(&L->h_ids), bytes, hipHostMallocCoherent | hipHostMallocMapped) !=
        hipSuccess)
      return fail(MOE_ERR_NOMEM, "pinned routing buffer failed");
    std::memset(L->h_ids, 0, bytes);
    HIP_OK(hipHostGetDevicePointer(&L->d_host_ids, L->h_ids, 0));
  }
  if (!L->ev_fill) HIP_OK(hipEventCreate(&L->ev_fill));
  if (!L->ev_fill_start) HIP_OK(hipEventCreate(&L->ev_fill_start));
  if (!L->ev_ahead) HIP_OK(hipEventCreate(&L->ev_ahead));
  return MOE_OK;
}
// Forget where the layer's experts were (every entry absent).
moe_status clear_addresses(moe_layer* L) {
  std::memset(L->h_addr, 0, (size_t)L->E * 8);
  HIP_OK(hipMemcpy(L->d_expert_addr, L->h_addr, (size_t)L->E * 8, hipMemcpyHostToDevice));
  L->addr_dirty = false;
  return MOE_OK;
}
}  // namespace

moe_status moe_cache_attach(moe_layer* L, int32_t n_slots, void* side_stream) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (L->residency != MOE_STREAMED) return fail(MOE_ERR_STATE, "layer is not MOE_STREAMED");
  if (L->lfu || L->pool) return fail(MOE_ERR_STATE, "layer already has a cache");
  if (n_slots < L->K || n_slots > L->E) return fail(MOE_ERR_INVALID, "n_slots=%d not in top_k..n_experts", n_slots);
  HIP_OK(hipSetDevice(L->dev));
  const size_t bytes = (size_t)n_slots * L->rl.stride;
  if (dalloc(&L->d_slots, bytes) != hipSuccess) return fail(MOE_ERR_NOMEM, "slot pool of %zu bytes failed", bytes);
  moe_status st = cache_common(L);
  if (st != MOE_OK) return st;
  if (side_stream) {
    L->side = static_cast<hipStream_t>(side_stream);
  } else {
    HIP_OK(hipStreamCreateWithFlags(&L->side, hipStreamNonBlocking));
    L->own_side = true;
  }
  L->n_slots = n_slots;
  L->lfu.reset(new LfuPolicy(n_slots));
  L->device_bytes += bytes;
  return MOE_OK;
}

moe_status moe_cache_pool_create(uint64_t budget_bytes, uint64_t expert_bytes, void* side_stream,
                                 moe_cache_pool** out) {
  if (!out) return fail(MOE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (expert_bytes == 0 || budget_bytes < expert_bytes || budget_bytes / expert_bytes > (1u << 20))
    return fail(MOE_ERR_INVALID, "budget %llu B holds no expert of %llu B (or more than 2^20)",
                (unsigned long long)budget_bytes, (unsigned long long)expert_bytes);
  std::unique_ptr<moe_cache_pool> P(new (std::nothrow) moe_cache_pool());
  if (!P) return fail(MOE_ERR_NOMEM, "host allocation failed");
  HIP_OK(hipGetDevice(&P->dev));
  P->expert_bytes = expert_bytes;
  P->n_slots = (int)(budget_bytes / expert_bytes);
  if (dalloc(&P->d_slots, (size_t)P->n_slots * expert_bytes) != hipSuccess)
    return fail(MOE_ERR_NOMEM, "slot pool of %llu bytes failed", (unsigned long long)budget_bytes);
  (void)side_stream;  // fills run on the calls' streams; the pool fetches nothing ahead
  P->policy.reset(new LruPool(P->n_slots));
  *out = P.release();
  return MOE_OK;
}

moe_status moe_cache_pool_destroy(moe_cache_pool* P) {
  if (!P) return MOE_OK;
  (void)hipSetDevice(P->dev);
  (void)hipDeviceSynchronize();
  for (moe_layer* L : P->members)
    if (L) {  // the layer keeps running only after a new cache is attached
      L->pool = nullptr;
      L->pool_id = -1;
      (void)clear_addresses(L);
    }
  (void)hipFree(P->d_slots);
  delete P;
  return MOE_OK;
}

moe_status moe_cache_attach_pool(moe_layer* L, moe_cache_pool* P) {
  if (!L || !P) return fail(MOE_ERR_INVALID, "layer/pool is NULL");
  if (L->residency != MOE_STREAMED) return fail(MOE_ERR_STATE, "layer is not MOE_STREAMED");
  if (L->lfu || L->pool) return fail(MOE_ERR_STATE, "layer already has a cache");
  if (L->dev != P->dev) return fail(MOE_ERR_INVALID, "layer and pool are on different devices");
  if (L->rl.stride != P->expert_bytes)
    return fail(MOE_ERR_INVALID, "expert blob of %zu B, the pool's slots hold %llu B", L->rl.stride,
                (unsigned long long)P->expert_bytes);
  if (P->n_slots < L->K * L->max_tokens && P->n_slots < L->E)
    return fail(MOE_ERR_INVALID, "pool of %d slots cannot hold one call's %d experts", P->n_slots,
                std::min(L->K * L->max_tokens, L->E));
  HIP_OK(hipSetDevice(L->dev));
  moe_status st = cache_common(L);
  if (st != MOE_OK) return st;
  L->pool = P;
  L->pool_id = (int)P->members.size();
  P->members.push_back(L);
  return MOE_OK;
}

moe_status moe_cache_detach(moe_layer* L) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (!L->lfu && !L->pool) return fail(MOE_ERR_STATE, "layer has no cache");
  HIP_OK(hipSetDevice(L->dev));
  HIP_OK(hipDeviceSynchronize());
  if (L->pool) {
    leave_pool(L);
  } else {
    (void)hipFree(L->d_slots);
    L->device_bytes -= (uint64_t)L->n_slots * L->rl.stride;
    L->d_slots = nullptr;
    L->n_slots = 0;
    L->lfu.reset();
    if (L->own_side && L->side) (void)hipStreamDestroy(L->side);
    L->side = nullptr;
    L->own_side = false;
  }
  L->fill_pending = false;
  L->ahead_pending = false;
  L->stats = moe_cache_stats{};
  L->hist.clear();
  return clear_addresses(L);
}

moe_status moe_cache_prefetch(moe_layer* L, const int32_t* experts, int32_t n, void* stream) {
  if (!L || (n > 0 && !experts)) return fail(MOE_ERR_INVALID, "NULL argument");
  if (!L->lfu) return fail(MOE_ERR_STATE, "prefetch needs the layer's own cache (moe_cache_attach)");
  if (n < 0 || n > L->n_slots) return fail(MOE_ERR_INVALID, "n=%d not in 0..%d", n, L->n_slots);
  HIP_OK(hipSetDevice(L->dev));
  HIP_OK(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  return prefetch_impl(L, experts, n, nullptr);
}

moe_status moe_cache_pool_stats(const moe_cache_pool* P, moe_cache_stats* out) {
  if (!P || !out) return fail(MOE_ERR_INVALID, "pool/out is NULL");
  HIP_OK(hipSetDevice(P->dev));
  HIP_OK(hipDeviceSynchronize());
  moe_cache_stats st = P->stats;
  st.h2d_ns = 0;
  for (moe_layer* L : P->members) {
    if (!L) continue;
    moe_cache_stats ls{};
    moe_status r = moe_cache_stats_get(L, &ls);
    if (r != MOE_OK) return r;
    st.h2d_ns += ls.h2d_ns;
  }
  *out = st;
  return MOE_OK;
}

moe_status moe_cache_pool_contents(const moe_cache_pool* P, int32_t* layer_of_slot, int32_t* expert_of_slot) {
  if (!P) return fail(MOE_ERR_INVALID, "pool is NULL");
  for (int s = 0; s < P->n_slots; ++s) {
    if (layer_of_slot) layer_of_slot[s] = P->policy->slots[s].layer;
    if (expert_of_slot) expert_of_slot[s] = P->policy->slots[s].expert;
  }
  return MOE_OK;
}

moe_status moe_cache_stats_get(const moe_layer* L, moe_cache_stats* out) {
  if (!L || !out) return fail(MOE_ERR_INVALID, "layer/out is NULL");
  moe_layer* M = const_cast<moe_layer*>(L);
  if (M->fill_pending) {
    HIP_OK(hipEventSynchronize(M->ev_fill));
    account_fills(M);
  }
  *out = L->stats;
  return MOE_OK;
}

moe_status moe_cache_reset(moe_layer* L, int32_t drop_contents) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (!L->lfu && !L->pool) return fail(MOE_ERR_STATE, "layer has no cache");
  HIP_OK(hipSetDevice(L->dev));
  HIP_OK(hipDeviceSynchronize());
  L->fill_pending = false;
  L->stats = moe_cache_stats{};
  if (L->lfu) L->lfu->clear_counters();
  if (drop_contents) {
    if (L->lfu)
      L->lfu->clear_contents();
    else
      L->pool->policy->drop_layer(L->pool_id);
    return clear_addresses(L);
  }
  return MOE_OK;
}

moe_status moe_cache_contents(const moe_layer* L, int32_t* expert_of_slot, uint32_t* use_count) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (!L->lfu) return fail(MOE_ERR_STATE, L->pool ? "layer uses a shared pool: see moe_cache_pool_contents"
                                                  : "layer has no cache");
  for (int s = 0; s < L->n_slots; ++s) {
    if (expert_of_slot) expert_of_slot[s] = L->lfu->slots[s].expert;
    if (use_count) use_count[s] = L->lfu->slots[s].count;
  }
  return MOE_OK;
}

moe_status moe_cache_fail_expert(moe_layer* L, int32_t expert, int32_t failflag) {
  if (!L) return fail(MOE_ERR_INVALID, "layer is NULL");
  if (L->residency != MOE_STREAMED) return fail(MOE_ERR_STATE, "layer is not MOE_STREAMED");
  if (expert < 0 || expert >= L->E) return fail(MOE_ERR_INVALID, "expert %d out of range", expert);
  L->fail_expert[expert] = failflag ? 1 : 0;
  return MOE_OK;
}

// ---- stack ----
moe_status moe_stack_create(moe_layer* const* layers, int32_t n, float eps, moe_stack** out) {
  if (!out) return fail(MOE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!layers || n < 1) return fail(MOE_ERR_INVALID, "need at least one layer");
  for (int i = 0; i < n; ++i) {
    if (!layers[i]) return fail(MOE_ERR_INVALID, "layer %d is NULL", i);
    if (layers[i]->d != layers[0]->d || layers[i]->act != layers[0]->act)
      return fail(MOE_ERR_INVALID, "layer %d has a different d_model or activation type", i);
  }
  if (!(eps > 0.f)) return fail(MOE_ERR_INVALID, "rms_eps must be positive");
  for (int i = 0; i < n; ++i)
    if (layers[i]->dev != layers[0]->dev) return fail(MOE_ERR_INVALID, "layer %d is on another device", i);
  std::unique_ptr<moe_stack> S(new (std::nothrow) moe_stack());
  if (!S) return fail(MOE_ERR_NOMEM, "host allocation failed");
  S->layers.assign(layers, layers + n);
  S->eps = eps;
  S->dev = layers[0]->dev;
  HIP_OK(hipSetDevice(S->dev));
  std::vector<std::array<int, 4>> shapes;
  for (int i = 0; i < n; ++i) {
    const moe_layer* L = layers[i];
    const std::array<int, 4> key{L->E, L->K, L->f, L->fs};
    size_t j = std::find(shapes.begin(), shapes.end(), key) - shapes.begin();
    if (j == shapes.size()) {
      shapes.push_back(key);
      const size_t F = (size_t)L->fs + (size_t)L->K * L->f;
      uint32_t* cnt = nullptr;
      void* rep = nullptr;
      if (dalloc(&cnt, decode_sync_bytes(L->E)) != hipSuccess || dalloc(&rep, decode_arep_bytes((int)F)) != hipSuccess) {
        (void)hipFree(cnt);
        (void)hipFree(rep);
        for (size_t k = 0; k < S->d_counter.size(); ++k) {
          (void)hipFree(S->d_counter[k]);
          (void)hipFree(S->d_arep[k]);
        }
        return fail(MOE_ERR_NOMEM, "stack synchronisation area failed");
      }
      S->d_counter.push_back(cnt);
      S->d_arep.push_back(rep);
      HIP_OK(hipMemset(cnt, 0, decode_sync_bytes(L->E)));
      HIP_OK(hipMemset(rep, 0, decode_arep_bytes((int)F)));  // parity 0: older than any launch
    }
    S->area_of.push_back((int)j);
  }
  HIP_OK(hipDeviceSynchronize());
  *out = S.release();
  return MOE_OK;
}

moe_status moe_stack_forward(void* h, moe_stack* S, int32_t n_tokens, const uint8_t* reuse_mask, int32_t* ids_out,
                             void* stream) {
  if (!S || !h) return fail(MOE_ERR_INVALID, "stack/h is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (size_t l = 0; l < S->layers.size(); ++l) {
    moe_layer* L = S->layers[l];
    LayerArgs a = base_args(L, h, h, n_tokens);
    a.rms = 1;
    a.eps = S->eps;
    a.resid = h;
    a.counter = S->d_counter[S->area_of[l]];  // shared by the stack's layers of this shape (see moe_stack)
    a.arep = S->d_arep[S->area_of[l]];
    moe_fwd_opts o{};
    o.reuse_previous = reuse_mask ? reuse_mask[l] : 0;
    o.topk_ids = ids_out ? ids_out + l * (size_t)n_tokens * L->K : nullptr;
    o.path = MOE_PATH_AUTO;  // the rmsnorm input rules out the prefill path
    moe_layer* next = l + 1 < S->layers.size() ? S->layers[l + 1] : nullptr;
    moe_status st = forward_impl(L, a, &o, s, next, S->prefetch_depth);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_stack_set_prefetch(moe_stack* S, int32_t depth) {
  if (!S) return fail(MOE_ERR_INVALID, "stack is NULL");
  if (depth < 0 || depth > 64) return fail(MOE_ERR_INVALID, "depth=%d not in 0..64", depth);
  S->prefetch_depth = depth;
  return MOE_OK;
}

moe_status moe_stack_destroy(moe_stack* S) {
  if (S) {
    (void)hipSetDevice(S->dev);
    (void)hipDeviceSynchronize();
    for (size_t k = 0; k < S->d_counter.size(); ++k) {
      (void)hipFree(S->d_counter[k]);
      (void)hipFree(S->d_arep[k]);
    }
  }
  delete S;
  return MOE_OK;
}

// ---- host-only policy ----
moe_status moe_lfu_create(int32_t n_slots, moe_lfu** out) {
  if (!out) return fail(MOE_ERR_INVALID, "out is NULL");
  if (n_slots < 1 || n_slots > 1 << 20) return fail(MOE_ERR_INVALID, "n_slots=%d invalid", n_slots);
  *out = new (std::nothrow) moe_lfu(n_slots);
  return *out ? MOE_OK : fail(MOE_ERR_NOMEM, "host allocation failed");
}

moe_status moe_lfu_step(moe_lfu* P, const int32_t* chosen, int32_t n, int32_t* slot_out, int32_t* miss_out) {
  if (!P || (n > 0 && (!chosen || !slot_out || !miss_out))) return fail(MOE_ERR_INVALID, "NULL argument");
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < i; ++j)
      if (chosen[i] == chosen[j]) return fail(MOE_ERR_INVALID, "chosen ids must be distinct");
  if (!P->policy.step(chosen, n, slot_out, miss_out, nullptr))
    return fail(MOE_ERR_STATE, "%d chosen experts exceed %zu slots", n, P->policy.slots.size());
  return MOE_OK;
}

moe_status moe_lfu_stats(const moe_lfu* P, moe_cache_stats* out) {
  if (!P || !out) return fail(MOE_ERR_INVALID, "NULL argument");
  *out = moe_cache_stats{P->policy.accesses, P->policy.hits,       P->policy.misses,       P->policy.evictions, 0, 0,
                         P->policy.prefetches, P->policy.prefetch_used};
  return MOE_OK;
}

moe_status moe_lfu_prefetch(moe_lfu* P, const int32_t* experts, int32_t n, int32_t* slot_out) {
  if (!P || (n > 0 && (!experts || !slot_out))) return fail(MOE_ERR_INVALID, "NULL argument");
  if (n < 0) return fail(MOE_ERR_INVALID, "n=%d negative", n);
  std::vector<int32_t> ev(n > 0 ? n : 1);
  P->policy.prefetch(experts, n, slot_out, ev.data());
  return MOE_OK;
}

moe_status moe_lfu_destroy(moe_lfu* P) {
  delete P;
  return MOE_OK;
}

moe_status moe_lru_create(int32_t n_slots, moe_lru** out) {
  if (!out) return fail(MOE_ERR_INVALID, "out is NULL");
  if (n_slots < 1 || n_slots > 1 << 20) return fail(MOE_ERR_INVALID, "n_slots=%d invalid", n_slots);
  *out = new (std::nothrow) moe_lru(n_slots);
  return *out ? MOE_OK : fail(MOE_ERR_NOMEM, "host allocation failed");
}

moe_status moe_lru_step(moe_lru* P, int32_t layer, const int32_t* chosen, int32_t n, int32_t* slot_out,
                        int32_t* miss_out) {
  if (!P || (n > 0 && (!chosen || !slot_out || !miss_out))) return fail(MOE_ERR_INVALID, "NULL argument");
  if (layer < 0) return fail(MOE_ERR_INVALID, "layer key %d must be >= 0", layer);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < i; ++j)
      if (chosen[i] == chosen[j]) return fail(MOE_ERR_INVALID, "chosen ids must be distinct");
  std::vector<int32_t> el(n > 0 ? n : 1), ee(n > 0 ? n : 1);
  if (!P->policy.step(layer, chosen, n, slot_out, miss_out, el.data(), ee.data()))
    return fail(MOE_ERR_STATE, "%d chosen experts exceed %zu slots", n, P->policy.slots.size());
  return MOE_OK;
}

moe_status moe_lru_stats(const moe_lru* P, moe_cache_stats* out) {
  if (!P || !out) return fail(MOE_ERR_INVALID, "NULL argument");
  *out = moe_cache_stats{P->policy.accesses, P->policy.hits, P->policy.misses, P->policy.evictions, 0, 0, 0, 0};
  return MOE_OK;
}

moe_status moe_lru_destroy(moe_lru* P) {
  delete P;
  return MOE_OK;
}

}  // extern "C"

// Kernel-side argument blocks and launchers shared by the host library code.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

constexpr int kThreads = 256;  // decode kernels: 4 wavefronts of 64

// Optional host-side hook for live per-kernel timing: hands out a pair of HIP
// events that the launch attaches to the kernel's own start and stop.
struct Profiler {
  virtual void pair(int kernel, hipEvent_t* start, hipEvent_t* stop) = 0;
  virtual ~Profiler() = default;
};

// Launch `kernel`; with a profiler, through hipExtLaunchKernelGGL so the
// events record the kernel's start and end on stream `s`.
template <class Kern, class... Args>
inline void launch_timed(Profiler* prof, int kid, Kern kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         Args... args) {
  if (prof) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    prof->pair(kid, &e0, &e1);
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0, args...);
  } else {
    kernel<<<grid, block, lds, s>>>(args...);
  }
}
enum : int { kKRouteShared = 0, kKRoutedGateUp = 1, kKDownCombine = 2, kKSort = 3, kKPrefillGateUp = 4,
             kKPrefillDown = 5, kKPrefillCombine = 6, kKPrefillRoute = 7, kKTopK = 8, kKFusedLayer = 9,
             kNumKernels = 10 };

// Offsets of gate/up/down Q and SB regions inside an expert blob.
struct BlobOffsets {
  uint32_t gq, gsb, uq, usb, dq, dsb;
};

struct LayerArgs {
  int d, E, K, f, fs, T;
  int act;       // 0 = fp32, 1 = bf16 activations
  int rms;       // 1: the input is a residual stream h; the layer sees act(rmsnorm(h))
  float eps;
  const void* x;  // [T][d]
  // router
  const int8_t* router_w;
  const uint16_t* router_scale;
  const float* router_bias;  // nullable
  // experts
  const uint64_t* expert_addr;  // [E] device address of each expert blob (0 = absent)
  const uint8_t* expert_base;   // resident layers: blob of expert e at expert_base + e * expert_stride
  uint64_t expert_stride;
  const uint8_t* shared_blob;   // nullable when fs == 0
  const uint8_t* zero_blob;     // one all-zero routed blob (read in place of a missing expert)
  BlobOffsets ro, so;           // routed / shared blob offsets
  // workspace
  float* logits;       // [T][E]
  int32_t* ids;        // [T][K]
  uint64_t* sel_addr;  // [T][K] blob address of each chosen expert (written with the ids)
  float* wts;          // [T][K]
  uint32_t* counter;   // synchronisation area of the fused kernel (decode_sync_bytes(E)), zeroed at creation
  void* abuf;          // [T][F] F = fs + K*f: fp16 pair-permuted (bf16 mode) or fp32
  void* arep;          // fused kernel: its own parity-tagged copies of the activation vector
  int32_t* err;        // sticky error flags
  // options
  const int32_t* forced;  // [T][K] or null
  int32_t* ids_out;       // [T][K] or null
  float* w_out;           // [T][K] or null
  void* out;              // [T][d]
  const void* resid;      // [T][d] or null
  // which parts to run (0 = all): 1 router + top-K, 2 shared gate/up,
  // 4 routed gate/up, 8 down + combine; the router and the shared gate/up
  // share a launch when both are asked for
  int stages;
  int topk_in_gate_up;  // 1: every routed gate/up workgroup runs the top-K itself
  int32_t* host_ids;    // T == 1, streamed layers: the routed gate/up's top-K workgroup also writes the
  uint32_t* host_flag;  // chosen ids here (host memory, device view), then host_seq into *host_flag
  uint32_t host_seq;
  // One token: routed gate/up and down kernels queued before the host's cache
  // step.  The device expert table then holds exactly what the cache holds, so
  // a nonzero address marks a hit: gate/up computes those slots only, and the
  // down kernel runs only when every chosen expert was a hit.  The host
  // launches the misses behind their fills, then the down kernel again.
  int hits_only;
  uint32_t run_mask;    // one token: the routed gate/up launch computes only the slots set here (0 = all);
                        // its grid holds popcount(run_mask) * f/8 workgroups
  int shared_in_routed;  // 1: the routed gate/up launch also runs the shared expert's gate/up, in its
                         // first fs/8 workgroups (which wait for nothing)
  int sel_from_table;   // 1: routed gate/up takes each chosen expert's address from expert_addr[ids]
                        // (current after the call's fills) and writes it to sel_addr for the down kernel
  int fused;            // 1: one launch per layer (batch 1, bf16, resident experts)
  Profiler* prof;  // host pointer, never read by the kernels
};

enum : int { kStageRouter = 1, kStageShared = 2, kStageRouted = 4, kStageDown = 8, kStageAll = 15 };

enum : int32_t { kErrBadForcedId = 1, kErrMissingExpert = 2, kErrSyncTimeout = 4, kErrRange = 8 };

// The decode kernels hand the intermediate activations silu(g)*u between
// workgroups as fp16; a value at or above this magnitude (the largest fp16
// value) would not survive the hand-off, so the kernel raises kErrRange.
constexpr float kF16HandoffMax = 65504.f;

hipError_t launch_decode(const LayerArgs& a, hipStream_t s);

// Cache fills by a kernel on the call's stream: each blob is read from pinned
// host memory over the host link and written to its slot; then the layer's
// device expert table gets the filled experts' addresses, and zeros for the
// experts the fills evicted.  Kernel arguments only, no workspace.
constexpr int kMaxFills = 32;
struct FillArgs {
  int n;           // blobs (<= kMaxFills)
  uint64_t bytes;  // per blob, a multiple of 16
  const uint8_t* src[kMaxFills];  // device view of pinned host memory
  uint8_t* dst[kMaxFills];        // cache slots
  uint64_t* table;                // [E] device expert table
  int32_t expert[kMaxFills];      // table[expert[i]] = dst[i]
  int32_t evicted[kMaxFills];     // table[evicted[i]] = 0 (when >= 0)
};
hipError_t launch_fill(const FillArgs& f, hipStream_t s);
// The allocation-free forward's workspace: a device array of this many bytes
// per GPU; *ptr receives its address on the current device.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void** ptr);
// Dequantise one matrix of an expert blob from the device layout into fp32
// out[rows][cols] = fma(scale, q, bias) (test hook).
hipError_t launch_dequant(const uint8_t* blob, uint32_t q_off, uint32_t sb_off, int rows, int cols, float* out,
                          hipStream_t s);
// Whether the single-launch decode kernel can serve these arguments.
bool decode_fused_ok(const LayerArgs& a);
// Bytes of its synchronisation area for E experts.
size_t decode_sync_bytes(int E);

struct PrefillArgs {
  LayerArgs L;
  int32_t* counts;   // [E] of a chunk; the router launch gets chunk 0's and writes [chunks][E]
  int32_t* offsets;  // [E+1]
  int32_t* perm;     // [T*K]
  int32_t* inv;      // [T*K]
  int32_t* tiles;    // work list for the grouped GEMMs
  uint32_t* route_cnt;  // arrival counters: per token tile of the call, then per chunk (zero between calls)
  void* xact;        // [T][d] bf16 layer input (after rmsnorm in stack mode)
  uint16_t* A;       // [T*K][f] bf16 routed activations, in perm order
  uint16_t* As;      // [T][fs] bf16 shared activations
  float* Y;          // [T*K][d] fp32 routed outputs, in grouped order
  float* Ys;         // [T][d] fp32 shared-expert outputs
  int32_t* sort_offsets_out;
  int32_t* sort_perm_out;
  struct PrefillStreamer* streamer;  // host object (streamed experts), never read by the kernels
};

// Prefill of a layer whose experts live in host memory: after a chunk's
// routing and grouping are enqueued, the chunk's experts go through the cache
// in groups; the grouped GEMMs run once per group on that group's tile list.
struct PrefillStreamer {
  // the chunk's grouping is enqueued on s (C tokens); returns the group count
  virtual hipError_t plan(const PrefillArgs& p, int C, hipStream_t s, int* n_groups) = 0;
  // group g's experts are made resident and the device table updated, all
  // ordered before what is enqueued next on s; *tiles: its work list (device)
  virtual hipError_t group(int g, hipStream_t s, int32_t** tiles) = 0;
  // group g's GEMMs are enqueued on s
  virtual hipError_t done(int g, hipStream_t s) = 0;
  virtual ~PrefillStreamer() = default;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_sort(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, hipStream_t s);

}  // namespace moe

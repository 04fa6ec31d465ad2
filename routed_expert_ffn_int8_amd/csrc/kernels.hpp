// Kernel-side argument blocks and launchers shared by the host library code.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

constexpr int kThreads = 128;  // every kernel: 2 wavefronts of 64

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
  const uint8_t* shared_blob;   // nullable when fs == 0
  BlobOffsets ro, so;           // routed / shared blob offsets
  // workspace
  float* logits;       // [T][E]
  int32_t* ids;        // [T][K]
  float* wts;          // [T][K]
  uint32_t* counter;   // [T], zero between calls
  void* abuf;          // [T][F] F = fs + K*f: fp16 pair-permuted (bf16 mode) or fp32
  float* asum_part;    // [T][F/8]
  int32_t* err;        // sticky error flags
  // options
  const int32_t* forced;  // [T][K] or null
  int32_t* ids_out;       // [T][K] or null
  float* w_out;           // [T][K] or null
  void* out;              // [T][d]
  const void* resid;      // [T][d] or null
  // which parts to run (0 = all): 1 router + top-K, 2 shared gate/up,
  // 4 routed gate/up, 8 down + combine
  int stages;
};

enum : int { kStageRouter = 1, kStageShared = 2, kStageRouted = 4, kStageDown = 8, kStageAll = 15 };

enum : int32_t { kErrBadForcedId = 1, kErrMissingExpert = 2 };

hipError_t launch_decode(const LayerArgs& a, hipStream_t s);

struct PrefillArgs {
  LayerArgs L;
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E+1]
  int32_t* perm;     // [T*K]
  int32_t* inv;      // [T*K]
  int32_t* tiles;    // work list for the grouped GEMMs
  void* xact;        // [T][d] bf16 layer input (after rmsnorm in stack mode)
  uint16_t* A;       // [T*K][f] bf16 routed activations, in perm order
  uint16_t* As;      // [T][fs] bf16 shared activations
  float* Y;          // [T*K][d] fp32 routed outputs, in perm order
  int32_t* sort_offsets_out;
  int32_t* sort_perm_out;
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_sort(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, hipStream_t s);

}  // namespace moe

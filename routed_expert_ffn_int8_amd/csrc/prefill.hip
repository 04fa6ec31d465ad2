// Prefill path: a chunk of many tokens per call.
//
// Rockchip-NPU MoE streaming plan, §2.5 and §8.4: prompts are processed in
// 128-token chunks so that one fetched expert serves every row of the chunk
// that chose it.  Per chunk:
//   1. router logits on bf16 MFMA (int8 weights are exact in bf16) and the
//      softmax top-K of every token, in one kernel;
//   2. token->expert grouping: counting sort, stable in token order, plus a
//      list of 16-token tiles per expert (and per shared-expert row block);
//   3. grouped gate/up GEMM on bf16 MFMA (v_mfma_f32_16x16x32_bf16): the
//      tile's 16 token rows are staged in LDS, each wavefront owns 16 weight
//      rows and streams their packed nibbles straight from HBM into the MFMA
//      B operand (nibble pair -> bf16 128+q with one and-or), one fresh
//      accumulator per 64-wide group so the group's (scale, bias) is applied
//      in an fp32 epilogue; SiLU(gate)*up is stored as bf16;
//   4. grouped down GEMM the same way, fp32 outputs in grouped order;
//   5. gather-combine y_t = shared_t + sum_k w_{t,k} * Y[pos(t,k)] in fixed
//      k order (no atomics), optional residual, bf16 store.
// BigMoeOnEdge, "re-routing at every token and layer": every token of the
// chunk is routed on its own, and the union of chosen experts can be large.
#include "device.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

template <class T>
__device__ __forceinline__ T ldg(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(reinterpret_cast<uintptr_t>(p));
}

constexpr int kTile = 16;      // tokens per MFMA tile
#ifndef MOE_GU_WAVES
#define MOE_GU_WAVES 16
#endif
#ifndef MOE_DN_WAVES
#define MOE_DN_WAVES 8
#endif
constexpr int kGuThreads = 64 * MOE_GU_WAVES;  // threads of a gate/up GEMM workgroup
constexpr int kDnThreads = 64 * MOE_DN_WAVES;  // threads of a down GEMM workgroup

// ------------------------------------------------------------ sort + tiles
// Exclusive prefix sum of one int per thread over the workgroup (up to 1024
// threads); *total receives the sum.  sh: 16 ints of LDS.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < nw ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(t, o, 64);
      if (lane >= o) t += y;
    }
    if (lane < nw) sh[lane] = t;
  }
  __syncthreads();
  const int base = w > 0 ? sh[w - 1] : 0;
  *total = sh[nw - 1];
  __syncthreads();  // sh may be reused by the caller
  return base + x - v;
}

// Deterministic token->expert grouping by one workgroup of 1024 threads.
// Each expert gets a bitmask over the chunk's tokens (set with LDS atomic-or,
// whose result does not depend on order); its count is the mask's popcount,
// offsets are the exclusive scan, and a pair (t, k) choosing expert e lands at
// offsets[e] + popcount of e's mask below bit t, i.e. the pairs of an expert
// are in ascending token order.  With a tile list it also emits (expert, tile)
// entries: ceil(n_e/16) per chosen expert in expert order, then ceil(T/16) for
// the shared expert (expert id E).  Needs E * ceil(T/32) words of LDS;
// repeated ids in one token's set are counted once.  E <= 1024.
// DEV: the ids were stored by other workgroups of the running kernel and are
// read with device-scope loads.  sh: (E + 1 + E * ceil(T/32)) words of LDS,
// scan_sh: 16 ints.
template <bool DEV>
__device__ __forceinline__ int load_id(const int32_t* p) {
  if (DEV) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool DEV>
__device__ void sort_body(const int32_t* __restrict__ ids, int T, int K, int E, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* tiles, int with_shared, uint32_t* sh, int* scan_sh) {
  const int NW = (T + 31) >> 5;
  int32_t* off = reinterpret_cast<int32_t*>(sh);
  uint32_t* mask = sh + E + 1;
  const int tid = threadIdx.x, n = T * K;
  for (int i = tid; i < E * NW; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = load_id<DEV>(ids + i), t = i / K;
    if (e >= 0 && e < E) atomicOr(&mask[e * NW + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  int c = 0;
  if (tid < E)
    for (int w = 0; w < NW; ++w) c += __popc(mask[tid * NW + w]);
  int total = 0, ntile_total = 0;
  const int o = block_excl_scan(c, scan_sh, &total);
  const int nt_e = (c + kTile - 1) / kTile;
  const int to = block_excl_scan(nt_e, scan_sh, &ntile_total);
  if (tid < E) {
    off[tid] = o;
    counts[tid] = c;
    offsets[tid] = o;
    if (tiles)
      for (int tt = 0; tt < nt_e; ++tt) {
        tiles[1 + 2 * (to + tt)] = tid;
        tiles[2 + 2 * (to + tt)] = tt;
      }
  }
  if (tid == 0) {
    off[E] = total;
    offsets[E] = total;
  }
  if (tiles) {
    const int ns = with_shared ? (T + kTile - 1) / kTile : 0;
    for (int tt = tid; tt < ns; tt += blockDim.x) {
      tiles[1 + 2 * (ntile_total + tt)] = E;
      tiles[2 + 2 * (ntile_total + tt)] = tt;
    }
    if (tid == 0) tiles[0] = ntile_total + ns;
  }
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = load_id<DEV>(ids + i), t = i / K;
    if (e < 0 || e >= E) continue;
    const uint32_t* m = mask + e * NW;
    int rank = __popc(m[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(m[w]);
    const int pos = off[e] + rank;
    perm[pos] = i;
    inv[i] = pos;
  }
}

__global__ __launch_bounds__(1024) void sort_kernel(const int32_t* __restrict__ ids, int T, int K, int E,
                                                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                                   int32_t* tiles, int with_shared) {
  extern __shared__ uint32_t sh[];  // off[E+1], mask[E][NW]
  __shared__ int scan_sh[16];
  sort_body<false>(ids, T, K, E, counts, offsets, perm, inv, tiles, with_shared, sh, scan_sh);
}

constexpr int kChunkTokens = 128;  // prefill chunk (Rockchip-NPU plan §8.4)
constexpr int kChunkTiles = kChunkTokens / 16;  // token tiles per chunk

// Entries of a chunk's (expert, tile) list: at most T*K/16 + E tiles of
// routed experts and ceil(T/16) of the shared expert.
__host__ __device__ inline size_t max_tiles(int T, int K, int E) {
  return (size_t)T * K / 16 + E + (T + 15) / 16 + 1;
}
__host__ __device__ inline size_t tile_list_ints(int K, int E) { return 1 + 2 * max_tiles(kChunkTokens, K, E); }

// ------------------------------------------------------------ router + top-K
// Workgroup (16-token tile, 16 experts) of 16 wavefronts: they split d in
// sixteen and each runs v_mfma_f32_16x16x32_bf16 over its share, A = the
// token rows (bf16, straight from memory), B = the int8 router rows
// converted exactly to bf16; the 16 partial 16x16 blocks are summed in a fixed
// order in LDS and scaled: logit = scale_e * acc + bias_e.  Logits go to the
// layer's logit array with device-scope stores.  The workgroup that completes
// a token tile (an arrival counter, which that workgroup resets for the next
// call) runs the softmax top-K of the tile's tokens, one wavefront per token;
// the one that completes a chunk's last tile then groups the chunk's tokens
// by expert.  One launch covers every token of a prefill call.
constexpr int kRouteWaves = 16;
constexpr int kRoutePre = 4;  // k-blocks of router weights in flight per lane

__device__ __forceinline__ uint32_t int8x2_to_bf16x2(uint32_t w, int j) {  // bytes 2j, 2j+1 of w
  const float lo = (float)(((int)(w << (24 - 16 * j))) >> 24);
  const float hi = (float)(((int)(w << (16 - 16 * j))) >> 24);
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);  // exact: |q| <= 128
}

size_t route_lds_bytes(int E) { return (size_t)kTile * E * 4; }

template <int NE>
__global__ __launch_bounds__(64 * kRouteWaves) void pf_route_kernel(PrefillArgs p) {
  extern __shared__ __align__(16) char smem[];  // [16][E] logits of the tile, then the sort's words (last workgroup)
  __shared__ float part[kRouteWaves][64][4];
  __shared__ uint32_t scratch[kRouteWaves][2 * 64];
  __shared__ uint32_t last_sh;
  __shared__ int sort_sh[16];
  const LayerArgs& a = p.L;
  const int d = a.d, E = a.E, T = a.T;
  const int t0 = blockIdx.x * kTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int e = 16 * blockIdx.y + n, ec = min(e, E - 1);
  const int KB = d / 32;
  const int k_lo = (KB * wave) / kRouteWaves, k_hi = (KB * (wave + 1)) / kRouteWaves;
  const int8_t* wrow = a.router_w + (size_t)ec * d + 8 * kb;
  const uint16_t* xrow = static_cast<const uint16_t*>(a.x) + (size_t)min(t0 + n, T - 1) * d + 8 * kb;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = k_lo; k0 < k_hi; k0 += kRoutePre) {
    v2u wq[kRoutePre];
    v4u xv[kRoutePre];
#pragma unroll
    for (int i = 0; i < kRoutePre; ++i) {
      const int k = min(k0 + i, k_hi - 1);
      wq[i] = ldg<v2u>(wrow + (size_t)k * 32);
      xv[i] = ldg<v4u>(xrow + (size_t)k * 32);
    }
#pragma unroll
    for (int i = 0; i < kRoutePre; ++i) {
      if (k0 + i < k_hi) {
        v4u bv;
        bv[0] = int8x2_to_bf16x2(wq[i][0], 0);
        bv[1] = int8x2_to_bf16x2(wq[i][0], 1);
        bv[2] = int8x2_to_bf16x2(wq[i][1], 0);
        bv[3] = int8x2_to_bf16x2(wq[i][1], 1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[i]), __builtin_bit_cast(bf16x8, bv),
                                                      acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][lane][i] = acc[i];
  __syncthreads();
  if (wave == 0) {
    const float sc = f16_to_f32(ldg<uint16_t>(a.router_scale + ec));
    const float bi = a.router_bias ? ldg<float>(a.router_bias + ec) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // C row m = 4 kb + i (token), column n (expert)
      float v = 0.f;
      for (int w = 0; w < kRouteWaves; ++w) v += part[w][lane][i];
      const int t = t0 + 4 * kb + i;
      if (t < T && e < E)
        __hip_atomic_store(a.logits + (size_t)t * E + e, fmaf(sc, v, bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // logit stores done before the arrival
    if (lane == 0) {
      const uint32_t old = atomicAdd(p.route_cnt + blockIdx.x, 1u);
      last_sh = old == gridDim.y - 1 ? 1u : 0u;
      if (last_sh) __hip_atomic_store(p.route_cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (!last_sh) return;
  const int t = t0 + wave;
  if (t < T) {
    float* s_log = reinterpret_cast<float*>(smem) + (size_t)wave * E;
    const float* lt = a.logits + (size_t)t * E;
    float v[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) v[i] = __hip_atomic_load(lt + min(lane + 64 * i, E - 1), __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < NE; ++i)
      if (lane + 64 * i < E) s_log[lane + 64 * i] = v[i];
    int id;
    float w;
    topk_wave<NE>(a, t, s_log, &id, &w, scratch[wave]);
    publish_routing(a, t, lane, id, w);  // ids with device-scope stores
  }
  // The workgroup that completes a chunk's last token tile (a per-chunk
  // arrival counter after the tiles', reset by that workgroup) groups the
  // chunk's tokens by expert into the chunk's buffers, reading the other
  // tiles' ids with device-scope loads.  The launch covers every chunk of
  // the call, so no chunk pays a launch of its own for routing or grouping.
  __builtin_amdgcn_s_waitcnt(0);  // this tile's ids are stored before the arrival
  __syncthreads();
  const int c = blockIdx.x / kChunkTiles;
  if (threadIdx.x == 0) {
    const uint32_t tiles_c = min((uint32_t)kChunkTiles, gridDim.x - (uint32_t)c * kChunkTiles);
    uint32_t* cnt = p.route_cnt + gridDim.x + c;
    const uint32_t old = atomicAdd(cnt, 1u);
    last_sh = old == tiles_c - 1 ? 1u : 0u;
    if (last_sh) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last_sh) return;
  const int c0 = c * kChunkTokens, C = min(kChunkTokens, T - c0);
  sort_body<true>(a.ids + (size_t)c0 * a.K, C, a.K, E, p.counts + (size_t)c * E, p.offsets + (size_t)c * (E + 1),
                  p.perm + (size_t)c0 * a.K, p.inv + (size_t)c0 * a.K, p.tiles + (size_t)c * tile_list_ints(a.K, E),
                  a.fs > 0 ? 1 : 0, reinterpret_cast<uint32_t*>(smem), sort_sh);
}

// ------------------------------------------------------------ tile staging
struct TileInfo {
  bool valid;
  bool shared;
  int e, tt, rows, base;  // rows of this expert (or T), first grouped row
  int m_valid;             // valid token rows in this tile
  const uint8_t* blob;
};

__device__ __forceinline__ TileInfo tile_info(const PrefillArgs& p, int tile) {
  TileInfo ti{};
  const LayerArgs& a = p.L;
  if (tile >= p.tiles[0]) return ti;
  ti.valid = true;
  ti.e = p.tiles[1 + 2 * tile];
  ti.tt = p.tiles[2 + 2 * tile];
  ti.shared = (ti.e == a.E);
  ti.rows = ti.shared ? a.T : p.counts[ti.e];
  ti.base = ti.shared ? 0 : p.offsets[ti.e];
  ti.m_valid = min(kTile, ti.rows - ti.tt * kTile);
  ti.blob = ti.shared ? a.shared_blob
                      : (a.expert_base ? a.expert_base + (size_t)ti.e * a.expert_stride  // resident
                                       : reinterpret_cast<const uint8_t*>(a.expert_addr[ti.e]));  // cache slot
  return ti;
}

// Stage 16 rows of bf16 activations into LDS: pair-permuted words
// (v[8j+m], v[8j+m+4]) per 16-byte word, rows padded by 16 bytes against bank
// conflicts, and per-group sums gsum[g][m].  rows[m] is the source row (or
// nullptr for an empty row), natural order when PERMUTE, already paired
// otherwise.  STG = 16-byte words per thread (16 rows x width columns / NTH
// threads).  In two steps, so that a kernel can request its first weights
// between them: stage_rows_load issues every load of the thread (branch-free,
// all in flight at once); stage_rows_commit writes LDS and ends with a
// barrier.  A wavefront's loads complete in order, so the commit waits for
// the row loads only and weights requested after them stay in flight.
template <int NTH, int STG>
__device__ __forceinline__ void stage_rows_load(int width, const uint16_t* const* rows, v4u (&buf)[STG]) {
  const int W = width >> 3;
  const int total = kTile * W;
  const uint16_t* any_row = rows[0] ? rows[0] : rows[kTile - 1];
#pragma unroll
  for (int it = 0; it < STG; ++it) {
    const int idx = min((int)threadIdx.x + NTH * it, total - 1);
    const int m = idx / W, j = idx - m * W;
    const uint16_t* src = rows[m] ? rows[m] : any_row;
    const v4u w = ldg<v4u>(src + (size_t)j * 8);
    buf[it] = rows[m] ? w : v4u{0u, 0u, 0u, 0u};
  }
}
template <int NTH, bool PERMUTE, int STG>
__device__ __forceinline__ void stage_rows_commit(int width, v4u (&buf)[STG], v4u* lds, float* gsum) {
  const int W = width >> 3, stride = W + 1;
  const int total = kTile * W;
#pragma unroll
  for (int it = 0; it < STG; ++it) {
    const int idx = threadIdx.x + NTH * it;
    if (idx < total) {  // uniform across each aligned group of 8 lanes
      const int m = idx / W, j = idx - m * W;
      const v4u w = buf[it];
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      }
      if (PERMUTE) {
        v4u pw;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pw[q] = (uint32_t)f32_to_bf16(v[q]) | ((uint32_t)f32_to_bf16(v[q + 4]) << 16);
        lds[m * stride + j] = pw;
      } else {
        lds[m * stride + j] = w;
      }
      float part = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
      part = xor_sum(part, 1, 4);  // the 8 words of one group sit in 8 consecutive lanes
      if ((j & 7) == 0) gsum[(j >> 3) * kTile + m] = part;
    }
  }
  __syncthreads();
}

// The nibble mask held in a vector register: the compiler cannot fold it
// into an immediate (vector ALU instructions with three operands take none
// on gfx9), so each pair is one v_and_or_b32 (mask in a VGPR, exponent in an
// SGPR) instead of an and plus an or: 7 instructions per packed word, not 11.
__device__ __forceinline__ uint32_t nibble_mask_v() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m));
  return m;
}

// MFMA B operand of one packed word: four bf16 pairs 128 + q (see nib_pairs).
__device__ __forceinline__ bf16x8 b_operand(uint32_t w, uint32_t mask) {
  constexpr uint32_t M = (kExpBf16 << 8) * 0x00010001u;
  v4u v;
  v[0] = (w & mask) | M;
  v[1] = ((w >> 4) & mask) | M;
  v[2] = ((w >> 8) & mask) | M;
  v[3] = ((w >> 12) & mask) | M;
  return __builtin_bit_cast(bf16x8, v);
}

// Word v of lane (lane & 15) + 16 j of the wavefront (j uniform).
__device__ __forceinline__ uint32_t from_quarter(uint32_t v, int j) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 15) + 16 * j) << 2), (int)v);
}

__device__ __forceinline__ void group_epilogue(f32x4& acc, const f32x4& t, uint32_t sb, const float* xs4) {
  const float s = f16_to_f32((uint16_t)(sb & 0xFFFFu));
  const float bb = f16_to_f32((uint16_t)(sb >> 16)) - 128.f * s;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, t[i], fmaf(bb, xs4[i], acc[i]));
}

#ifndef MOE_PF_PRE
#define MOE_PF_PRE 4
#endif
constexpr int kPre = MOE_PF_PRE;  // groups of weights in flight per lane (gate/up)

// Raw buffer resource over an expert blob (no range check: every offset is
// inside the blob by construction) and a 4-byte load at voffset + soffset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t blob_rsrc(const uint8_t* blob) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint32_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ v2u bload2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
}

// ------------------------------------------------------------ gate/up GEMM
// One workgroup: one (expert, 16-token tile) x 256 rows of gate and up, one
// 16-row tile per wavefront (16 wavefronts), so a 512-row expert stages each
// token tile in two workgroups (with 8 wavefronts, four: 56.7-57.0 against
// 58.0 us per 128-token chunk).  Lane (n = lane & 15, kb = lane >> 4) of
// wavefront w owns weight row n0 + 16 t + n of tile t; for MFMA j of a group
// it feeds word 2 kb + j of the row (B operand) and of the tile rows (A
// operand, from LDS), so both operands share one order of the 64 k values,
// and a lane's two words of a group are adjacent in the packed layout: one
// 8-byte load.  The scale/bias words go out four groups at a time: lane
// quarter kb loads group g0 + kb of its row, and each group's word is taken
// from its quarter through ds_bpermute (a quarter of the load instructions
// for them).
#ifndef MOE_GU_TILES
#define MOE_GU_TILES 1
#endif
constexpr int kGuTiles = MOE_GU_TILES;
constexpr int kGuRowsPerWG = 16 * kGuTiles * MOE_GU_WAVES;

template <int STG>
__global__ __launch_bounds__(kGuThreads) void pf_gate_up_kernel(PrefillArgs p) {
  extern __shared__ __align__(16) char smem[];
  const LayerArgs& a = p.L;
  const int nch = (max(a.f, a.fs) + kGuRowsPerWG - 1) / kGuRowsPerWG;
  const int tile = blockIdx.x / nch, ch = blockIdx.x - tile * nch;
  const TileInfo ti = tile_info(p, tile);
  if (!ti.valid) return;
  const int fdim = ti.shared ? a.fs : a.f;
  if (ch * kGuRowsPerWG >= fdim) return;
  const int d = a.d, G = d >> 6, W = d >> 3;
  v4u* xs_lds = reinterpret_cast<v4u*>(smem);
  float* gsum = reinterpret_cast<float*>(smem + (size_t)kTile * (W + 1) * 16);
  const BlobOffsets& o = ti.shared ? a.so : a.ro;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int n0 = ch * kGuRowsPerWG + wave * 16 * kGuTiles;
  // Buffer loads: the blob is the resource, a per-lane offset is computed
  // once and the group's offset is a uniform (scalar) operand, so a load
  // costs no vector address arithmetic.
  const auto rs = blob_rsrc(ti.blob);
  uint32_t vgq[kGuTiles], vuq[kGuTiles], vgs[kGuTiles], vus[kGuTiles];
#pragma unroll
  for (int t = 0; t < kGuTiles; ++t) {
    const int row = min(n0 + 16 * t, fdim - 16) + n;
    const int rb = row >> 3, r = row & 7;
    const uint32_t vq = (uint32_t)rb * G * 256 + (kb >> 1) * 128 + r * 16 + (kb & 1) * 8;  // + g * 256
    const uint32_t vsb = ((uint32_t)rb * G * 8 + r) * 4;           // + g * 32
    vgq[t] = o.gq + vq;
    vuq[t] = o.uq + vq;
    vgs[t] = o.gsb + vsb;
    vus[t] = o.usb + vsb;
  }
  __shared__ const uint16_t* rows[kTile];
  if (threadIdx.x < kTile) {
    const int m = threadIdx.x, q = ti.tt * kTile + m;
    const int tok = (m >= ti.m_valid) ? -1 : (ti.shared ? q : p.perm[ti.base + q] / a.K);
    rows[m] = tok < 0 ? nullptr : static_cast<const uint16_t*>(p.xact) + (size_t)tok * d;
  }
  __syncthreads();
  // The token rows are requested first and the first kPre groups of weights
  // right behind them; then the rows are committed to LDS, which waits for
  // the row loads only (a wavefront's loads complete in order), so the
  // weights stream while the tile is staged.  Measured: 57.9 against 59.7 us
  // per 128-token chunk.
  v4u sbuf[STG];
  stage_rows_load<kGuThreads, STG>(d, rows, sbuf);
  v2u wg[kPre][kGuTiles], wu[kPre][kGuTiles];
  uint32_t sgc[kGuTiles], suc[kGuTiles], sgn[kGuTiles], sun[kGuTiles];
  auto fetch = [&](int i, uint32_t g) {
#pragma unroll
    for (int t = 0; t < kGuTiles; ++t) {
      wg[i][t] = bload2(rs, vgq[t], g * 256);
      wu[i][t] = bload2(rs, vuq[t], g * 256);
    }
  };
  auto fetch_sb = [&](int g0) {  // lane quarter kb: scale/bias of group g0 + kb
    const uint32_t go = (uint32_t)min(g0 + kb, G - 1) * 32;
#pragma unroll
    for (int t = 0; t < kGuTiles; ++t) {
      sgn[t] = bload(rs, vgs[t] + go, 0);
      sun[t] = bload(rs, vus[t] + go, 0);
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  fetch_sb(0);
#pragma unroll
  for (int i = 0; i < kPre; ++i) {  // in slot order (see the refill below)
    __builtin_amdgcn_sched_barrier(0);
    fetch(i, (uint32_t)min(i, G - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
  stage_rows_commit<kGuThreads, true, STG>(d, sbuf, xs_lds, gsum);
  __builtin_amdgcn_sched_barrier(0);
  if (n0 >= fdim) return;  // no barrier follows
  f32x4 accg[kGuTiles], accu[kGuTiles];
#pragma unroll
  for (int t = 0; t < kGuTiles; ++t) accg[t] = accu[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const v4u* arow = xs_lds + n * (W + 1);  // A operand: tile row m = lane & 15
  const uint32_t nmask = nibble_mask_v();
  // Branch-free loads and products (clamped group index; the epilogue of a
  // group past the end is skipped) so the compiler can keep kPre groups of
  // loads in flight across iterations.
  for (int g0 = 0; g0 < G; g0 += kPre) {
#pragma unroll
    for (int t = 0; t < kGuTiles; ++t) {
      sgc[t] = sgn[t];
      suc[t] = sun[t];
    }
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int g = g0 + i;
      const int gc = min(g, G - 1);
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, arow[gc * 8 + 2 * kb]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, arow[gc * 8 + 2 * kb + 1]);
      const float* xs4 = gsum + gc * kTile + 4 * kb;
#pragma unroll
      for (int t = 0; t < kGuTiles; ++t) {
        f32x4 tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b_operand(wg[i][t].x, nmask), zero, 0, 0, 0);
        tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b_operand(wg[i][t].y, nmask), tg, 0, 0, 0);
        f32x4 tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b_operand(wu[i][t].x, nmask), zero, 0, 0, 0);
        tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b_operand(wu[i][t].y, nmask), tu, 0, 0, 0);
        if (g < G) {  // uniform: groups past the end (clamped loads) are dropped
          group_epilogue(accg[t], tg, from_quarter(sgc[t], i), xs4);
          group_epilogue(accu[t], tu, from_quarter(suc[t], i), xs4);
        }
      }
      // refill this slot with group g + kPre, as one batch after this
      // group's products: slots then complete in order, so the next
      // group's wait leaves the other slots' loads in flight
      __builtin_amdgcn_sched_barrier(0);
      if (i == 0) fetch_sb(g0 + kPre);
      fetch(i, (uint32_t)min(g + kPre, G - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // D layout: lane holds column n (weight row) for tile rows 4*kb + i
  uint16_t* dst = ti.shared ? p.As : p.A;
#pragma unroll
  for (int t = 0; t < kGuTiles; ++t) {
    const int c = n0 + 16 * t + n;
    if (n0 + 16 * t >= fdim) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kb + i;
      if (m < ti.m_valid) {
        const float v = silu(accg[t][i]) * accu[t][i];
        const size_t grow = (size_t)(ti.base + ti.tt * kTile + m);
        const int j = c >> 3, q = c & 7;
        dst[grow * fdim + j * 8 + (q & 3) * 2 + (q >> 2)] = f32_to_bf16(v);
      }
    }
  }
}

// ------------------------------------------------------------ down GEMM
// One workgroup: one (expert, 16-token tile) x 256 rows of the down
// projection, two 16-row tiles per wavefront sharing each A operand read;
// outputs fp32 rows in grouped order (shared: token order).
#ifndef MOE_DN_TILES
#define MOE_DN_TILES 2
#endif
#ifndef MOE_DN_PRE
#define MOE_DN_PRE 4
#endif
constexpr int kDnTiles = MOE_DN_TILES;                   // 16-row tiles per wavefront
constexpr int kDnRowsPerWG = 16 * kDnTiles * MOE_DN_WAVES;
constexpr int kDnPre = MOE_DN_PRE;                       // groups in flight per lane

template <int STG>
__global__ __launch_bounds__(kDnThreads) void pf_down_kernel(PrefillArgs p) {
  extern __shared__ __align__(16) char smem[];
  const LayerArgs& a = p.L;
  const int nch = (a.d + kDnRowsPerWG - 1) / kDnRowsPerWG;
  const int tile = blockIdx.x / nch, ch = blockIdx.x - tile * nch;
  const TileInfo ti = tile_info(p, tile);
  if (!ti.valid) return;
  const int fdim = ti.shared ? a.fs : a.f;
  const int G = fdim >> 6, W = fdim >> 3;
  v4u* as_lds = reinterpret_cast<v4u*>(smem);
  float* gsum = reinterpret_cast<float*>(smem + (size_t)kTile * (W + 1) * 16);
  const BlobOffsets& o = ti.shared ? a.so : a.ro;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int n0 = ch * kDnRowsPerWG + wave * 16 * kDnTiles;  // tile t covers rows n0 + 16 t ..
  const auto rs = blob_rsrc(ti.blob);
  uint32_t vq[kDnTiles], vs[kDnTiles];
#pragma unroll
  for (int t = 0; t < kDnTiles; ++t) {
    const int row = min(n0 + 16 * t, a.d - 16) + n;
    const int rb = row >> 3, r = row & 7;
    vq[t] = o.dq + (uint32_t)rb * G * 256 + (kb >> 1) * 128 + r * 16 + (kb & 1) * 8;  // + g * 256 (as gate/up)
    vs[t] = o.dsb + ((uint32_t)rb * G * 8 + r) * 4;           // + g * 32
  }
  __shared__ const uint16_t* rows[kTile];
  if (threadIdx.x < kTile) {
    const int m = threadIdx.x;
    const uint16_t* src = ti.shared ? p.As : p.A;
    rows[m] = (m >= ti.m_valid) ? nullptr : src + (size_t)(ti.base + ti.tt * kTile + m) * fdim;
  }
  __syncthreads();
  v4u sbuf[STG];
  stage_rows_load<kDnThreads, STG>(fdim, rows, sbuf);  // then the first weights, then the commit (as in gate/up)
  v2u w[kDnPre][kDnTiles];
  uint32_t sbc[kDnTiles], sbn[kDnTiles];
  // slot i's loads go out as one batch, slots in order (scheduling
  // barriers), so each group waits only for its own slot; the scale/bias
  // words of four groups go out with slot 0 (as in gate/up)
  auto fetch = [&](int i, uint32_t g) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) w[i][t] = bload2(rs, vq[t], g * 256);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto fetch_sb = [&](int g0) {
    const uint32_t go = (uint32_t)min(g0 + kb, G - 1) * 32;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) sbn[t] = bload(rs, vs[t] + go, 0);
  };
  fetch_sb(0);
#pragma unroll
  for (int i = 0; i < kDnPre; ++i) fetch(i, (uint32_t)min(i, G - 1));
  stage_rows_commit<kDnThreads, false, STG>(fdim, sbuf, as_lds, gsum);
  __builtin_amdgcn_sched_barrier(0);
  if (n0 >= a.d) return;  // no barrier follows
  f32x4 acc[kDnTiles];
#pragma unroll
  for (int t = 0; t < kDnTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const v4u* arow = as_lds + n * (W + 1);
  const uint32_t nmask = nibble_mask_v();
  for (int g0 = 0; g0 < G; g0 += kDnPre) {
#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) sbc[t] = sbn[t];
#pragma unroll
    for (int i = 0; i < kDnPre; ++i) {
      const int g = g0 + i;
      const int gc = min(g, G - 1);
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, arow[gc * 8 + 2 * kb]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, arow[gc * 8 + 2 * kb + 1]);
      const float* xs4 = gsum + gc * kTile + 4 * kb;
#pragma unroll
      for (int t = 0; t < kDnTiles; ++t) {
        f32x4 m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b_operand(w[i][t].x, nmask), zero, 0, 0, 0);
        m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b_operand(w[i][t].y, nmask), m, 0, 0, 0);
        if (g < G) group_epilogue(acc[t], m, from_quarter(sbc[t], i), xs4);  // uniform: past-the-end groups dropped
      }
      if (i == 0) fetch_sb(g0 + kDnPre);
      fetch(i, (uint32_t)min(g + kDnPre, G - 1));
    }
  }
  float* dst = ti.shared ? p.Ys : p.Y;
#pragma unroll
  for (int t = 0; t < kDnTiles; ++t) {
    const int c0 = n0 + 16 * t;
    if (c0 >= a.d) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kb + i;
      if (m < ti.m_valid) dst[(size_t)(ti.base + ti.tt * kTile + m) * a.d + c0 + n] = acc[t][i];
    }
  }
}

// ------------------------------------------------------------ combine
// y_t = shared_t + sum_k w_{t,k} * Y[inv[t*K + k]] (k ascending), + residual.
// One thread per 4 consecutive columns (d is a multiple of 64): 16-byte loads
// of the fp32 rows, 8-byte bf16 residual loads and output stores.
constexpr int kCombineCols = 4 * 256;  // columns per workgroup
__global__ __launch_bounds__(256) void pf_combine_kernel(PrefillArgs p) {
  const LayerArgs& a = p.L;
  const int t = blockIdx.y;
  const int c = blockIdx.x * kCombineCols + threadIdx.x * 4;
  if (c >= a.d) return;
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
  if (a.fs > 0) y = *reinterpret_cast<const f32x4*>(p.Ys + (size_t)t * a.d + c);
  for (int k = 0; k < a.K; ++k) {
    const int pos = p.inv[t * a.K + k];
    const float w = a.wts[t * a.K + k];
    const f32x4 v = *reinterpret_cast<const f32x4*>(p.Y + (size_t)pos * a.d + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = fmaf(w, v[j], y[j]);
  }
  const size_t o = (size_t)t * a.d + c;
  if (a.resid) {
    const v2u r = *reinterpret_cast<const v2u*>(static_cast<const uint16_t*>(a.resid) + o);
    y[0] += bf16_to_f32((uint16_t)(r.x & 0xFFFFu));
    y[1] += bf16_to_f32((uint16_t)(r.x >> 16));
    y[2] += bf16_to_f32((uint16_t)(r.y & 0xFFFFu));
    y[3] += bf16_to_f32((uint16_t)(r.y >> 16));
  }
  v2u out;
  out.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
  out.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
  *reinterpret_cast<v2u*>(static_cast<uint16_t*>(a.out) + o) = out;
}

}  // namespace

// Dynamic LDS granted to the prefill kernels (below the 160 KB per workgroup
// so their few static LDS words still fit).
constexpr int kMaxDynLds = 144 * 1024;

size_t sort_lds_bytes(int T, int E) { return ((size_t)E + 1 + (size_t)E * ((T + 31) / 32)) * 4; }

hipError_t launch_sort(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, hipStream_t s) {
  const size_t lds = sort_lds_bytes(T, E);
  if (lds > kMaxDynLds) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sort_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDynLds);
    if (e != hipSuccess) return e;
  }
  sort_kernel<<<1, 1024, lds, s>>>(ids, T, K, E, counts, offsets, perm, inv, nullptr, 0);
  return hipGetLastError();
}


static size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Layout for calls of up to T tokens, the same for every call: the arrival
// counters first (zero between calls: the workgroup that completes one resets
// it), then each chunk's grouping (counts, offsets, tile list; perm and inv
// [T][K], chunk-local indices), then one chunk's activations and outputs.
size_t prefill_workspace_bytes(int T, int d, int E, int K, int f, int fs) {
  const int C = T < kChunkTokens ? T : kChunkTokens;
  const size_t nc = (size_t)(T + kChunkTokens - 1) / kChunkTokens;
  size_t b = 0;
  b += align_up(((size_t)(T + kTile - 1) / kTile + nc) * 4);                       // arrivals: tiles, chunks
  b += align_up(nc * E * 4) + align_up(nc * (E + 1) * 4);                          // counts, offsets
  b += 2 * align_up((size_t)T * K * 4);                                            // perm, inv
  b += align_up(nc * tile_list_ints(K, E) * 4);                                    // tile lists
  b += align_up((size_t)C * K * f * 2) + align_up((size_t)C * (fs > 0 ? fs : 64) * 2);  // A, As
  b += align_up((size_t)C * K * d * 4) + align_up((size_t)C * d * 4);                  // Y, Ys
  return b;
}

void prefill_carve(PrefillArgs& p, char* ws, int T, int d, int E, int K, int f, int fs) {
  const int C = T < kChunkTokens ? T : kChunkTokens;
  const size_t nc = (size_t)(T + kChunkTokens - 1) / kChunkTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = ws + off;
    off += align_up(bytes);
    return q;
  };
  p.route_cnt = reinterpret_cast<uint32_t*>(take(((size_t)(T + kTile - 1) / kTile + nc) * 4));
  p.counts = reinterpret_cast<int32_t*>(take(nc * E * 4));
  p.offsets = reinterpret_cast<int32_t*>(take(nc * (E + 1) * 4));
  p.perm = reinterpret_cast<int32_t*>(take((size_t)T * K * 4));
  p.inv = reinterpret_cast<int32_t*>(take((size_t)T * K * 4));
  p.tiles = reinterpret_cast<int32_t*>(take(nc * tile_list_ints(K, E) * 4));
  p.A = reinterpret_cast<uint16_t*>(take((size_t)C * K * f * 2));
  p.As = reinterpret_cast<uint16_t*>(take((size_t)C * (fs > 0 ? fs : 64) * 2));
  p.Y = reinterpret_cast<float*>(take((size_t)C * K * d * 4));
  p.Ys = reinterpret_cast<float*>(take((size_t)C * d * 4));
}

// Staging words per thread for 16 rows of `width` bf16 values, rounded up to a power of two.
static int stage_words(int width, int threads) {
  const int need = (kTile * (width / 8) + threads - 1) / threads;
  int s = 1;
  while (s < need) s <<= 1;
  return s;
}

size_t prefill_lds_gate_up(int d) { return (size_t)kTile * (d / 8 + 1) * 16 + (size_t)(d / 64) * kTile * 4; }

// Whole prefill forward over T tokens, in chunks of 128 tokens.
hipError_t launch_prefill(const PrefillArgs& p0, hipStream_t s) {
  const LayerArgs& a0 = p0.L;
  static bool lds_raised = false;  // the gate/up tile needs more than 64 KB of LDS for d > 1984
  if (!lds_raised) {
    const void* fns[] = {reinterpret_cast<const void*>(pf_gate_up_kernel<1>),
                         reinterpret_cast<const void*>(pf_gate_up_kernel<2>),
                         reinterpret_cast<const void*>(pf_gate_up_kernel<4>),
                         reinterpret_cast<const void*>(pf_gate_up_kernel<8>),
                         reinterpret_cast<const void*>(pf_gate_up_kernel<16>),
                         reinterpret_cast<const void*>(pf_down_kernel<1>),
                         reinterpret_cast<const void*>(pf_down_kernel<2>),
                         reinterpret_cast<const void*>(pf_down_kernel<4>),
                         reinterpret_cast<const void*>(pf_down_kernel<8>),
                         reinterpret_cast<const void*>(pf_down_kernel<16>)};
    for (const void* f : fns) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDynLds);
      if (e != hipSuccess) return e;
    }
    // the router's tile of logits for up to 1024 experts (64 KB) next to its 24 KB of static LDS
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(pf_route_kernel<16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)route_lds_bytes(1024));
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  // 1. router + top-K of every token of the call, and each chunk's grouping
  //    and tile list, in one launch
  {
    PrefillArgs p = p0;
    const LayerArgs& a = p.L;
    p.xact = const_cast<void*>(a.x);
    const dim3 g_rt((unsigned)((a.T + kTile - 1) / kTile), (unsigned)((a.E + 15) / 16));
    const dim3 b_rt(64 * kRouteWaves);
    const size_t l_rt = std::max(route_lds_bytes(a.E), sort_lds_bytes(kChunkTokens, a.E));
    if (a.E <= 64)
      launch_timed(a.prof, kKPrefillRoute, pf_route_kernel<1>, g_rt, b_rt, l_rt, s, p);
    else if (a.E <= 128)
      launch_timed(a.prof, kKPrefillRoute, pf_route_kernel<2>, g_rt, b_rt, l_rt, s, p);
    else if (a.E <= 256)
      launch_timed(a.prof, kKPrefillRoute, pf_route_kernel<4>, g_rt, b_rt, l_rt, s, p);
    else
      launch_timed(a.prof, kKPrefillRoute, pf_route_kernel<16>, g_rt, b_rt, l_rt, s, p);
  }
  for (int c0 = 0; c0 < a0.T; c0 += kChunkTokens) {
    PrefillArgs p = p0;
    LayerArgs& a = p.L;
    const int C = (a0.T - c0 < kChunkTokens) ? a0.T - c0 : kChunkTokens;
    const int ci = c0 / kChunkTokens;
    a.T = C;
    p.counts = p0.counts + (size_t)ci * a.E;  // this chunk's grouping
    p.offsets = p0.offsets + (size_t)ci * (a.E + 1);
    p.perm = p0.perm + (size_t)c0 * a.K;
    p.inv = p0.inv + (size_t)c0 * a.K;
    p.tiles = p0.tiles + (size_t)ci * tile_list_ints(a.K, a.E);
    const size_t xo = (size_t)c0 * a.d * 2;
    a.x = static_cast<const char*>(a0.x) + xo;
    a.out = static_cast<char*>(a0.out) + xo;
    if (a0.resid) a.resid = static_cast<const char*>(a0.resid) + xo;
    // The call's routing workspace is [T][K]: each chunk keeps its own rows, so
    // a later call that reuses this call's sets finds every chunk's sets.
    a.ids = a0.ids + (size_t)c0 * a.K;
    a.wts = a0.wts + (size_t)c0 * a.K;
    a.sel_addr = a0.sel_addr + (size_t)c0 * a.K;
    if (a0.forced) a.forced = a0.forced + (size_t)c0 * a.K;
    if (a0.ids_out) a.ids_out = a0.ids_out + (size_t)c0 * a.K;
    if (a0.w_out) a.w_out = a0.w_out + (size_t)c0 * a.K;
    p.xact = const_cast<void*>(a.x);
    hipError_t e;
    // 2. gate/up, 3. down (per group of cached experts when they are streamed), 4. combine
    const size_t mt = max_tiles(C, a.K, a.E);
    int n_groups = 1;
    if (p0.streamer && (e = p0.streamer->plan(p, C, s, &n_groups)) != hipSuccess) return e;
    for (int grp = 0; grp < n_groups; ++grp) {
      if (p0.streamer && (e = p0.streamer->group(grp, s, &p.tiles)) != hipSuccess) return e;
      const int nch_gu = (((a.f > a.fs) ? a.f : a.fs) + kGuRowsPerWG - 1) / kGuRowsPerWG;
      const size_t lds_gu = prefill_lds_gate_up(a.d);
      const dim3 g_gu((unsigned)(mt * nch_gu)), blk(kGuThreads);
      switch (stage_words(a.d, kGuThreads)) {
        case 1: launch_timed(a.prof, kKPrefillGateUp, pf_gate_up_kernel<1>, g_gu, blk, lds_gu, s, p); break;
        case 2: launch_timed(a.prof, kKPrefillGateUp, pf_gate_up_kernel<2>, g_gu, blk, lds_gu, s, p); break;
        case 4: launch_timed(a.prof, kKPrefillGateUp, pf_gate_up_kernel<4>, g_gu, blk, lds_gu, s, p); break;
        case 8: launch_timed(a.prof, kKPrefillGateUp, pf_gate_up_kernel<8>, g_gu, blk, lds_gu, s, p); break;
        default: launch_timed(a.prof, kKPrefillGateUp, pf_gate_up_kernel<16>, g_gu, blk, lds_gu, s, p); break;
      }
      const int fmax = (a.f > a.fs) ? a.f : a.fs;
      const int nch_dn = (a.d + kDnRowsPerWG - 1) / kDnRowsPerWG;
      const size_t lds_dn = (size_t)kTile * (fmax / 8 + 1) * 16 + (size_t)(fmax / 64) * kTile * 4;
      const dim3 g_dn((unsigned)(mt * nch_dn));
      const dim3 blk_dn(kDnThreads);
      switch (stage_words(fmax, kDnThreads)) {
        case 1: launch_timed(a.prof, kKPrefillDown, pf_down_kernel<1>, g_dn, blk_dn, lds_dn, s, p); break;
        case 2: launch_timed(a.prof, kKPrefillDown, pf_down_kernel<2>, g_dn, blk_dn, lds_dn, s, p); break;
        case 4: launch_timed(a.prof, kKPrefillDown, pf_down_kernel<4>, g_dn, blk_dn, lds_dn, s, p); break;
        case 8: launch_timed(a.prof, kKPrefillDown, pf_down_kernel<8>, g_dn, blk_dn, lds_dn, s, p); break;
        default: launch_timed(a.prof, kKPrefillDown, pf_down_kernel<16>, g_dn, blk_dn, lds_dn, s, p); break;
      }
      if (p0.streamer && (e = p0.streamer->done(grp, s)) != hipSuccess) return e;
    }
    launch_timed(a.prof, kKPrefillCombine, pf_combine_kernel, dim3((a.d + kCombineCols - 1) / kCombineCols, C),
                 dim3(256), 0, s, p);
    if (p0.sort_offsets_out)  // one row of E + 1 offsets per chunk
      if ((e = hipMemcpyAsync(p0.sort_offsets_out + (size_t)(c0 / kChunkTokens) * (a.E + 1), p.offsets,
                              (a.E + 1) * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return e;
    if (p0.sort_perm_out)
      if ((e = hipMemcpyAsync(p0.sort_perm_out + (size_t)c0 * a.K, p.perm, (size_t)C * a.K * 4,
                              hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe

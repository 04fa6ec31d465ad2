// Decode path (few tokens per call): three kernels per layer.
//
//   A  route_shared : int8 router GEMV (one router row per wavefront) with the
//                     softmax top-K run by the last router workgroup of each
//                     token, side by side with the shared expert's gate/up
//                     GEMV + SiLU*mul (routing-independent, so it overlaps the
//                     router; Rockchip-NPU plan §2.4 computes the shared
//                     expert while routed experts are still being fetched).
//   B  routed_gu    : gate/up GEMV + SiLU*mul of the K chosen experts.
//   C  down_combine : down GEMV of the shared and K chosen experts and the
//                     weighted sum y = shared + sum_k w_k * down_k
//                     (BigMoeOnEdge, "re-routing at every token and layer":
//                     weighted merge of the chosen experts), optional
//                     residual, one store per output element.
//
// Gate/up and down workgroups own an 8-row block of a matrix: lane
// (r = tid & 7, jj = tid >> 3) reads the 16-byte halves of row r for the
// 64-wide groups g = jj + 16 i, so every wavefront load instruction covers
// eight whole 128-byte lines.  Each lane issues all of its weight loads in
// straight-line code (clamped addresses, no branches) right after the token
// or activation loads, so LDS staging overlaps the weight fetch and every
// byte of the kernel is requested within its first microseconds.
//
// Arithmetic per 64-wide group (affine weights w = s*q + b, Rockchip-NPU
// plan §2.1): sum_c w_c x_c = s * sum_c q_c x_c + b * sum_c x_c.
// bf16 activations: a nibble pair becomes two bf16 values 128 + q with one
// and-or and feeds v_dot2_f32_bf16 against bf16 pairs of x; the 128*sum(x)
// offset is folded into the bias term.  The down projection does the same
// with fp16 (1024 + q) against fp16-rounded activations.  fp32 activations
// use an exact byte->float convert and fp32 FMAs.
#include <algorithm>
#include <mutex>

#include "device.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Bound of every wait loop for another workgroup's results (each round
// sleeps and reloads, so this is well above 100 ms; the waits that occur
// take microseconds): past it the workgroup sets an error flag and goes on,
// so a broken hand-off ends the kernel instead of hanging it.
constexpr uint32_t kSpinLimit = 1u << 18;

// Load through the global address space (the pointers come from tables, so
// the compiler cannot infer it and would emit flat loads).
template <class T>
__device__ __forceinline__ T ldg(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(reinterpret_cast<uintptr_t>(p));
}

// Results handed from one workgroup to another inside the fused kernel are
// written and read with device-scope relaxed atomics (coherent across the
// XCDs' L2 caches without whole-cache write-back or invalidation); ordering
// comes from waiting for the stores before the counter increment.
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same coherence for 16-byte words: buffer loads/stores with the sc1
// cache-policy bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ v4u ld_dev16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
}
__device__ __forceinline__ void st_dev16(__amdgpu_buffer_rsrc_t r, uint32_t off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolSc1);
}

// The fused kernel keeps kAReps copies of the intermediate activation vector,
// a_rep_stride(F) bytes apart, so that the hundreds of down workgroups
// reading it spread over several copies and memory channels.  Values are fp16
// in the pair order of the down projection, rounded to 9 mantissa bits; the
// freed last bit holds the parity of the launch tag, so a reader can tell a
// value of this launch from the previous launch's and clears the bit before
// use (the value is then the same whatever the parity).
constexpr int kAReps = 32;
__host__ __device__ inline size_t a_rep_stride(int F) { return ((size_t)F * 2 + 4095) / 4096 * 4096 + 512; }
__device__ __forceinline__ uint16_t f32_to_f16_tagged(float v, uint32_t tag) {
  uint32_t u = __float_as_uint(v);
  u = (u + 0x1FFFu + ((u >> 14) & 1u)) & ~0x3FFFu;  // round to nearest even at 9 mantissa bits
  return (uint16_t)((f32_to_f16(__uint_as_float(u)) & 0xFFFEu) | (tag & 1u));  // fp16 subnormals may round odd
}
__device__ __forceinline__ bool fresh4(const v4u& w, uint32_t par) {  // par: 0 or 0x00010001
  return ((w[0] & 0x00010001u) == par) & ((w[1] & 0x00010001u) == par) & ((w[2] & 0x00010001u) == par) &
         ((w[3] & 0x00010001u) == par);
}

struct XStage {
  float* xf;   // [d] input as fp32 (after rounding to the activation type)
  v4u* xp;     // [d/64][9] per group: 8 words of bf16 pairs (x[8j+m], x[8j+m+4]),
               // m = 0..3, and one pad word so that the groups read by the 8
               // lanes-groups of a wavefront fall in different LDS banks
  float* xs;   // [d/64] group sums
  float* red;  // [128] cross-wave scratch
};

__device__ __forceinline__ XStage carve_x(char* smem, int d) {
  XStage S;
  S.xf = reinterpret_cast<float*>(smem);
  S.xp = reinterpret_cast<v4u*>(smem + (size_t)d * 4);
  S.xs = reinterpret_cast<float*>(smem + (size_t)d * 4 + (size_t)(d / 64) * 144);
  S.red = S.xs + d / 64;
  return S;
}

__host__ __device__ inline size_t x_stage_bytes(int d) { return (size_t)d * 4 + (size_t)(d / 64) * 148 + 128 * 4; }

// Token loads issued before the weights: words j = tid + 256 i, i < kXPre.
constexpr int kXPre = 2;
struct XRegs {
  v4u w[kXPre * 2];  // bf16: one 16-byte word per slot; fp32: two per slot
};

template <int ACT>
__device__ __forceinline__ void x_issue(const LayerArgs& a, int t, XRegs& R) {
  const int tid = threadIdx.x, W = a.d >> 3;
  const char* base = static_cast<const char*>(a.x) + (size_t)t * a.d * (ACT == 1 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < kXPre; ++i) {
    const int j = min(tid + kThreads * i, W - 1);
    if (ACT == 1) {
      R.w[i] = ldg<v4u>(base + (size_t)j * 16);
    } else {
      R.w[2 * i] = ldg<v4u>(base + (size_t)j * 32);
      R.w[2 * i + 1] = ldg<v4u>(base + (size_t)j * 32 + 16);
    }
  }
}

template <int ACT>
__device__ __forceinline__ void word_values(const LayerArgs& a, int t, const XRegs& R, int i, int j, float v[8]) {
  v4u p0, p1;
  if (i < kXPre) {
    p0 = R.w[ACT == 1 ? i : 2 * i];
    p1 = R.w[ACT == 1 ? i : 2 * i + 1];
  } else {  // words beyond the pre-issued ones (d > 4096)
    const char* base = static_cast<const char*>(a.x) + (size_t)t * a.d * (ACT == 1 ? 2 : 4);
    if (ACT == 1) {
      p0 = ldg<v4u>(base + (size_t)j * 16);
    } else {
      p0 = ldg<v4u>(base + (size_t)j * 32);
      p1 = ldg<v4u>(base + (size_t)j * 32 + 16);
    }
  }
  if (ACT == 1) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v[2 * m] = __uint_as_float(p0[m] << 16);
      v[2 * m + 1] = __uint_as_float(p0[m] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v[m] = __uint_as_float(p0[m]);
      v[4 + m] = __uint_as_float(p1[m]);
    }
  }
}

// Finish staging token t: optional rmsnorm (unit gain) + rounding to the
// activation type, then xf / xp / xs in LDS.  Called by all threads.
template <int ACT>
__device__ void x_commit(const LayerArgs& a, int t, const XRegs& R, const XStage& S) {
  const int tid = threadIdx.x;
  const int d = a.d, W = d >> 3;
  float inv = 1.f;
  if (a.rms) {
    float ss = 0.f;
    for (int i = 0, j = tid; j < W; ++i, j += kThreads) {
      float v[8];
      word_values<ACT>(a, t, R, i, j, v);
#pragma unroll
      for (int m = 0; m < 8; ++m) ss = fmaf(v[m], v[m], ss);
    }
    ss = xor_sum(ss, 1, 32);
    if ((tid & 63) == 0) S.red[tid >> 6] = ss;
    __syncthreads();
    inv = 1.0f / sqrtf(((S.red[0] + S.red[1]) + (S.red[2] + S.red[3])) / (float)d + a.eps);
  }
  for (int i = 0, j = tid; j < W; ++i, j += kThreads) {
    float v[8];
    word_values<ACT>(a, t, R, i, j, v);
    if (a.rms) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        v[m] *= inv;
        if (ACT == 1) v[m] = bf16_to_f32(f32_to_bf16(v[m]));
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) S.xf[8 * j + m] = v[m];
    if (ACT == 1) {
      v4u p;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        p[m] = (uint32_t)f32_to_bf16(v[m]) | ((uint32_t)f32_to_bf16(v[m + 4]) << 16);
      S.xp[(j >> 3) * 9 + (j & 7)] = p;
    }
    float part = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    part = xor_sum(part, 1, 4);  // the 8 words of one group sit in 8 consecutive lanes
    if ((j & 7) == 0) S.xs[j >> 3] = part;
  }
  __syncthreads();
}

// One 64-wide group: sum_c q_c * x_c (bf16 mode: sum_c (128+q_c) x_c).
template <int ACT>
__device__ __forceinline__ float group_dot(const v4u& q0, const v4u& q1, const XStage& S, int g) {
  float p = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const v4u q = h ? q1 : q0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w = q[m];
      const int word = g * 8 + h * 4 + m;
      if (ACT == 1) {
        const v4u xw = S.xp[g * 9 + h * 4 + m];
        uint32_t np[4];
        nib_pairs<kExpBf16>(w, np);
        p = dot2_bf16(np[0], xw[0], p);
        p = dot2_bf16(np[1], xw[1], p);
        p = dot2_bf16(np[2], xw[2], p);
        p = dot2_bf16(np[3], xw[3], p);
      } else {
        const float4 x0 = reinterpret_cast<const float4*>(S.xf)[word * 2];
        const float4 x1 = reinterpret_cast<const float4*>(S.xf)[word * 2 + 1];
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
        p = fmaf((float)(lo & 0xFFu), x0.x, p);
        p = fmaf((float)(hi & 0xFFu), x0.y, p);
        p = fmaf((float)((lo >> 8) & 0xFFu), x0.z, p);
        p = fmaf((float)((hi >> 8) & 0xFFu), x0.w, p);
        p = fmaf((float)((lo >> 16) & 0xFFu), x1.x, p);
        p = fmaf((float)((hi >> 16) & 0xFFu), x1.y, p);
        p = fmaf((float)(lo >> 24), x1.z, p);
        p = fmaf((float)(hi >> 24), x1.w, p);
      }
    }
  }
  return p;
}

// Group contribution s*sum(q x) + b*sum(x), with the magic offset folded in.
template <int ACT>
__device__ __forceinline__ float group_term(float p, uint32_t sb, float xsum, float offset) {
  const float s = f16_to_f32((uint16_t)(sb & 0xFFFFu));
  const float b = f16_to_f32((uint16_t)(sb >> 16));
  const float bb = (ACT == 1) ? b - offset * s : b;
  return fmaf(s, p, bb * xsum);
}

// Store one element of the intermediate activation vector a (position P of
// the token's [shared | expert 0 | ... | expert K-1] vector); fp16 words hold
// the pairs (P, P + 4) of each 8-aligned run.
template <int ACT>
__device__ __forceinline__ void store_a(void* abuf_t, int P, float v) {
  if (ACT == 1) {
    const int m = P & 7;
    st_dev(static_cast<uint16_t*>(abuf_t) + (P & ~7) + (m & 3) * 2 + (m >> 2), f32_to_f16(v));
  } else {
    st_dev(static_cast<float*>(abuf_t) + P, v);
  }
}

__device__ __forceinline__ char* abuf_of(const LayerArgs& a, int t, int act) {
  const int F = a.fs + a.K * a.f;
  return static_cast<char*>(a.abuf) + (size_t)t * F * (act == 1 ? 2 : 4);
}

// gate/up GEMV + SiLU*mul for rows ROWS*rb .. ROWS*rb+ROWS-1 (ROWS = 8 or
// 16) of one expert blob; the results go to positions apos + row of the
// activation vector.  Lane (r = tid % ROWS, jj = tid / ROWS) reads row r for
// the groups jj + JJ i (JJ = 256 / ROWS): each wavefront load covers eight
// whole 128-byte runs.  `xr` holds the token loads, issued by the caller
// before it waited on anything, so they overlap the weight fetch.  REPS
// (bf16 only): the ROWS results, tagged with `tag`, go to every copy of the
// fused kernel's activation vector in 16-byte stores, and the token is
// staged before the weights are requested (its loads went out long before):
// staging it after them would make the first product wait for every weight,
// as the wait for the token loads cannot be told apart from theirs.
// `staged`: the caller has staged the token already.
template <int ACT, int MAXI, int ROWS = 8, bool REPS = false>
__device__ void gate_up_block(const LayerArgs& a, int t, const uint8_t* blob, const BlobOffsets& o, int rb,
                              int apos, const XStage& S, const XRegs& xr, uint32_t tag = 0, bool staged = false) {
  constexpr int JJ = kThreads / ROWS;
  const int tid = threadIdx.x, r = tid % ROWS, jj = tid / ROWS;
  const int G = a.d >> 6;
  const int row = rb * ROWS + r;
  const int rb8 = row >> 3, r8 = row & 7;  // 8-row block of the packed layout
  const uint8_t* gq = blob + o.gq;
  const uint8_t* uq = blob + o.uq;
  const uint8_t* gsb = blob + o.gsb + ((size_t)rb8 * G * 8 + r8) * 4;  // + g * 32
  const uint8_t* usb = blob + o.usb + ((size_t)rb8 * G * 8 + r8) * 4;
  float accg = 0.f, accu = 0.f;
  if (REPS && !staged) x_commit<ACT>(a, t, xr, S);
  for (int base = 0; base < G; base += JJ * MAXI) {
    v4u qg0[MAXI], qg1[MAXI], qu0[MAXI], qu1[MAXI];
    uint32_t sg[MAXI], su[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int g = min(base + jj + JJ * i, G - 1);
      const size_t off = (((size_t)rb8 * G + g) * 2) * 128 + r8 * 16;
      qg0[i] = ldg<v4u>(gq + off);
      qg1[i] = ldg<v4u>(gq + off + 128);
      qu0[i] = ldg<v4u>(uq + off);
      qu1[i] = ldg<v4u>(uq + off + 128);
      sg[i] = ldg<uint32_t>(gsb + g * 32);
      su[i] = ldg<uint32_t>(usb + g * 32);
    }
    if (!REPS && !staged && base == 0) x_commit<ACT>(a, t, xr, S);
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int g = base + jj + JJ * i;
      if (g < G) {
        accg += group_term<ACT>(group_dot<ACT>(qg0[i], qg1[i], S, g), sg[i], S.xs[g], 128.f);
        accu += group_term<ACT>(group_dot<ACT>(qu0[i], qu1[i], S, g), su[i], S.xs[g], 128.f);
      }
    }
  }
  accg = xor_sum(accg, ROWS, 32);  // lanes r, r + ROWS, ... of a wavefront
  accu = xor_sum(accu, ROWS, 32);
  if ((tid & 63) < ROWS) {
    S.red[(tid >> 6) * 2 * ROWS + r * 2] = accg;
    S.red[(tid >> 6) * 2 * ROWS + r * 2 + 1] = accu;
  }
  __syncthreads();
  if (tid < ROWS) {
    constexpr int W = 2 * ROWS;  // one wavefront's partials
    const float gsum = (S.red[r * 2] + S.red[W + r * 2]) + (S.red[2 * W + r * 2] + S.red[3 * W + r * 2]);
    const float usum =
        (S.red[r * 2 + 1] + S.red[W + r * 2 + 1]) + (S.red[2 * W + r * 2 + 1] + S.red[3 * W + r * 2 + 1]);
    const float v = silu(gsum) * usum;
    if (ACT == 1 && !(fabsf(v) < kF16HandoffMax)) atomicOr(a.err, kErrRange);
    if (REPS) {  // S.xf is free: the bf16 products read S.xp
      const int m = r & 7;
      reinterpret_cast<uint16_t*>(S.xf)[(r & ~7) + (m & 3) * 2 + (m >> 2)] = f32_to_f16_tagged(v, tag);
    } else {
      store_a<ACT>(abuf_of(a, t, ACT), apos + row, v);
    }
  }
  if (REPS) {
    __syncthreads();
    constexpr int CH = ROWS / 8;  // 16-byte words of this row block
    if (tid < CH * kAReps) {
      const int c = tid % CH, q = tid / CH;
      const size_t off = (size_t)q * a_rep_stride(a.fs + a.K * a.f) + (size_t)(apos + rb * ROWS) * 2 + c * 16;
      st_dev16(buf_rsrc(a.arep), (uint32_t)off, reinterpret_cast<const v4u*>(S.xf)[c]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the copies land before the arrival: consumers then read them once
  }
}

// Copy the logits of token t into LDS with straight-line loads (E <= 1024),
// ending with a workgroup barrier.  `nthreads` threads take part.
template <int NTH>
__device__ __forceinline__ void stage_logits(const LayerArgs& a, int t, float* s_logits) {
  const float* lt = a.logits + (size_t)t * a.E;
  constexpr int N = (1024 + NTH - 1) / NTH;
  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = ldg<float>(lt + min((int)threadIdx.x + NTH * i, a.E - 1));
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int e = threadIdx.x + NTH * i;
    if (e < a.E) s_logits[e] = v[i];
  }
  __syncthreads();
}

// ---------------------------------------------------------------- kernel A
constexpr int kRouterPre = 8;  // 16-byte router chunks per lane issued up front (d <= 8192)
constexpr int kWaves = kThreads / 64;

// Logit of router row e for token t by one wavefront (rows e >= E repeat
// row E-1); every lane returns it.  The row's scale and bias are loaded with
// the weights, before the token is waited for.
template <int ACT>
__device__ float router_row(const LayerArgs& a, int t, int e, const XStage& S) {
  const int lane = threadIdx.x & 63;
  const int ec = min(e, a.E - 1);
  const int NC = a.d >> 4;  // 16-byte chunks per router row
  const int8_t* wrow = a.router_w + (size_t)ec * a.d;
  XRegs xr;
  x_issue<ACT>(a, t, xr);
  v4u wr[kRouterPre];
#pragma unroll
  for (int i = 0; i < kRouterPre; ++i) wr[i] = ldg<v4u>(wrow + (size_t)min(lane + 64 * i, NC - 1) * 16);
  const float s = f16_to_f32(ldg<uint16_t>(a.router_scale + ec));
  const float b = a.router_bias ? ldg<float>(a.router_bias + ec) : 0.f;
  x_commit<ACT>(a, t, xr, S);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kRouterPre; ++i) {
    const int c = lane + 64 * i;
    if (c < NC) {
      const float4* xv = reinterpret_cast<const float4*>(S.xf + c * 16);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float4 xx = xv[m];
        const int w = (int)wr[i][m];
        acc = fmaf((float)((w << 24) >> 24), xx.x, acc);
        acc = fmaf((float)((w << 16) >> 24), xx.y, acc);
        acc = fmaf((float)((w << 8) >> 24), xx.z, acc);
        acc = fmaf((float)(w >> 24), xx.w, acc);
      }
    }
  }
  acc = wave_sum_f32(acc);  // every lane holds the same sum (DPP, fixed order)
  return fmaf(s, acc, b);
}

// Workgroups of the router part of a route_shared launch (none when the
// launch runs the shared gate/up alone).
__host__ __device__ inline int route_blocks(const LayerArgs& a) {
  return (a.stages == 0 || (a.stages & kStageRouter)) ? (a.E + kWaves - 1) / kWaves : 0;
}

template <int ACT, int MAXI>
__global__ __launch_bounds__(kThreads) void route_shared_kernel(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const XStage S = carve_x(smem, a.d);
  const int t = blockIdx.y;
  const int NR = route_blocks(a);  // one router row per wavefront
  if ((int)blockIdx.x >= NR) {
    XRegs xr;
    x_issue<ACT>(a, t, xr);
    gate_up_block<ACT, MAXI>(a, t, a.shared_blob, a.so, blockIdx.x - NR, 0, S, xr);
    return;
  }
  const int e = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const float v = router_row<ACT>(a, t, e, S);
  if (e < a.E && (threadIdx.x & 63) == 0) a.logits[(size_t)t * a.E + e] = v;
}

// Stand-alone top-K (one wavefront per token), used when the routing must be
// known before the expert kernels are enqueued.
template <int NE>
__global__ __launch_bounds__(64) void topk_kernel(LayerArgs a) {
  __shared__ uint32_t scratch[128];
  __shared__ float s_logits[1024];
  stage_logits<64>(a, blockIdx.x, s_logits);
  int id;
  float w;
  topk_wave<NE>(a, blockIdx.x, s_logits, &id, &w, scratch);
  publish_routing(a, blockIdx.x, threadIdx.x, id, w);
}

// ---------------------------------------------------------------- kernel B
// Routed gate/up, workgroups in this order:
//   - with the top-K done here (topk_in_gate_up): one workgroup that runs it
//     for the token and publishes ids, weights and chosen addresses for the
//     down kernel (and, for a one-token streamed call, the ids and then the
//     sequence number into host memory), first so it is dispatched first;
//   - the shared expert's fs/8 (shared_in_routed), which need no routing;
//   - f/8 workgroups of 8 rows per chosen slot (all K slots, or the slots of
//     run_mask).
// Each slot's expert blob comes from the top-K run by the workgroup itself
// (then from expert_base, or from the device expert table), from the table
// through the published ids (sel_from_table), or from sel_addr.
template <int ACT, int MAXI, int NE>
__global__ __launch_bounds__(kThreads) void routed_gu_kernel(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  __shared__ uint32_t scratch[128];
  __shared__ float s_logits[1024];
  const XStage S = carve_x(smem, a.d);
  const int t = blockIdx.y;
  int b = blockIdx.x;
  if (a.topk_in_gate_up) {
    if (b == 0) {
      stage_logits<kThreads>(a, t, s_logits);
      if (threadIdx.x < 64) {
        int id;
        float w;
        topk_wave<NE>(a, t, s_logits, &id, &w, scratch);
        publish_routing(a, t, threadIdx.x, id, w);
        if (a.host_ids && threadIdx.x < a.K)
          __hip_atomic_store(a.host_ids + threadIdx.x, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      if (a.host_ids) {  // the sequence number after every id
        __syncthreads();
        if (threadIdx.x == 0)
          __hip_atomic_store(a.host_flag, a.host_seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      return;
    }
    --b;
  }
  const int NS = a.shared_in_routed ? a.fs >> 3 : 0;
  if (b < NS) {  // the shared expert's gate/up: no routing needed
    XRegs xr;
    x_issue<ACT>(a, t, xr);
    gate_up_block<ACT, MAXI>(a, t, a.shared_blob, a.so, b, 0, S, xr);
    return;
  }
  b -= NS;
  const int RB = a.f >> 3;
  const int j = b / RB, rb = b - j * RB;
  int k = j;
  if (a.run_mask) {  // one token, some slots only: k = the j-th set bit
    uint32_t m = a.run_mask;
    for (int i = 0; i < j; ++i) m &= m - 1u;
    k = __builtin_ctz(m);
  }
  XRegs xr;
  x_issue<ACT>(a, t, xr);
  const uint8_t* blob;
  if (a.topk_in_gate_up) {  // every workgroup finds its expert itself
    stage_logits<kThreads>(a, t, s_logits);
    if (threadIdx.x < 64) {
      const int id = topk_kth<NE>(a, t, s_logits, k);
      if (threadIdx.x == 0) scratch[0] = (uint32_t)id;
    }
    __syncthreads();
    const uint32_t id = scratch[0];
    if (a.sel_from_table) {  // streamed experts: a zero address marks one that is not cached
      const uint64_t addr = a.expert_addr[id];
      if (a.hits_only && addr == 0) return;  // the host launches it again behind its fill
      blob = reinterpret_cast<const uint8_t*>(addr);
    } else {
      blob = a.expert_base + (size_t)id * a.expert_stride;
    }
  } else if (a.sel_from_table) {  // streamed experts: the table was brought up to date after the routing
    const size_t o = (size_t)t * a.K + k;
    const uint64_t addr = a.expert_addr[a.ids[o]];
    if (a.hits_only && addr == 0) return;  // not cached: the host launches it again behind its fill
    if (rb == 0 && threadIdx.x == 0) a.sel_addr[o] = addr;  // for the down kernel, which runs after this one
    blob = reinterpret_cast<const uint8_t*>(addr);
  } else {
    blob = reinterpret_cast<const uint8_t*>(a.sel_addr[(size_t)t * a.K + k]);
  }
  if (blob == nullptr) {  // expert not resident: flag it and read the zero blob
    if (threadIdx.x == 0) atomicOr(a.err, kErrMissingExpert);
    blob = a.zero_blob;
  }
  gate_up_block<ACT, MAXI>(a, t, blob, a.ro, rb, a.fs + k * a.f, S, xr);
}

// ---------------------------------------------------------------- kernel C
// The activation vector sits in LDS as [group][WPG + 1] 16-byte words (WPG =
// 8 fp16 or 16 fp32 words per 64-wide group, plus one pad word): the 8 groups
// a wavefront reads at once then start in different LDS banks.
__host__ __device__ constexpr int a_words(int act) { return act == 1 ? 8 : 16; }
__host__ __device__ inline size_t down_lds_bytes(int F, int NI, int K, int act) {
  (void)F;
  return (size_t)NI * (a_words(act) + 1) * 16 + (size_t)NI * 4 + (size_t)K * 4 + 40 * 4;
}
__device__ __forceinline__ int a_slot(int j, int wpg) { return (j / wpg) * (wpg + 1) + j % wpg; }

constexpr int kAPre = 4;  // 16-byte activation words per thread held in registers for staging

// asum[i] = sum of the 64 values of group i of the staged activation vector
// (as the down projection reads them), ending with a workgroup barrier.
template <int ACT>
__device__ __forceinline__ void group_sums(const char* lds_a, float* asum, int NI) {
  constexpr int WPG = a_words(ACT);  // 16-byte words per group, in consecutive lanes
  for (int i = threadIdx.x; i < NI * WPG; i += kThreads) {
    const v4u w = reinterpret_cast<const v4u*>(lds_a)[a_slot(i, WPG)];
    float s;
    if (ACT == 1) {
      float h[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        h[2 * m] = f16_to_f32((uint16_t)(w[m] & 0xFFFFu));
        h[2 * m + 1] = f16_to_f32((uint16_t)(w[m] >> 16));
      }
      s = ((h[0] + h[1]) + (h[2] + h[3])) + ((h[4] + h[5]) + (h[6] + h[7]));
    } else {
      s = (__uint_as_float(w[0]) + __uint_as_float(w[1])) + (__uint_as_float(w[2]) + __uint_as_float(w[3]));
    }
    s = xor_sum(s, 1, WPG / 2);
    if ((i & (WPG - 1)) == 0) asum[i / WPG] = s;
  }
  __syncthreads();
}

// Down GEMV of the shared and chosen experts for output rows 8*rb..8*rb+7 of
// token t and the weighted combine.  sel[k] / wk_src[k]: blob address and
// weight of the k-th chosen expert.  The activation vector is complete, so
// its loads go out before the weights.
template <int ACT, int MAXI>
__device__ void down_block(const LayerArgs& a, int t, int rb, const uint64_t* sel, const float* wk_src,
                           char* smem) {
  const int tid = threadIdx.x, r = tid & 7, jj = tid >> 3;
  const int row = rb * 8 + r;
  const int Gs = a.fs >> 6, Gf = a.f >> 6, K = a.K;
  const int NI = Gs + K * Gf;
  const int F = a.fs + K * a.f;
  constexpr int WPG = a_words(ACT);
  char* lds_a = smem;
  float* asum = reinterpret_cast<float*>(smem + (size_t)NI * (WPG + 1) * 16);
  float* wk = asum + NI;
  float* red = wk + K;
  const char* abuf_t = abuf_of(a, t, ACT);
  const int NW = F * (ACT == 1 ? 2 : 4) / 16;  // 16-byte words of the activation vector
  v4u ar[kAPre];
#pragma unroll
  for (int i = 0; i < kAPre; ++i) ar[i] = ldg<v4u>(abuf_t + (size_t)min(tid + kThreads * i, NW - 1) * 16);
  float acc = 0.f;
  for (int base = 0; base < NI; base += 32 * MAXI) {
    v4u q0[MAXI], q1[MAXI];
    uint32_t sb[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int it = min(base + jj + 32 * i, NI - 1);
      const uint8_t* blob;
      int G, g;
      uint32_t oq, osb;
      if (it < Gs) {
        blob = a.shared_blob; G = Gs; g = it; oq = a.so.dq; osb = a.so.dsb;
      } else {
        const int k = (it - Gs) / Gf;
        g = (it - Gs) - k * Gf;
        G = Gf;
        blob = reinterpret_cast<const uint8_t*>(sel[k]);
        if (blob == nullptr) blob = a.zero_blob;  // flagged by the gate/up kernel
        oq = a.ro.dq; osb = a.ro.dsb;
      }
      const size_t off = (((size_t)rb * G + g) * 2) * 128 + r * 16;
      q0[i] = ldg<v4u>(blob + oq + off);
      q1[i] = ldg<v4u>(blob + oq + off + 128);
      sb[i] = ldg<uint32_t>(blob + osb + (((size_t)rb * G + g) * 8 + r) * 4);
    }
    if (base == 0) {
#pragma unroll
      for (int i = 0; i < kAPre; ++i) {
        const int j = tid + kThreads * i;
        if (j < NW) reinterpret_cast<v4u*>(lds_a)[a_slot(j, WPG)] = ar[i];
      }
      for (int j = tid + kThreads * kAPre; j < NW; j += kThreads)
        reinterpret_cast<v4u*>(lds_a)[a_slot(j, WPG)] = ldg<v4u>(abuf_t + (size_t)j * 16);
      if (tid < K) wk[tid] = wk_src[tid];
      __syncthreads();
      group_sums<ACT>(lds_a, asum, NI);
    }
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int it = base + jj + 32 * i;
      if (it < NI) {
        float p = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v4u q = h ? q1[i] : q0[i];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t w = q[m];
            if (ACT == 1) {
              const v4u av = reinterpret_cast<const v4u*>(lds_a)[it * 9 + h * 4 + m];
              uint32_t np[4];
              nib_pairs<kExpF16>(w, np);
              p = dot2_f16(np[0], av[0], p);
              p = dot2_f16(np[1], av[1], p);
              p = dot2_f16(np[2], av[2], p);
              p = dot2_f16(np[3], av[3], p);
            } else {
              const float4 x0 = reinterpret_cast<const float4*>(lds_a)[it * 17 + (h * 4 + m) * 2];
              const float4 x1 = reinterpret_cast<const float4*>(lds_a)[it * 17 + (h * 4 + m) * 2 + 1];
              const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
              p = fmaf((float)(lo & 0xFFu), x0.x, p);
              p = fmaf((float)(hi & 0xFFu), x0.y, p);
              p = fmaf((float)((lo >> 8) & 0xFFu), x0.z, p);
              p = fmaf((float)((hi >> 8) & 0xFFu), x0.w, p);
              p = fmaf((float)((lo >> 16) & 0xFFu), x1.x, p);
              p = fmaf((float)((hi >> 16) & 0xFFu), x1.y, p);
              p = fmaf((float)(lo >> 24), x1.z, p);
              p = fmaf((float)(hi >> 24), x1.w, p);
            }
          }
        }
        const float term = group_term<ACT>(p, sb[i], asum[it], 1024.f);
        const float wgt = (it < Gs) ? 1.f : wk[(it - Gs) / Gf];
        acc = fmaf(wgt, term, acc);
      }
    }
  }
  acc = xor_sum(acc, 8, 32);
  if ((tid & 63) < 8) red[(tid >> 6) * 8 + r] = acc;
  __syncthreads();
  if (tid < 8) {
    const float y = (red[r] + red[8 + r]) + (red[16 + r] + red[24 + r]);
    const size_t o = (size_t)t * a.d + row;
    if (ACT == 1) {
      float v = y;
      if (a.resid) v += bf16_to_f32(static_cast<const uint16_t*>(a.resid)[o]);
      static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(v);
    } else {
      float v = y;
      if (a.resid) v += static_cast<const float*>(a.resid)[o];
      static_cast<float*>(a.out)[o] = v;
    }
  }
}

template <int ACT, int MAXI>
__global__ __launch_bounds__(kThreads) void down_combine_kernel(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int t = blockIdx.y;
  if (a.hits_only) {  // queued before the cache step: runs when every chosen expert was cached
    const int lane = threadIdx.x & 63;  // (every wavefront reads the same words: one decision per workgroup)
    const bool miss = lane < a.K && a.expert_addr[a.ids[(size_t)t * a.K + lane]] == 0;
    if (__ballot(miss)) return;
  }
  down_block<ACT, MAXI>(a, t, blockIdx.x, a.sel_addr + (size_t)t * a.K, a.wts + (size_t)t * a.K, smem);
}

// ---------------------------------------------------------------- fused layer
// One launch per batch-1 bf16 layer on resident experts.  Workgroups, in
// block order: router rows | shared gate/up | routed gate/up | down+combine;
// gate/up workgroups take 16 rows.  A workgroup only waits for results of
// lower-numbered workgroups, and workgroups are dispatched in block order, so
// the lowest unfinished workgroup can always run: no deadlock even when the
// grid does not fit the GPU at once.  Waits are bounded spins (a timeout
// raises an error flag and the workgroup carries on).
//
// Hand-offs go through counters that only grow.  Each launch has a tag (the
// launch count + 1, read from an epoch word); a stage is complete when its
// counter has grown by its number of producer workgroups to tag * members.
// A producer issues its results as tagged device-scope stores and, without
// waiting for them, adds one to part (its index mod 8) of the counter, in all
// 8 replicas of that part; a consumer polls the 8 parts of its replica with 8
// lanes of one wavefront, then reads the data, re-reading any word that still
// carries an old tag.
//   router rows    -> logits (64 replicas of the table)     + router counter
//   shared gate/up -> shared part of the activation vector  + shared counter
//   routed gate/up -> routed part of the activation vector  + routed counter
// Routed gate/up and down workgroups run the top-K themselves on the staged
// logits.  Down workgroups fetch the shared expert's down weights at once and
// the chosen experts' as soon as the routing is known.  They are also the
// last to need the tag: each counts itself once it has seen the routed
// counter complete, and that count is where every workgroup of the next
// launch reads its tag from (launch_tag), so nothing is reset between
// launches and nothing waits for an atomic's result.  Every counter word has
// its own cache lines (4160 bytes apart).
constexpr int kSyncStride = 4160 / 4;  // words between counter words
constexpr int kParts = 8;  // a stage counter is split in parts: producer i adds to part i % kParts
constexpr int kReps = 8;   // each part is kept in replicas: a consumer polls replica (workgroup % kReps)
constexpr int kLogitReplicas = 64;
// Counter 0 is free: the routing needs no counter, its logits carry the full
// launch tag and readers re-read stale entries.
enum : int { kCntShared = 1, kCntRouted = 2, kCntDone = 3, kNumCnt = 4 };
constexpr int kSyncSlots = kNumCnt * kParts * kReps;

// Logit table entries: tag << 32 | fp32 bits.  Entries between replicas (the
// table rounded up to 4 KB, so 4-entry runs of the last router rows fit, plus
// 64 bytes to spread the replicas over channels).
__host__ __device__ inline size_t logit_rep_stride(int E) { return ((size_t)E * 8 + 4095) / 4096 * 512 + 8; }
__host__ __device__ inline size_t sync_area_bytes(int E) {
  return (size_t)kSyncSlots * kSyncStride * 4 + (size_t)kLogitReplicas * logit_rep_stride(E) * 8;
}

__device__ __forceinline__ uint32_t* sync_slot(uint32_t* area, int slot) {
  return area + (size_t)slot * kSyncStride;
}
__device__ __forceinline__ uint32_t* counter_rep(uint32_t* area, int c, int part, int r) {
  return sync_slot(area, (c * kParts + part) * kReps + r);
}

// Called by every thread once the workgroup's tagged device-scope stores have
// been issued: producer i of a stage adds one to every replica of part
// i % kParts of the stage's counter (lanes 0..kReps-1, no return value).
// Atomics and polls on one address queue where they are performed, so each
// address sees 1/kParts of the arrivals and 1/kReps of the pollers.  The
// stores are not waited for: a consumer that sees the counter complete reads
// the data and re-reads any word whose tag is not yet this launch's.
__device__ __forceinline__ void arrive(uint32_t* area, int c, int i) {
  __syncthreads();
  if (threadIdx.x < kReps)
    __hip_atomic_fetch_add(counter_rep(area, c, i % kParts, threadIdx.x), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Lanes 0..kParts-1 poll the parts of counter c of a stage with n producers
// (replica workgroup % kReps) until each part has grown to tag * (its number
// of producers) (wrap-safe), pausing about 64 * SLEEP cycles between rounds;
// ends with a workgroup barrier.
template <int SLEEP>
__device__ __forceinline__ void wait_count(const LayerArgs& a, uint32_t* area, int c, uint32_t tag, int n) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    bool pending = lane < kParts && lane < n;
    const uint32_t target = tag * (uint32_t)((n - lane + kParts - 1) / kParts);
    const uint32_t* p = counter_rep(area, c, min(lane, kParts - 1), blockIdx.x % kReps);
    if (pending) pending = (int32_t)(ld_dev(p) - target) < 0;
    for (uint32_t it = 0; __ballot(pending) != 0; ++it) {
      if (it == kSpinLimit) {
        if (lane == 0) atomicOr(a.err, kErrSyncTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(SLEEP);
      if (pending) pending = (int32_t)(ld_dev(p) - target) < 0;
    }
  }
  __syncthreads();
}

// Copy the logits of this launch from replica `rep` (the router counter was
// seen complete) into LDS with device-coherent loads, re-reading entries
// whose tag is still a previous launch's; ends with a workgroup barrier.
template <int NE>
__device__ __forceinline__ void stage_logits_dev(const LayerArgs& a, const uint64_t* rep, uint32_t tag,
                                                 float* s_logits) {
  constexpr int N = (64 * NE + kThreads - 1) / kThreads;
  uint64_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = ld_dev(rep + min((int)threadIdx.x + kThreads * i, a.E - 1));
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int e = threadIdx.x + kThreads * i;
    if (e < a.E) {
      for (uint32_t it = 0; (uint32_t)(v[i] >> 32) != tag; ++it) {
        if (it == kSpinLimit) {
          atomicOr(a.err, kErrSyncTimeout);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        v[i] = ld_dev(rep + e);
      }
      s_logits[e] = __uint_as_float((uint32_t)v[i]);
    }
  }
  __syncthreads();
}

// The launch tag comes from a 64-bit count of down workgroups that have
// passed their last wait (8 parts, replica 0; part i % 8 for down workgroup
// i).  A down workgroup passes it only after every other workgroup of the
// launch has started and read the count (shared and routed workgroups arrive
// on the counters it waits for; it has itself read every router workgroup's
// logits, which carry the tag the router read), and the count
// cannot reach the next multiple of nd before every down workgroup, the
// reader included, has passed.  So every workgroup of launch n reads a total
// in [(n-1) nd, n nd) and takes tag = total / nd + 1 = n, with no reset
// between launches and no atomic whose result anyone waits for.  Called by
// whole wavefronts (lanes 0..7 load the parts).
__device__ __forceinline__ uint32_t launch_tag(uint32_t* area, int nd) {
  const int lane = threadIdx.x & 63;
  uint64_t v = lane < kParts
                   ? ld_dev(reinterpret_cast<const uint64_t*>(counter_rep(area, kCntDone, lane, 0)))
                   : 0ull;
#pragma unroll
  for (int m = 1; m < kParts; m <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    v += ((uint64_t)hi << 32) | lo;
  }
  const uint64_t total = ((uint64_t)__shfl((uint32_t)(v >> 32), 0, 64) << 32) | __shfl((uint32_t)v, 0, 64);
  return (uint32_t)(total / (uint64_t)nd) + 1u;
}
// Down workgroup i has passed its last wait of this launch (one atomic, no
// return value).
__device__ __forceinline__ void count_done(uint32_t* area, int i) {
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(counter_rep(area, kCntDone, i % kParts, 0)), 1ull,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kFusedGuRows = 16;  // gate/up rows per workgroup of the fused kernel

// Workgroups whose weight fetch does not wait for the routing (shared gate/up,
// the shared part of the down projection) hold it back for about 3 us (the
// router's time), so that the router's loads, on the critical path, do not
// queue behind megabytes of weights in the memory controllers; the shared
// weights then stream while the routing is handed off.  Measured on the
// d_model 2816 / 128-expert layer: 0 -> 18.8 us per token, 3 us -> 18.3 us,
// 4 us or more -> slower again.
#ifndef MOE_FUSED_BULK_DELAY
#define MOE_FUSED_BULK_DELAY 14
#endif
__device__ __forceinline__ void bulk_delay() {
  for (int i = 0; i < MOE_FUSED_BULK_DELAY; ++i) __builtin_amdgcn_s_sleep(8);  // 512 cycles each
}

__host__ __device__ inline int fused_groups(int E, int K, int d, int f, int fs, int* NR, int* NS, int* NG, int* ND) {
  *NR = (E + kWaves - 1) / kWaves;
  *NS = fs / kFusedGuRows;
  *NG = K * (f / kFusedGuRows);
  *ND = d / 8;
  return *NR + *NS + *NG + *ND;
}

// Stage groups [g0, g1) of the activation vector (written by other
// workgroups of this launch, parity-tagged) into LDS from this workgroup's
// copy with device-coherent loads, re-reading words that still carry the
// previous launch's parity and clearing the parity bits; then their group
// sums.  Ends with a workgroup barrier.
__device__ __forceinline__ void stage_a_coherent(const LayerArgs& a, char* lds_a, float* asum, int g0, int g1,
                                                 uint32_t tag) {
  constexpr int WPG = a_words(1);
  const int tid = threadIdx.x;
  const uint32_t par = (tag & 1u) * 0x00010001u;
  const auto rs = buf_rsrc(a.arep);
  const uint32_t base = (uint32_t)((blockIdx.x % kAReps) * a_rep_stride(a.fs + a.K * a.f) + (size_t)g0 * 64 * 2);
  const int nw = (g1 - g0) * WPG;  // 16-byte words
  constexpr int kAD = 4;
  for (int j0 = 0; j0 < nw; j0 += kThreads * kAD) {
    v4u v[kAD];
#pragma unroll
    for (int i = 0; i < kAD; ++i) v[i] = ld_dev16(rs, base + (uint32_t)min(j0 + tid + kThreads * i, nw - 1) * 16);
#pragma unroll
    for (int i = 0; i < kAD; ++i) {
      const int j = j0 + tid + kThreads * i;
      if (j < nw) {
        for (uint32_t it = 0; !fresh4(v[i], par); ++it) {
          if (it == kSpinLimit) {
            atomicOr(a.err, kErrSyncTimeout);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          v[i] = ld_dev16(rs, base + (uint32_t)j * 16);
        }
        v4u p;
#pragma unroll
        for (int m = 0; m < 4; ++m) p[m] = v[i][m] & 0xFFFEFFFEu;
        reinterpret_cast<v4u*>(lds_a)[a_slot(g0 * WPG + j, WPG)] = p;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < (g1 - g0) * WPG; i += kThreads) {
    const v4u x = reinterpret_cast<const v4u*>(lds_a)[a_slot(g0 * WPG + i, WPG)];
    float h[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      h[2 * m] = f16_to_f32((uint16_t)(x[m] & 0xFFFFu));
      h[2 * m + 1] = f16_to_f32((uint16_t)(x[m] >> 16));
    }
    float sum = ((h[0] + h[1]) + (h[2] + h[3])) + ((h[4] + h[5]) + (h[6] + h[7]));
    sum = xor_sum(sum, 1, WPG / 2);
    if ((i & (WPG - 1)) == 0) asum[g0 + i / WPG] = sum;
  }
  __syncthreads();
}

// Down workgroup of output rows 8*rb..8*rb+7 of the fused kernel: the shared
// expert's groups [0, Gs) as soon as the shared gate/up is done, then the
// chosen experts' groups [Gs, NI) once the routed gate/up is done.  Lane
// (r = tid & 7, jj = tid >> 3) owns row r and the groups jj + 32 i of each
// part; SS shared and SR routed weight slots.  The shared slots are loaded at
// once, the routed ones as soon as the routing is known.
template <int SS, int SR, int NE>
__device__ void down_fused(const LayerArgs& a, int rb, int nd, uint32_t members_shared,
                           uint32_t members_routed, const uint64_t* lrep, char* smem, float* s_logits,
                           uint32_t* scratch, uint64_t* s_sel, float* s_w) {
  const int tid = threadIdx.x, r = tid & 7, jj = tid >> 3;
  uint32_t* area = a.counter;
  const uint32_t tag = launch_tag(area, nd);
  const int Gs = a.fs >> 6, Gf = a.f >> 6;
  const int NI = Gs + a.K * Gf, NRG = NI - Gs;
  constexpr int WPG = a_words(1);
  char* lds_a = smem;
  float* asum = reinterpret_cast<float*>(smem + (size_t)NI * (WPG + 1) * 16);
  float* red = asum + NI;
  v4u q0[SS + SR], q1[SS + SR];
  uint32_t sb[SS + SR];
  auto load_slot = [&](int s, const uint8_t* blob, int G, int g, uint32_t oq, uint32_t osb) {
    const size_t off = (((size_t)rb * G + g) * 2) * 128 + r * 16;
    q0[s] = ldg<v4u>(blob + oq + off);
    q1[s] = ldg<v4u>(blob + oq + off + 128);
    sb[s] = ldg<uint32_t>(blob + osb + (((size_t)rb * G + g) * 8 + r) * 4);
  };
  bulk_delay();
#pragma unroll
  for (int s = 0; s < SS; ++s) load_slot(s, a.shared_blob, Gs, min(jj + 32 * s, Gs - 1), a.so.dq, a.so.dsb);
  // routing: the tagged logits are read as they arrive (no counter round trip)
  stage_logits_dev<NE>(a, lrep, tag, s_logits);
  if (threadIdx.x < 64) {
    int id;
    float w;
    topk_wave<NE>(a, 0, s_logits, &id, &w, scratch);
    if (threadIdx.x < a.K) {
      s_sel[threadIdx.x] = reinterpret_cast<uint64_t>(a.expert_base + (size_t)id * a.expert_stride);
      s_w[threadIdx.x] = w;
    }
    if (rb == 0) publish_routing(a, 0, threadIdx.x, id, w);
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < SR; ++s) {
    const int c = min(jj + 32 * s, NRG - 1);
    const int k = c / Gf;
    load_slot(SS + s, reinterpret_cast<const uint8_t*>(s_sel[k]), Gf, c - k * Gf, a.ro.dq, a.ro.dsb);
  }
  float acc = 0.f;
  auto accumulate = [&](int s, int it) {
    float pp = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4u q = h ? q1[s] : q0[s];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w = q[m];
        const v4u av = reinterpret_cast<const v4u*>(lds_a)[it * (WPG + 1) + h * 4 + m];
        uint32_t np[4];
        nib_pairs<kExpF16>(w, np);
        pp = dot2_f16(np[0], av[0], pp);
        pp = dot2_f16(np[1], av[1], pp);
        pp = dot2_f16(np[2], av[2], pp);
        pp = dot2_f16(np[3], av[3], pp);
      }
    }
    const float term = group_term<1>(pp, sb[s], asum[it], 1024.f);
    const float wgt = (it < Gs) ? 1.f : s_w[(it - Gs) / Gf];
    acc = fmaf(wgt, term, acc);
  };
  if (SS > 0) {  // shared part
    wait_count<4>(a, area, kCntShared, tag, (int)members_shared);
    stage_a_coherent(a, lds_a, asum, 0, Gs, tag);
#pragma unroll
    for (int s = 0; s < SS; ++s)
      if (jj + 32 * s < Gs) accumulate(s, jj + 32 * s);
  }
  wait_count<2>(a, area, kCntRouted, tag, (int)members_routed);
  // the residual row, loaded with the activations and parked in LDS (in
  // place of a load whose latency would come at the very end)
  uint32_t hres = 0;
  if (tid < 8 && a.resid) hres = (uint32_t)ldg<uint16_t>(static_cast<const uint16_t*>(a.resid) + rb * 8 + r) << 16;
  stage_a_coherent(a, lds_a, asum, Gs, NI, tag);
  if (tid < 8) red[32 + r] = __uint_as_float(hres);
  count_done(area, rb);  // after the staging: its loads would otherwise also wait for this atomic
#pragma unroll
  for (int s = 0; s < SR; ++s)
    if (jj + 32 * s < NRG) accumulate(SS + s, Gs + jj + 32 * s);
  acc = xor_sum(acc, 8, 32);
  if ((tid & 63) < 8) red[(tid >> 6) * 8 + r] = acc;
  __syncthreads();
  if (tid < 8) {
    const float y = (red[r] + red[8 + r]) + (red[16 + r] + red[24 + r]);
    const int row = rb * 8 + r;
    float v = y;
    if (a.resid) v += red[32 + r];
    static_cast<uint16_t*>(a.out)[row] = f32_to_bf16(v);
  }
}

template <int MAXI, int NE, int SS, int SR>
__global__ __launch_bounds__(kThreads, 4) void fused_layer_kernel(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  __shared__ uint32_t scratch[128];
  __shared__ float s_logits[64 * NE];
  __shared__ uint64_t s_sel[64];
  __shared__ float s_w[64];
  int NR, NS, NG, ND;
  fused_groups(a.E, a.K, a.d, a.f, a.fs, &NR, &NS, &NG, &ND);
  const int b = blockIdx.x;
  uint32_t* area = a.counter;
  uint64_t* lrep = reinterpret_cast<uint64_t*>(area + (size_t)kSyncSlots * kSyncStride);
  const size_t rstride = logit_rep_stride(a.E);
  const uint64_t* my_rep = lrep + (size_t)(b % kLogitReplicas) * rstride;
  const XStage S = carve_x(smem, a.d);
  if (b < NR) {
    __builtin_amdgcn_s_setprio(2);  // on the critical path: ahead of the streaming wavefronts
    const uint32_t tag = launch_tag(area, ND);
    const float v = router_row<1>(a, 0, b * kWaves + (threadIdx.x >> 6), S);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x < kLogitReplicas) {  // lane j: the 4 tagged logits of this workgroup into replica j
      const size_t off = ((size_t)threadIdx.x * rstride + (size_t)b * kWaves) * 8;
      const auto rs = buf_rsrc(lrep);
      st_dev16(rs, (uint32_t)off, v4u{__float_as_uint(s_w[0]), tag, __float_as_uint(s_w[1]), tag});
      st_dev16(rs, (uint32_t)off + 16, v4u{__float_as_uint(s_w[2]), tag, __float_as_uint(s_w[3]), tag});
    }
  } else if (b < NR + NS) {
    const uint32_t tag = launch_tag(area, ND);
    XRegs xr;
    x_issue<1>(a, 0, xr);
    bulk_delay();
    gate_up_block<1, MAXI, kFusedGuRows, true>(a, 0, a.shared_blob, a.so, b - NR, 0, S, xr, tag);
    arrive(area, kCntShared, b - NR);
  } else if (b < NR + NS + NG) {
    const int g = b - NR - NS, RB = a.f / kFusedGuRows;
    const int k = g / RB, rb = g - k * RB;
    const uint32_t tag = launch_tag(area, ND);
    XRegs xr;
    x_issue<1>(a, 0, xr);
    // A residual-stream input is normalised (a block reduction) as it is
    // staged: that is done while the router runs, off the critical path
    // (30-layer stack 20.3 against 21.1 us per layer).  A plain token is
    // staged after the top-K, as before: staged early it cost the layer
    // 0.6 us, at either wave priority.
    if (a.rms) x_commit<1>(a, 0, xr, S);
    __builtin_amdgcn_s_setprio(2);
    // re-reads entries until they carry this launch's tag.  Forced sets (a
    // reused routing) name the experts without the logits: the weights then
    // stream from the start; only the down workgroups, which compute the
    // coefficients, wait for the logits.
    if (!a.forced) stage_logits_dev<NE>(a, my_rep, tag, s_logits);
    if (threadIdx.x < 64) {  // one wavefront finds the expert
      const int id = topk_kth<NE>(a, 0, s_logits, k);
      if (threadIdx.x == 0) scratch[0] = (uint32_t)id;
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    const int id = (int)scratch[0];
    gate_up_block<1, MAXI, kFusedGuRows, true>(a, 0, a.expert_base + (size_t)id * a.expert_stride, a.ro, rb,
                                               a.fs + k * a.f, S, xr, tag, a.rms != 0);
    arrive(area, kCntRouted, g);
  } else {
    down_fused<SS, SR, NE>(a, b - NR - NS - NG, ND, (uint32_t)NS, (uint32_t)NG, my_rep, smem,
                           s_logits, scratch, s_sel, s_w);
  }
}

template <int ACT, int MAXI, int NE>
hipError_t launch_ab(const LayerArgs& a, int stages, hipStream_t s) {
  const size_t lds = x_stage_bytes(a.d);
  if (stages & (kStageRouter | kStageShared)) {
    const int NR = route_blocks(a);
    const int NS = (stages & kStageShared) ? a.fs / 8 : 0;
    if (NR + NS > 0)
      launch_timed(a.prof, kKRouteShared, route_shared_kernel<ACT, MAXI>, dim3(NR + NS, a.T), dim3(kThreads), lds, s,
                   a);
    if ((stages & kStageRouter) && !a.topk_in_gate_up)
      launch_timed(a.prof, kKTopK, topk_kernel<NE>, dim3(a.T), dim3(64), 0, s, a);
  }
  if (stages & kStageRouted) {
    const int extra = a.topk_in_gate_up ? 1 : 0;  // the publishing workgroup
    const int slots = a.run_mask ? __builtin_popcount(a.run_mask) : a.K;
    const int NS = a.shared_in_routed ? a.fs / 8 : 0;
    launch_timed(a.prof, kKRoutedGateUp, routed_gu_kernel<ACT, MAXI, NE>,
                 dim3(NS + slots * (a.f / 8) + extra, a.T), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_c(const LayerArgs& a, hipStream_t s) {
  const int NI = a.fs / 64 + a.K * (a.f / 64);
  const int F = a.fs + a.K * a.f;
  const size_t lds = down_lds_bytes(F, NI, a.K, ACT);
  if (NI <= 128)
    launch_timed(a.prof, kKDownCombine, down_combine_kernel<ACT, 4>, dim3(a.d / 8, a.T), dim3(kThreads), lds, s, a);
  else
    launch_timed(a.prof, kKDownCombine, down_combine_kernel<ACT, 8>, dim3(a.d / 8, a.T), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int ACT, int NE>
hipError_t launch_ab_ne(const LayerArgs& a, int stages, hipStream_t s) {
  const int maxi = (a.d / 64 + 31) / 32;
  if (maxi <= 1) return launch_ab<ACT, 1, NE>(a, stages, s);
  if (maxi == 2) return launch_ab<ACT, 2, NE>(a, stages, s);
  if (maxi == 3) return launch_ab<ACT, 3, NE>(a, stages, s);
  return launch_ab<ACT, 4, NE>(a, stages, s);
}

template <int ACT>
hipError_t launch_all(const LayerArgs& a, hipStream_t s) {
  const int stages = a.stages ? a.stages : kStageAll;
  hipError_t e;
  if (a.E <= 64)
    e = launch_ab_ne<ACT, 1>(a, stages, s);
  else if (a.E <= 128)
    e = launch_ab_ne<ACT, 2>(a, stages, s);
  else if (a.E <= 256)
    e = launch_ab_ne<ACT, 4>(a, stages, s);
  else
    e = launch_ab_ne<ACT, 16>(a, stages, s);
  if (e != hipSuccess || !(stages & kStageDown)) return e;
  return launch_c<ACT>(a, s);
}

size_t fused_lds_bytes(const LayerArgs& a) {
  const int NI = a.fs / 64 + a.K * (a.f / 64);
  const int F = a.fs + a.K * a.f;
  return std::max(x_stage_bytes(a.d), down_lds_bytes(F, NI, a.K, 1));
}

template <int NE, int MAXI, int SS, int SR>
hipError_t launch_fused_k(const LayerArgs& a, hipStream_t s) {
  int NR, NS, NG, ND;
  const int total = fused_groups(a.E, a.K, a.d, a.f, a.fs, &NR, &NS, &NG, &ND);
  launch_timed(a.prof, kKFusedLayer, fused_layer_kernel<MAXI, NE, SS, SR>, dim3(total), dim3(kThreads),
               fused_lds_bytes(a), s, a);
  return hipGetLastError();
}

// Weight slots of a down workgroup: ceil(Gs / 32) for the shared part (0..2)
// and ceil(K * Gf / 32) for the routed part (1..4).
template <int NE, int MAXI>
hipError_t launch_fused_mi(const LayerArgs& a, hipStream_t s) {
  const int ss = (a.fs / 64 + 31) / 32, sr = (a.K * (a.f / 64) + 31) / 32;
  const int code = (ss <= 1 ? ss : 2) * 8 + (sr <= 2 ? 2 : 4);
  switch (code) {
    case 2: return launch_fused_k<NE, MAXI, 0, 2>(a, s);
    case 4: return launch_fused_k<NE, MAXI, 0, 4>(a, s);
    case 10: return launch_fused_k<NE, MAXI, 1, 2>(a, s);
    case 12: return launch_fused_k<NE, MAXI, 1, 4>(a, s);
    case 18: return launch_fused_k<NE, MAXI, 2, 2>(a, s);
    default: return launch_fused_k<NE, MAXI, 2, 4>(a, s);
  }
}

// Gate/up weight slots per lane: ceil(G / 16) with 16 lanes per row (1..4).
template <int NE>
hipError_t launch_fused_ne(const LayerArgs& a, hipStream_t s) {
  const int maxi = (a.d / 64 + kThreads / kFusedGuRows - 1) / (kThreads / kFusedGuRows);
  if (maxi <= 1) return launch_fused_mi<NE, 1>(a, s);
  if (maxi == 2) return launch_fused_mi<NE, 2>(a, s);
  if (maxi == 3) return launch_fused_mi<NE, 3>(a, s);
  return launch_fused_mi<NE, 4>(a, s);
}

hipError_t launch_fused(const LayerArgs& a, hipStream_t s) {
  if (a.E <= 64) return launch_fused_ne<1>(a, s);
  if (a.E <= 128) return launch_fused_ne<2>(a, s);
  if (a.E <= 256) return launch_fused_ne<4>(a, s);
  return launch_fused_ne<16>(a, s);
}

// One thread per weight: the 16-byte word and the scale/bias word that the
// GEMV kernels read for (row, col), decoded the same way.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* blob, uint32_t q_off, uint32_t sb_off, int rows,
                                                      int cols, float* out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * cols) return;
  const int row = (int)(i / cols), col = (int)(i % cols);
  const int G = cols >> 6, rb = row >> 3, r = row & 7, g = col >> 6, c = col & 63;
  const size_t off = (((size_t)rb * G + g) * 2) * 128 + (c >> 5) * 128 + r * 16;  // as gate_up_block / down_block
  const v4u q = ldg<v4u>(blob + q_off + off);
  const uint32_t w = q[(c & 31) >> 3];
  const uint32_t nib = (w >> (4 * (c & 7))) & 0xFu;
  const uint32_t sb = ldg<uint32_t>(blob + sb_off + (((size_t)rb * G + g) * 8 + r) * 4);
  out[i] = fmaf(f16_to_f32((uint16_t)(sb & 0xFFFFu)), (float)nib, f16_to_f32((uint16_t)(sb >> 16)));
}

// Fills: kFillBlocks workgroups per blob stream it with 16-byte loads, four
// in flight per lane (about 50 GB/s from pinned host memory for one blob).
constexpr int kFillBlocks = 128;
__global__ __launch_bounds__(256) void fill_kernel(FillArgs f) {
  const int i = blockIdx.x / kFillBlocks, part = blockIdx.x - i * kFillBlocks;
  const v4u* src = reinterpret_cast<const v4u*>(f.src[i]);
  v4u* dst = reinterpret_cast<v4u*>(f.dst[i]);
  const size_t n16 = f.bytes / 16, stride = (size_t)kFillBlocks * 256;
  size_t j = (size_t)part * 256 + threadIdx.x;
  for (; j + 3 * stride < n16; j += 4 * stride) {
    const v4u w0 = src[j], w1 = src[j + stride], w2 = src[j + 2 * stride], w3 = src[j + 3 * stride];
    dst[j] = w0;
    dst[j + stride] = w1;
    dst[j + 2 * stride] = w2;
    dst[j + 3 * stride] = w3;
  }
  for (; j < n16; j += stride) dst[j] = src[j];
  if (blockIdx.x == 0 && (int)threadIdx.x < f.n) {
    f.table[f.expert[threadIdx.x]] = reinterpret_cast<uint64_t>(f.dst[threadIdx.x]);
    if (f.evicted[threadIdx.x] >= 0) f.table[f.evicted[threadIdx.x]] = 0;
  }
}

}  // namespace

hipError_t launch_fill(const FillArgs& f, hipStream_t s) {
  if (f.n <= 0) return hipSuccess;
  if (f.n > kMaxFills || f.bytes % 16 != 0) return hipErrorInvalidValue;
  fill_kernel<<<dim3((unsigned)(f.n * kFillBlocks)), dim3(256), 0, s>>>(f);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* blob, uint32_t q_off, uint32_t sb_off, int rows, int cols, float* out,
                          hipStream_t s) {
  const size_t n = (size_t)rows * cols;
  dequant_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(blob, q_off, sb_off, rows, cols, out);
  return hipGetLastError();
}

size_t decode_lds_bytes_x(int d) { return x_stage_bytes(d); }
size_t decode_sync_bytes(int E) { return sync_area_bytes(E); }
size_t decode_arep_bytes(int F) { return kAReps * a_rep_stride(F); }
size_t decode_lds_bytes_down(int F, int NI, int K, int act) { return down_lds_bytes(F, NI, K, act); }

// The fused layer kernel serves one bf16 token on resident experts, when its
// LDS (dynamic part plus about 6 KB of static routing state) fits in 64 KB.
// The down workgroups hold at most 2 shared and 4 routed weight slots (64 and
// 128 groups), the gate/up workgroups at most 4 (d_model <= 4096).
bool decode_fused_ok(const LayerArgs& a) {
  return a.T == 1 && a.act == 1 && a.E <= 1024 && a.d <= 4096 && fused_lds_bytes(a) + 6 * 1024 <= 64 * 1024 &&
         a.fs / 64 <= 64 && a.K * (a.f / 64) <= 128;
}

// Workspace of the allocation-free forward (moe_layer_forward_noalloc): a
// file-scope device array, one per GPU, held until the process ends.  Its
// address is taken once per device (host code never uses the array's name as
// an address) and handed to the kernels like any other workspace pointer.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const LayerArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.fused) return decode_fused_ok(a) ? launch_fused(a, s) : hipErrorInvalidValue;
  return a.act == 1 ? launch_all<1>(a, s) : launch_all<0>(a, s);
}

}  // namespace moe

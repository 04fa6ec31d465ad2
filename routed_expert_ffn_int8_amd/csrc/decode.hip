// Decode path (few tokens per call): three kernels per layer.
//
//   A  route_shared : int8 router GEMV for every expert (8 rows per workgroup)
//                     with the softmax top-K run by the last router workgroup
//                     of each token, side by side with the shared expert's
//                     gate/up GEMV + SiLU*mul (routing-independent, so it
//                     overlaps the router; Rockchip-NPU plan §2.4 runs the
//                     shared expert while the routed experts are fetched).
//   B  routed_gu    : gate/up GEMV + SiLU*mul of the K chosen experts.
//   C  down_combine : down GEMV of the shared and K chosen experts, weighted
//                     sum y = shared + sum_k w_k * down_k (BigMoeOnEdge,
//                     "re-routing at every token and layer": weighted merge of
//                     the chosen experts), optional residual, one store.
//
// Each workgroup owns an 8-row block of one matrix: lane (r = tid & 7,
// jj = tid >> 3) reads 16-byte pieces of row r for the 64-wide groups
// g = jj + 16 i, so every wavefront load instruction covers eight full
// 128-byte lines.  All of a lane's weight loads are issued before the token
// input is staged in LDS, to keep many bytes in flight.
//
// Arithmetic per 64-wide group (affine weights w = s*q + b, Rockchip-NPU
// plan §2.1): sum_c w_c x_c = s * sum_c q_c x_c + b * sum_c x_c.
// bf16 activations: nibble pairs become bf16 (128 + q) with one and-or and
// feed v_dot2_f32_bf16 against bf16 pairs of x, then the 128 * sum(x) offset
// is folded into the bias term.  The down projection uses fp16 (1024 + q)
// against fp16-rounded activations the same way.  fp32 activations use an
// exact byte->float convert and fp32 FMAs.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

struct XStage {
  float* xf;   // [d] input as fp32 (after rounding to the activation type)
  uint4* xp;   // [d/8] bf16 pairs (x[8j+m], x[8j+m+4]) for m = 0..3
  float* xs;   // [d/64] group sums
  float* red;  // [32] cross-wave scratch
};

__device__ __forceinline__ XStage carve_x(char* smem, int d) {
  XStage S;
  S.xf = reinterpret_cast<float*>(smem);
  S.xp = reinterpret_cast<uint4*>(smem + (size_t)d * 4);
  S.xs = reinterpret_cast<float*>(smem + (size_t)d * 6);
  S.red = S.xs + d / 64;
  return S;
}

__host__ __device__ inline size_t x_stage_bytes(int d) { return (size_t)d * 6 + (size_t)(d / 64) * 4 + 32 * 4; }

// Load token t, optionally apply rmsnorm (unit gain) and round to the
// activation type, and fill xf / xp / xs.  Called by all threads.
template <int ACT>
__device__ void stage_x(const LayerArgs& a, int t, const XStage& S) {
  const int tid = threadIdx.x;
  const int d = a.d, W = d >> 3;
  float ss = 0.f;
  for (int j = tid; j < W; j += kThreads) {
    float v[8];
    if (ACT == 1) {
      const uint4 raw = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)t * d)[j];
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v[2 * m] = __uint_as_float(w4[m] << 16);
        v[2 * m + 1] = __uint_as_float(w4[m] & 0xFFFF0000u);
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (size_t)t * d);
      const float4 p0 = src[2 * j], p1 = src[2 * j + 1];
      v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
      v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      S.xf[8 * j + m] = v[m];
      ss = fmaf(v[m], v[m], ss);
    }
  }
  float inv = 1.f;
  if (a.rms) {
    ss = xor_sum(ss, 1, 32);
    if ((tid & 63) == 0) S.red[tid >> 6] = ss;
    __syncthreads();
    const float tot = S.red[0] + S.red[1];
    inv = 1.0f / sqrtf(tot / (float)d + a.eps);
  }
  for (int j = tid; j < W; j += kThreads) {
    float v[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float u = S.xf[8 * j + m];
      if (a.rms) {
        u *= inv;
        if (ACT == 1) u = bf16_to_f32(f32_to_bf16(u));
        S.xf[8 * j + m] = u;
      }
      v[m] = u;
    }
    if (ACT == 1) {
      uint4 p;
      p.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[4]) << 16);
      p.y = (uint32_t)f32_to_bf16(v[1]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
      p.z = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[6]) << 16);
      p.w = (uint32_t)f32_to_bf16(v[3]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
      S.xp[j] = p;
    }
    float part = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    part = xor_sum(part, 1, 4);  // the 8 words of one group sit in 8 consecutive lanes
    if ((j & 7) == 0) S.xs[j >> 3] = part;
  }
  __syncthreads();
}

// One 64-wide group: returns sum_c q_c * x_c (bf16 mode: sum_c (128+q_c) x_c).
template <int ACT>
__device__ __forceinline__ float group_dot(const uint4 q[2], const XStage& S, int g) {
  float p = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w4[4] = {q[h].x, q[h].y, q[h].z, q[h].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w = w4[m];
      const int word = g * 8 + h * 4 + m;
      if (ACT == 1) {
        const uint4 xw = S.xp[word];
        p = dot2_bf16(nib_pair<kMagicBf16>(w, 0), xw.x, p);
        p = dot2_bf16(nib_pair<kMagicBf16>(w, 1), xw.y, p);
        p = dot2_bf16(nib_pair<kMagicBf16>(w, 2), xw.z, p);
        p = dot2_bf16(nib_pair<kMagicBf16>(w, 3), xw.w, p);
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

// Group contribution s*sum(q x) + b*sum(x), with the bf16 magic offset folded in.
template <int ACT>
__device__ __forceinline__ float group_term(float p, uint32_t sb, float xsum) {
  const float s = f16_to_f32((uint16_t)(sb & 0xFFFFu));
  const float b = f16_to_f32((uint16_t)(sb >> 16));
  const float bb = (ACT == 1) ? b - 128.f * s : b;
  return fmaf(s, p, bb * xsum);
}

// Store one element of the intermediate activation vector a (position P of
// the token's [shared | expert 0 | ... | expert K-1] vector) and return the
// value as the down projection will see it.
template <int ACT>
__device__ __forceinline__ float store_a(void* abuf_t, int P, float v) {
  if (ACT == 1) {
    const uint16_t h = f32_to_f16(v);
    const int m = P & 7;
    static_cast<uint16_t*>(abuf_t)[(P & ~7) + (m & 3) * 2 + (m >> 2)] = h;
    return f16_to_f32(h);
  }
  static_cast<float*>(abuf_t)[P] = v;
  return v;
}

// gate/up GEMV + SiLU*mul for the 8-row block `rb` of one expert blob.
template <int ACT, int MAXI>
__device__ void gate_up_block(const LayerArgs& a, int t, const uint8_t* blob, const BlobOffsets& o, int rb,
                              int apos, const XStage& S) {
  const int tid = threadIdx.x, r = tid & 7, jj = tid >> 3;
  const int G = a.d >> 6;
  const int row = rb * 8 + r;
  const uint8_t* gq = blob + o.gq;
  const uint8_t* uq = blob + o.uq;
  const uint32_t* gsb = reinterpret_cast<const uint32_t*>(blob + o.gsb);
  const uint32_t* usb = reinterpret_cast<const uint32_t*>(blob + o.usb);
  float accg = 0.f, accu = 0.f;
  for (int base = 0; base < G; base += 16 * MAXI) {
    uint4 qg[MAXI][2], qu[MAXI][2];
    uint32_t sg[MAXI], su[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int g = base + jj + 16 * i;
      if (g < G) {
        const size_t off = (((size_t)rb * G + g) * 2) * 128 + r * 16;
        qg[i][0] = *reinterpret_cast<const uint4*>(gq + off);
        qg[i][1] = *reinterpret_cast<const uint4*>(gq + off + 128);
        qu[i][0] = *reinterpret_cast<const uint4*>(uq + off);
        qu[i][1] = *reinterpret_cast<const uint4*>(uq + off + 128);
        sg[i] = gsb[(size_t)row * G + g];
        su[i] = usb[(size_t)row * G + g];
      }
    }
    if (base == 0) stage_x<ACT>(a, t, S);
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int g = base + jj + 16 * i;
      if (g < G) {
        accg += group_term<ACT>(group_dot<ACT>(qg[i], S, g), sg[i], S.xs[g]);
        accu += group_term<ACT>(group_dot<ACT>(qu[i], S, g), su[i], S.xs[g]);
      }
    }
  }
  accg = xor_sum(accg, 8, 32);
  accu = xor_sum(accu, 8, 32);
  if ((tid & 63) < 8) {
    S.red[(tid >> 6) * 16 + r * 2] = accg;
    S.red[(tid >> 6) * 16 + r * 2 + 1] = accu;
  }
  __syncthreads();
  if (tid < 8) {
    const float gsum = S.red[r * 2] + S.red[16 + r * 2];
    const float usum = S.red[r * 2 + 1] + S.red[16 + r * 2 + 1];
    const int F = a.fs + a.K * a.f;
    char* abuf_t = static_cast<char*>(a.abuf) + (size_t)t * F * (ACT == 1 ? 2 : 4);
    const int P = apos + row;
    float seen = store_a<ACT>(abuf_t, P, silu(gsum) * usum);
    seen = xor_sum(seen, 1, 4);
    if (tid == 0) a.asum_part[(size_t)t * (F / 8) + (P >> 3)] = seen;
  }
}

// Orderable 64-bit key: larger logit first, then lower expert index.
__device__ __forceinline__ uint64_t topk_key(float l, int e) {
  uint32_t u = __float_as_uint(l + 0.0f);  // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Softmax top-K of token t by one wavefront (lane = threadIdx.x < 64).
// Ordering (logit desc, index asc); ids written ascending; weights are a
// softmax over the chosen set (= softmax over all experts renormalised).
__device__ void topk_token(const LayerArgs& a, int t) {
  const int lane = threadIdx.x;
  const int E = a.E, K = a.K;
  const float* lt = a.logits + (size_t)t * E;
  int my_id = 0;
  if (a.forced) {
    if (lane < K) {
      my_id = a.forced[(size_t)t * K + lane];
      if (my_id < 0 || my_id >= E) {
        atomicOr(a.err, kErrBadForcedId);
        my_id = 0;
      }
    }
  } else {
    uint64_t key[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      key[i] = (e < E) ? topk_key(lt[e], e) : 0ull;
    }
    for (int k = 0; k < K; ++k) {
      uint64_t m = key[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = key[i] > m ? key[i] : m;
      m = wave_max_u64(m);
      const int win = (int)(0xFFFFFFFFu - (uint32_t)m);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (lane + 64 * i == win) key[i] = 0ull;
      if (lane == k) my_id = win;
    }
  }
  const float l = (lane < K) ? lt[my_id] : -INFINITY;
  const float lmax = wave_max_f32(l);
  const float v = (lane < K) ? expf(l - lmax) : 0.f;
  const float den = xor_sum(v, 1, 32);
  int rank = 0;
  for (int j = 0; j < K; ++j) {  // unique rank even if a forced set repeats an id
    const int o = __shfl(my_id, j, 64);
    rank += (o < my_id || (o == my_id && j < lane)) ? 1 : 0;
  }
  if (lane < K) {
    const float w = v / den;
    a.ids[(size_t)t * K + rank] = my_id;
    a.wts[(size_t)t * K + rank] = w;
    if (a.ids_out) a.ids_out[(size_t)t * K + rank] = my_id;
    if (a.w_out) a.w_out[(size_t)t * K + rank] = w;
  }
}

// ---------------------------------------------------------------- kernel A
template <int ACT, int MAXI>
__global__ __launch_bounds__(kThreads) void route_shared_kernel(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const XStage S = carve_x(smem, a.d);
  const int t = blockIdx.y;
  const int NR = (a.E + 7) >> 3;
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= NR) {
    gate_up_block<ACT, MAXI>(a, t, a.shared_blob, a.so, blockIdx.x - NR, 0, S);
    return;
  }
  // router rows e0 .. e0+7
  const int r = tid & 7, jj = tid >> 3;
  const int e = blockIdx.x * 8 + r;
  const int d = a.d, NC = d >> 4;
  stage_x<ACT>(a, t, S);
  float acc = 0.f;
  if (e < a.E) {
    const int8_t* wrow = a.router_w + (size_t)e * d;
    for (int c = jj; c < NC; c += 16) {
      const int4 w16 = *reinterpret_cast<const int4*>(wrow + c * 16);
      const int w4[4] = {w16.x, w16.y, w16.z, w16.w};
      const float4* xv = reinterpret_cast<const float4*>(S.xf + c * 16);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float4 xx = xv[m];
        const int w = w4[m];
        acc = fmaf((float)((w << 24) >> 24), xx.x, acc);
        acc = fmaf((float)((w << 16) >> 24), xx.y, acc);
        acc = fmaf((float)((w << 8) >> 24), xx.z, acc);
        acc = fmaf((float)(w >> 24), xx.w, acc);
      }
    }
  }
  acc = xor_sum(acc, 8, 32);
  if ((tid & 63) < 8) S.red[(tid >> 6) * 8 + r] = acc;
  __syncthreads();
  if (tid < 8 && e < a.E) {
    const float tot = S.red[r] + S.red[8 + r];
    const float s = f16_to_f32(a.router_scale[e]);
    const float b = a.router_bias ? a.router_bias[e] : 0.f;
    a.logits[(size_t)t * a.E + e] = fmaf(s, tot, b);
  }
  // last router workgroup of this token runs the top-K
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (tid == 0) last = (atomicAdd(a.counter + t, 1u) == (unsigned)(NR - 1));
  __syncthreads();
  if (!last) return;
  __threadfence();
  if (tid < 64) topk_token(a, t);
  if (tid == 0) atomicExch(a.counter + t, 0u);
}

// ---------------------------------------------------------------- kernel B
template <int ACT, int MAXI>
__global__ __launch_bounds__(kThreads) void routed_gu_kernel(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const XStage S = carve_x(smem, a.d);
  const int t = blockIdx.y;
  const int RB = a.f >> 3;
  const int k = blockIdx.x / RB, rb = blockIdx.x % RB;
  const int id = a.ids[(size_t)t * a.K + k];
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.expert_addr[id]);
  if (blob == nullptr) {  // expert not resident: leave a marker, contribute zeros
    if (threadIdx.x == 0) atomicOr(a.err, kErrMissingExpert);
    const int F = a.fs + a.K * a.f;
    const int P = a.fs + k * a.f + rb * 8;
    if (threadIdx.x < 8) {
      char* abuf_t = static_cast<char*>(a.abuf) + (size_t)t * F * (ACT == 1 ? 2 : 4);
      store_a<ACT>(abuf_t, P + threadIdx.x, 0.f);
    }
    if (threadIdx.x == 0) a.asum_part[(size_t)t * (F / 8) + (P >> 3)] = 0.f;
    return;
  }
  gate_up_block<ACT, MAXI>(a, t, blob, a.ro, rb, a.fs + k * a.f, S);
}

// ---------------------------------------------------------------- kernel C
__host__ __device__ inline size_t down_lds_bytes(int F, int NI, int K, int act) {
  return (size_t)F * (act == 1 ? 2 : 4) + (size_t)NI * 4 + (size_t)K * 4 + 32 * 4;
}

template <int ACT, int MAXI>
__global__ __launch_bounds__(kThreads) void down_combine_kernel(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, r = tid & 7, jj = tid >> 3;
  const int t = blockIdx.y, rb = blockIdx.x;
  const int row = rb * 8 + r;
  const int Gs = a.fs >> 6, Gf = a.f >> 6, K = a.K;
  const int NI = Gs + K * Gf;
  const int F = a.fs + K * a.f;
  char* lds_a = smem;
  float* asum = reinterpret_cast<float*>(smem + (size_t)F * (ACT == 1 ? 2 : 4));
  float* wk = asum + NI;
  float* red = wk + K;
  const int32_t* ids_t = a.ids + (size_t)t * K;
  float acc = 0.f;
  for (int base = 0; base < NI; base += 16 * MAXI) {
    uint4 q[MAXI][2];
    uint32_t sb[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int it = base + jj + 16 * i;
      if (it < NI) {
        const uint8_t* blob;
        int G, g;
        uint32_t oq, osb;
        if (it < Gs) {
          blob = a.shared_blob; G = Gs; g = it; oq = a.so.dq; osb = a.so.dsb;
        } else {
          const int k = (it - Gs) / Gf;
          g = (it - Gs) - k * Gf;
          G = Gf;
          blob = reinterpret_cast<const uint8_t*>(a.expert_addr[ids_t[k]]);
          oq = a.ro.dq; osb = a.ro.dsb;
        }
        if (blob != nullptr) {
          const size_t off = (((size_t)rb * G + g) * 2) * 128 + r * 16;
          q[i][0] = *reinterpret_cast<const uint4*>(blob + oq + off);
          q[i][1] = *reinterpret_cast<const uint4*>(blob + oq + off + 128);
          sb[i] = reinterpret_cast<const uint32_t*>(blob + osb)[(size_t)row * G + g];
        } else {
          q[i][0] = q[i][1] = make_uint4(0, 0, 0, 0);
          sb[i] = 0;  // scale 0, bias 0
        }
      }
    }
    if (base == 0) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.abuf) +
                                                        (size_t)t * F * (ACT == 1 ? 2 : 4));
      const int nw = F * (ACT == 1 ? 2 : 4) / 16;
      for (int j = tid; j < nw; j += kThreads) reinterpret_cast<uint4*>(lds_a)[j] = src[j];
      const float* part = a.asum_part + (size_t)t * (F / 8);
      for (int i = tid; i < NI; i += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < 8; ++p) s += part[i * 8 + p];
        asum[i] = s;
      }
      if (tid < K) wk[tid] = a.wts[(size_t)t * K + tid];
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int it = base + jj + 16 * i;
      if (it < NI) {
        float p = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w4[4] = {q[i][h].x, q[i][h].y, q[i][h].z, q[i][h].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t w = w4[m];
            const int word = it * 8 + h * 4 + m;
            if (ACT == 1) {
              const uint4 av = reinterpret_cast<const uint4*>(lds_a)[word];
              p = dot2_f16(nib_pair<kMagicF16>(w, 0), av.x, p);
              p = dot2_f16(nib_pair<kMagicF16>(w, 1), av.y, p);
              p = dot2_f16(nib_pair<kMagicF16>(w, 2), av.z, p);
              p = dot2_f16(nib_pair<kMagicF16>(w, 3), av.w, p);
            } else {
              const float4 x0 = reinterpret_cast<const float4*>(lds_a)[word * 2];
              const float4 x1 = reinterpret_cast<const float4*>(lds_a)[word * 2 + 1];
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
        const float s = f16_to_f32((uint16_t)(sb[i] & 0xFFFFu));
        const float b = f16_to_f32((uint16_t)(sb[i] >> 16));
        const float bb = (ACT == 1) ? b - 1024.f * s : b;
        const float term = fmaf(s, p, bb * asum[it]);
        const float wgt = (it < Gs) ? 1.f : wk[(it - Gs) / Gf];
        acc = fmaf(wgt, term, acc);
      }
    }
  }
  acc = xor_sum(acc, 8, 32);
  if ((tid & 63) < 8) red[(tid >> 6) * 8 + r] = acc;
  __syncthreads();
  if (tid < 8) {
    const float y = red[r] + red[8 + r];
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
hipError_t launch_ab(const LayerArgs& a, int stages, hipStream_t s) {
  const size_t lds = x_stage_bytes(a.d);
  if (stages & (kStageRouter | kStageShared)) {
    const int NR = (a.E + 7) / 8;
    const int NS = (stages & kStageShared) ? a.fs / 8 : 0;
    route_shared_kernel<ACT, MAXI><<<dim3(NR + NS, a.T), kThreads, lds, s>>>(a);
  }
  if (stages & kStageRouted) routed_gu_kernel<ACT, MAXI><<<dim3(a.K * (a.f / 8), a.T), kThreads, lds, s>>>(a);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_c(const LayerArgs& a, hipStream_t s) {
  const int NI = a.fs / 64 + a.K * (a.f / 64);
  const int F = a.fs + a.K * a.f;
  const size_t lds = down_lds_bytes(F, NI, a.K, ACT);
  if (NI <= 64)
    down_combine_kernel<ACT, 4><<<dim3(a.d / 8, a.T), kThreads, lds, s>>>(a);
  else
    down_combine_kernel<ACT, 8><<<dim3(a.d / 8, a.T), kThreads, lds, s>>>(a);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_all(const LayerArgs& a, hipStream_t s) {
  const int stages = a.stages ? a.stages : kStageAll;
  const int G = a.d / 64;
  const int maxi = (G + 15) / 16;
  hipError_t e;
  if (maxi <= 1)
    e = launch_ab<ACT, 1>(a, stages, s);
  else if (maxi == 2)
    e = launch_ab<ACT, 2>(a, stages, s);
  else if (maxi == 3)
    e = launch_ab<ACT, 3>(a, stages, s);
  else
    e = launch_ab<ACT, 4>(a, stages, s);
  if (e != hipSuccess || !(stages & kStageDown)) return e;
  return launch_c<ACT>(a, s);
}

}  // namespace

size_t decode_lds_bytes_x(int d) { return x_stage_bytes(d); }
size_t decode_lds_bytes_down(int F, int NI, int K, int act) { return down_lds_bytes(F, NI, K, act); }

hipError_t launch_decode(const LayerArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return a.act == 1 ? launch_all<1>(a, s) : launch_all<0>(a, s);
}

}  // namespace moe

// Row-wise, HBM-bound kernels of the layer: RMSNorm of token rows, the fused
// QK-norm + RoPE + KV-cache store, the fp32 -> activation row store and the
// last-token LM-head GEMV.
//
// Operations follow oxibonsai-kernels metal_prefill.rs, encode_layer_prefill
// steps 1 and 5 (batched RMSNorm), step 3a-3d (QK-norm, RoPE, KV store) and
// the "Tail" block of encode_full_forward_prefill (final norm + LM head).
#include "common.h"
#include "launch.h"

namespace tlp {

// 8 consecutive elements <-> 8 floats; p must be 16-byte aligned for bf16 and
// 32-byte aligned for fp32 (rows are multiples of 8 elements).
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float v[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// One block of NT threads per row.  The row is assembled once in registers:
// x (activation type or fp32) plus the split-K partial sums of the projection
// that produced it; the sum may be stored as the fp32 residual stream and/or
// rounded to the activation type, and RMSNorm(sum) * gain is written when a
// gain is given.  NT is picked so that a thread holds one 8-element chunk
// (two at H = 16384): the stores of one chunk may alias the loads of the next
// (the residual is read and rewritten in place), so a second chunk per thread
// would wait for a second round trip to memory.
template <typename T, bool XF32, bool NORM_F32, int NT>
__global__ __launch_bounds__(NT) void rownorm_kernel(RowArgs a) {
  constexpr int CH = 2048 / NT;   // chunks of 8 elements per thread (H <= 16384)
  constexpr int MAXP = 8;         // partial slices summed per row
  __shared__ float red[NT / 64];
  const int r = blockIdx.x;
  const int chunks = a.H >> 3;
  const size_t roff = static_cast<size_t>(r) * a.H;
  float v[CH][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + c * NT;
    if (idx >= chunks) break;
    // issue the row chunk and every partial slice before summing
    if constexpr (XF32)
      load8(static_cast<const float*>(a.x) + static_cast<size_t>(r) * a.ldx + idx * 8, v[c]);
    else
      load8(static_cast<const T*>(a.x) + static_cast<size_t>(r) * a.ldx + idx * 8, v[c]);
    float q[MAXP][8];
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (p < a.n_part) load8(a.part + p * a.part_stride + roff + idx * 8, q[p]);
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (p < a.n_part)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] += q[p][i];
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[c][i] * v[c][i];
    if (a.res_out) store8(a.res_out + roff + idx * 8, v[c]);
    if (a.act_out)
      store8(static_cast<T*>(a.act_out) + static_cast<size_t>(r) * a.ld_act + idx * 8, v[c]);
  }
  if (!a.gain) return;
  ss = block_sum<NT / 64>(ss, red);
  const float inv = rsqrtf(ss / static_cast<float>(a.H) + a.eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + c * NT;
    if (idx >= chunks) break;
    float g[8];
    load8(static_cast<const T*>(a.gain) + idx * 8, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[c][i] = g[i] * (v[c][i] * inv);
    if constexpr (NORM_F32)
      store8(static_cast<float*>(a.norm_out) + roff + idx * 8, v[c]);
    else
      store8(static_cast<T*>(a.norm_out) + roff + idx * 8, v[c]);
  }
}

template <typename T, int NT>
static hipError_t rownorm_nt(const RowArgs& a, hipStream_t s) {
  dim3 grid(a.rows), block(NT);
  if (a.x_f32) {
    if (a.norm_f32) rownorm_kernel<T, true, true, NT><<<grid, block, 0, s>>>(a);
    else rownorm_kernel<T, true, false, NT><<<grid, block, 0, s>>>(a);
  } else {
    if (a.norm_f32) rownorm_kernel<T, false, true, NT><<<grid, block, 0, s>>>(a);
    else rownorm_kernel<T, false, false, NT><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t rownorm_t(const RowArgs& a, hipStream_t s) {
  const int chunks = a.H >> 3;
  if (chunks <= 256) return rownorm_nt<T, 256>(a, s);
  if (chunks <= 512) return rownorm_nt<T, 512>(a, s);
  return rownorm_nt<T, 1024>(a, s);
}

hipError_t launch_rownorm(Act act, const RowArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.H % 8 || a.H > 8 * 8 * 256 || a.n_part > 8) return hipErrorInvalidValue;
  return act == Act::F32 ? rownorm_t<float>(a, s) : rownorm_t<uint16_t>(a, s);
}

// E consecutive elements <-> floats (E = 2 or 4; the pointers are E-aligned).
template <int E> __device__ __forceinline__ void ldv(const float* p, float (&x)[E]) {
  if constexpr (E == 4) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
    const float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x; x[1] = v.y;
  }
}
template <int E> __device__ __forceinline__ void ldv(const uint16_t* p, float (&x)[E]) {
  uint32_t w[E / 2];
  if constexpr (E == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
#pragma unroll
  for (int e = 0; e < E / 2; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
template <int E> __device__ __forceinline__ void stv(float* p, const float (&x)[E]) {
  if constexpr (E == 4) *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  else *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
}
template <int E> __device__ __forceinline__ void stv(uint16_t* p, const float (&x)[E]) {
  if constexpr (E == 4) *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  else *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(x[0], x[1]);
}
template <int E> __device__ __forceinline__ void stv(f16_t* p, const float (&x)[E]) {
  uint32_t w[E / 2];
#pragma unroll
  for (int e = 0; e < E / 2; ++e)
    w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<f16_t>(x[2 * e]))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<f16_t>(x[2 * e + 1]))) << 16);
  if constexpr (E == 4) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  else *reinterpret_cast<uint32_t*>(p) = w[0];
}

// Block (t, y) covers token t and heads 16y .. 16y+15 of [Q heads | K heads |
// V heads]; a group of 16 lanes takes one head.  Lane j of a group owns the E
// = hd/32 consecutive elements E*j .. of each rotate-half half, so every pair
// (i, i + hd/2) stays in one lane, loads and stores are E-wide vectors, and
// the head's RMSNorm is a 16-lane reduction.  The projected row is either qkv
// itself (activation type) or, when the QKV GEMM split K, the sum of its
// n_part fp32 slices; roped Q is written back into qkv for the attention
// kernel either way, roped K and raw V go to the cache in its type C.
template <typename T, typename C, int HD>
__global__ __launch_bounds__(256) void qk_rope_store_kernel(
    T* __restrict__ qkv, int qkv_ld, const float* __restrict__ part, int n_part,
    size_t part_stride, const T* __restrict__ q_gain, const T* __restrict__ k_gain,
    int qk_norm, float eps, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, C* __restrict__ k_layer, C* __restrict__ v_layer,
    int max_seq, int start, int nq, int nkv) {
  constexpr int HALF = HD / 2, E = HALF / 16;
  const int t = blockIdx.x;
  const int pos = start + t;
  const int j = threadIdx.x & 15;
  const int hh = blockIdx.y * 16 + (threadIdx.x >> 4);
  if (hh >= nq + 2 * nkv) return;   // whole 16-lane groups; no block-wide sync follows
  T* row = qkv + static_cast<size_t>(t) * qkv_ld;
  const float* prow = part + static_cast<size_t>(t) * qkv_ld;
  const int c1 = hh * HD + E * j, c2 = c1 + HALF;
  float x1[E], x2[E];
  if (n_part == 0) {
    ldv<E>(row + c1, x1);
    ldv<E>(row + c2, x2);
  } else {
    constexpr int MAXP = 8;   // issue every slice load before summing
    float q1[MAXP][E], q2[MAXP][E];
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (p < n_part) {
        ldv<E>(prow + p * part_stride + c1, q1[p]);
        ldv<E>(prow + p * part_stride + c2, q2[p]);
      }
#pragma unroll
    for (int e = 0; e < E; ++e) x1[e] = x2[e] = 0.f;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (p < n_part)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          x1[e] += q1[p][e];
          x2[e] += q2[p][e];
        }
  }
  if (hh >= nq + nkv) {  // V head: raw copy into the cache slot
    C* dst = v_layer + (static_cast<size_t>(hh - nq - nkv) * max_seq + pos) * HD;
    stv<E>(dst + E * j, x1);
    stv<E>(dst + HALF + E * j, x2);
    return;
  }
  if (qk_norm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 16);
    const float inv = rsqrtf(ss / static_cast<float>(HD) + eps);
    const T* g = hh < nq ? q_gain : k_gain;
    float g1[E], g2[E];
    ldv<E>(g + E * j, g1);
    ldv<E>(g + HALF + E * j, g2);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      x1[e] = g1[e] * (x1[e] * inv);
      x2[e] = g2[e] * (x2[e] * inv);
    }
  }
  float cs[E], sn[E], y1[E], y2[E];
  ldv<E>(rope_cos + static_cast<size_t>(pos) * HALF + E * j, cs);
  ldv<E>(rope_sin + static_cast<size_t>(pos) * HALF + E * j, sn);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    y1[e] = x1[e] * cs[e] - x2[e] * sn[e];
    y2[e] = x2[e] * cs[e] + x1[e] * sn[e];
  }
  if (hh < nq) {
    stv<E>(row + c1, y1);
    stv<E>(row + c2, y2);
  } else {
    C* dst = k_layer + (static_cast<size_t>(hh - nq) * max_seq + pos) * HD;
    stv<E>(dst + E * j, y1);
    stv<E>(dst + HALF + E * j, y2);
  }
}

template <typename T, typename C>
static void rope_launch(int head_dim, dim3 grid, hipStream_t s, void* qkv, int qkv_ld,
                        const float* part, int n_part, size_t part_stride, const void* q_gain,
                        const void* k_gain, bool qk_norm, float eps, const float* rope_cos,
                        const float* rope_sin, void* k_layer, void* v_layer, int max_seq,
                        int start, int nq, int nkv) {
#define TLP_ROPE(HD_)                                                                        \
  qk_rope_store_kernel<T, C, HD_><<<grid, 256, 0, s>>>(                                     \
      static_cast<T*>(qkv), qkv_ld, part, n_part, part_stride, static_cast<const T*>(q_gain), \
      static_cast<const T*>(k_gain), qk_norm ? 1 : 0, eps, rope_cos, rope_sin,              \
      static_cast<C*>(k_layer), static_cast<C*>(v_layer), max_seq, start, nq, nkv)
  if (head_dim == 128) TLP_ROPE(128);
  else TLP_ROPE(64);
#undef TLP_ROPE
}

hipError_t launch_qk_rope_store(Act act, bool kv16, void* qkv, int M, int qkv_ld, const float* part,
                                int n_part, size_t part_stride, const void* q_gain,
                                const void* k_gain, bool qk_norm, float eps,
                                const float* rope_cos, const float* rope_sin, void* k_layer,
                                void* v_layer, int max_seq, int start, int nq, int nkv,
                                int head_dim, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (n_part > 8 || (head_dim != 64 && head_dim != 128)) return hipErrorInvalidValue;
  dim3 grid(M, (nq + 2 * nkv + 15) / 16);
  if (act == Act::F32)
    rope_launch<float, float>(head_dim, grid, s, qkv, qkv_ld, part, n_part, part_stride, q_gain,
                              k_gain, qk_norm, eps, rope_cos, rope_sin, k_layer, v_layer, max_seq,
                              start, nq, nkv);
  else if (kv16)
    rope_launch<uint16_t, f16_t>(head_dim, grid, s, qkv, qkv_ld, part, n_part, part_stride,
                                 q_gain, k_gain, qk_norm, eps, rope_cos, rope_sin, k_layer,
                                 v_layer, max_seq, start, nq, nkv);
  else
    rope_launch<uint16_t, uint16_t>(head_dim, grid, s, qkv, qkv_ld, part, n_part, part_stride,
                                    q_gain, k_gain, qk_norm, eps, rope_cos, rope_sin, k_layer,
                                    v_layer, max_seq, start, nq, nkv);
  return hipGetLastError();
}

// 8 weights loaded non-temporally: the LM head reads each once per call
typedef unsigned int lm_u32x4_t __attribute__((ext_vector_type(4)));
typedef float lm_f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8_w(const uint16_t* p, float v[8]) {
  const lm_u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const lm_u32x4_t*>(p));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8_w(const float* p, float v[8]) {
  const lm_f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const lm_f32x4_t*>(p));
  const lm_f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const lm_f32x4_t*>(p) + 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// LM head: each wavefront owns whole rows of W; a lane streams 16-byte chunks
// of the row, four chunks' loads in flight at a time, and the dot product ends
// in one wavefront reduction.  HBM-bound: the weight is read exactly once.
// (The chunks are summed in ascending order, as one chunk per step would.)
template <typename T>
__global__ __launch_bounds__(256) void lm_head_kernel(const float* __restrict__ xn,
                                                      const T* __restrict__ W,
                                                      float* __restrict__ logits, int V, int H) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const int chunks = H >> 3;
  for (int r = gw; r < V; r += nw) {
    const T* wr = W + static_cast<size_t>(r) * H;
    float acc = 0.f;
    for (int c0 = lane; c0 < chunks; c0 += 4 * 64) {
      float w[4][8], x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 64 * u;
        if (c < chunks) {
          load8_w(wr + c * 8, w[u]);
          load8(xn + c * 8, x[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + 64 * u < chunks)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc += w[u][i] * x[u][i];
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[r] = acc;
  }
}

hipError_t launch_lm_head(Act act, const float* xn, const void* W, float* logits, int V, int H,
                          hipStream_t s) {
  if (V <= 0) return hipSuccess;
  const int blocks = (V + 3) / 4 < 8192 ? (V + 3) / 4 : 8192;
  if (act == Act::F32)
    lm_head_kernel<float><<<blocks, 256, 0, s>>>(xn, static_cast<const float*>(W), logits, V, H);
  else
    lm_head_kernel<uint16_t><<<blocks, 256, 0, s>>>(xn, static_cast<const uint16_t*>(W), logits,
                                                    V, H);
  return hipGetLastError();
}

}  // namespace tlp

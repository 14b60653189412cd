// Shared device helpers for the gfx950 prefill kernels: element types,
// conversions, vector types for the MFMA builtins and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tlp {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// bf16 values travel as raw 16-bit patterns in memory.
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round-to-nearest-even float -> bf16 (gfx950 has a hardware convert).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// IEEE fp16 storage (KV-cache format); stores round to nearest-even.
typedef _Float16 f16_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Block-wide sum for blockDim.x == 64 * NW; every thread receives the total.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red /* LDS, NW floats */) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + lo + hi for a pair of fp16 values packed in one word
__device__ __forceinline__ float dot2_f16_sum(uint32_t pair, float acc) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pair),
                                __builtin_bit_cast(f16x2_t, 0x3C003C00u), acc, false);
}

// acc + lo + hi for a pair of bf16 values packed in one word (v_dot2 with 1.0)
__device__ __forceinline__ float dot2_bf16_sum(uint32_t pair, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

// 1-bit weight format: 8 bf16 weights from 8 sign bits (bit e -> element e; 1 -> +scale, 0 ->
// -scale) and the bf16 bit pattern of the scale: negating flips the sign bit.
__device__ __forceinline__ uint4 sign1_expand8(uint32_t bits8, uint32_t sbf) {
  const uint32_t ss = sbf | (sbf << 16);
  const uint32_t neg = ~bits8 & 0xffu;
  const uint32_t x2 = neg | (neg << 15);   // neg bit e at e, neg bit e at e + 15
  uint4 u;
  u.x = ss ^ ((x2 << 15) & 0x80008000u);
  u.y = ss ^ ((x2 << 13) & 0x80008000u);
  u.z = ss ^ ((x2 << 11) & 0x80008000u);
  u.w = ss ^ ((x2 << 9) & 0x80008000u);
  return u;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// 16-byte global -> LDS copy per lane (global_load_lds_dwordx4); `lds` must be
// the same for the whole wavefront (it becomes M0), lane l lands at lds + 16*l.
__device__ __forceinline__ void dma16(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

// Buffer-resource copy global -> LDS (buffer_load_dwordx4 ... lds): a
// wavefront-uniform descriptor (base address and byte size), a 32-bit
// per-lane byte offset and a scalar byte offset.  Stepping along K changes
// only the scalar offset, so a kernel keeps one 32-bit register per copy
// stream instead of a 64-bit address.  Lane l lands at lds + 16*l; `lds` must
// be wavefront-uniform (it becomes M0).
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ void tlp_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) uint32_t* lds,
                                    int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p)));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r.w = 0x00020000;   // raw buffer, 32-bit data format (GFX9 descriptor word 3)
  return r;
}

__device__ __forceinline__ void dma16_buf(i32x4_t rsrc, uint32_t voff, int soff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  tlp_buffer_load_lds(rsrc, (__attribute__((address_space(3))) uint32_t*)lds, 16,
                      static_cast<int>(voff), soff, 0, 0);
#endif
}

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (GFX9 layout)
template <int N>
struct VmWait {
  static constexpr int imm = (N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14);
};

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every outstanding global->LDS copy); LDS reads issued before it
// have completed.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane s supplies the address of 4 consecutive 16-bit values S[s][0..3]; lane i
// of the group receives S[4e + i/4][i%4] for e = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)p);
  return __builtin_bit_cast(uint2, v);
#else
  return make_uint2(0, 0);
#endif
}

}  // namespace tlp

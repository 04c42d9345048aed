// Shared device helpers for the gfx950 linear-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // four wavefronts per workgroup

// phi = ReLU on two packed bfloat16 values.  Comparing the raw bits as
// signed 16-bit integers against 0 keeps every value with a clear sign bit
// and clears every value with a set sign bit, which is max(x, 0) for every
// finite x (and -0 becomes +0).  One v_pk_max_i16 per pair.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t x) {
  s16x2 v = __builtin_bit_cast(s16x2, x);
  v = __builtin_elementwise_max(v, (s16x2){0, 0});
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint4 relu_bf16x8(uint4 x) {
  x.x = relu_bf16x2(x.x);
  x.y = relu_bf16x2(x.y);
  x.z = relu_bf16x2(x.z);
  x.w = relu_bf16x2(x.w);
  return x;
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16), one wavefront.
// Operand layout: lane l holds A[m = l % 16][k = 8 * (l / 16) + j] and
// B[k = 8 * (l / 16) + j][n = l % 16] for j = 0..7 (register element j);
// the result lane l holds D[m = 4 * (l / 16) + i][n = l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// float -> bfloat16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> bfloat16 hi/lo pairs, packed the way an MFMA operand holds
// consecutive k elements: *hi = {bf16(x0), bf16(x1)}, *lo = {bf16(x0 - hi0),
// bf16(x1 - hi1)}.  hi + lo carries 16 significant bits of each value.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t* hi, uint32_t* lo) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  const bf16x2 h = __builtin_convertvector(f32x2v{x0, x1}, bf16x2);
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xFFFF0000u);
  const bf16x2 l = __builtin_convertvector(f32x2v{x0 - h0, x1 - h1}, bf16x2);
  *hi = hb;
  *lo = __builtin_bit_cast(uint32_t, l);
}

// 1/x with v_rcp_f32 (1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float from_bf16(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Workgroup barrier for data exchanged through LDS only.  __syncthreads()
// also orders global memory, so the compiler waits for every outstanding
// global load (s_waitcnt vmcnt(0)) before it, including prefetches whose
// registers are not yet used: a kernel that loads tiles ahead in registers
// and stages them through LDS would drain its prefetch at every barrier.
// Fences on the LDS address space only leave "s_waitcnt lgkmcnt(0);
// s_barrier", and the global loads keep flying until their registers are
// read.  Use it only where no wave reads global memory another wave of the
// workgroup wrote before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Streaming (non-temporal) 16-byte load: data read exactly once.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

}  // namespace la

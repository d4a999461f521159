// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, storage-type conversions, fast exp2 and wave shuffles.
//
// MFMA operand layouts (checked on gfx950 with an in-bounds probe):
//   32x32x16 f16: lane l holds A[m = l%32][k = 8*(l/32) + i] and
//                 B[k = 8*(l/32) + i][n = l%32], i < 8; result element i of
//                 lane l is D[8*(i/4) + 4*(l/32) + i%4][l%32], i < 16.
//   16x16x32 f16: A[m = l%16][k = 8*(l/16) + i], B[k = 8*(l/16) + i][n = l%16];
//                 result i is D[4*(l/16) + i][l%16], i < 4.
//   16x16x16 f16: as 16x16x32 with k = 4*(l/16) + i, i < 4.
//   32x32x2  f32: A[m = l%32][k = l/32], B[k = l/32][n = l%32]; result as 32x32x16.
//   16x16x4  f32: A[m = l%16][k = l/16], B[k = l/16][n = l%16]; result as 16x16x32.
//   ds_read_tr16_b64: in each 16-lane group, lane a supplies the address of 4
//                 consecutive 16-bit values, read as row a/4, columns
//                 4*(a%4)..+3 of a 4x16 block; lane t receives column t of
//                 that block (rows 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvattn {

typedef _Float16 f16;
typedef f16 half2v __attribute__((ext_vector_type(2)));
typedef f16 half4v __attribute__((ext_vector_type(4)));
typedef f16 half8v __attribute__((ext_vector_type(8)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// storage type <-> float
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ---------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float16v mfma32x32x16(half8v a, half8v b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16x16x32(half8v a, half8v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16x16x16(half4v a, half4v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float16v mfma32x32x2f32(float a, float b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16x16x4f32(float a, float b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Wait for the last MFMA of a chain before its results are read.  The
// hardware needs several cycles after an MFMA issues before another
// instruction may read its destination registers; the compiler pads
// straight-line code correctly, but a read that follows a branch can be
// reached with too few wait states (seen as a partly accumulated last result
// element).  Call this after every MFMA chain whose results are consumed past
// control flow: it pins 24 wait states between the chain and what follows.
__device__ __forceinline__ void mfma_result_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// math
// ---------------------------------------------------------------------------
// v_exp_f32: 2^x, flushes to 0 for very negative x (and 2^-inf = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh(y) given u = 2 * log2(e) * y, within a few float32 ulps of the result:
// for |y| < 1/4 the odd Taylor polynomial through y^9 (the next term is below
// 1e-8 of the result), elsewhere 1 - 2 / (2^u + 1), whose cancellation there
// costs at most a factor of about three.  (1 - 2 / (2^u + 1) alone loses
// absolute, not relative, precision as y -> 0: after scaling by a large cap
// that is a visible error in a small score.)
__device__ __forceinline__ float tanh_from_u(float u) {
  if (fabsf(u) < 0.72134752f) {        // 0.25 * 2 * log2(e)
    const float y = u * 0.34657359f;   // ln(2) / 2
    const float y2 = y * y;
    float t = 62.f / 2835.f;
    t = fmaf(t, y2, -17.f / 315.f);
    t = fmaf(t, y2, 2.f / 15.f);
    t = fmaf(t, y2, -1.f / 3.f);
    return fmaf(t * y2, y, y);
  }
  return 1.f - 2.f * fast_rcp(fast_exp2(u) + 1.f);
}

// c * tanh(x / c) for c > 0.
__device__ __forceinline__ float softcap_apply(float x, float cap, float inv_cap) {
  return cap * tanh_from_u(2.0f * kLog2e * x * inv_cap);
}

// ---------------------------------------------------------------------------
// wave shuffles (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}
__device__ __forceinline__ float wave_max_xor(float v, int from_mask, int to_mask) {
  for (int m = from_mask; m <= to_mask; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum_xor(float v, int from_mask, int to_mask) {
  for (int m = from_mask; m <= to_mask; m <<= 1) v += shfl_xor(v, m);
  return v;
}

// ---------------------------------------------------------------------------
// 16-byte global loads of 8 storage elements (f16: one 16 B load; f32: two)
// ---------------------------------------------------------------------------
__device__ __forceinline__ half8v load_half8(const f16* p) {
  return *reinterpret_cast<const half8v*>(p);
}
__device__ __forceinline__ void store_half8(f16* p, half8v v) {
  *reinterpret_cast<half8v*>(p) = v;
}

template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&o)[8]);
template <>
__device__ __forceinline__ void load8_f32<f16>(const f16* p, float (&o)[8]) {
  half8v v = load_half8(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
template <>
__device__ __forceinline__ void load8_f32<float>(const float* p, float (&o)[8]) {
  float4v a = *reinterpret_cast<const float4v*>(p);
  float4v b = *reinterpret_cast<const float4v*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[i + 4] = b[i]; }
}

template <typename T>
__device__ __forceinline__ void store8_from_f32(T* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8_from_f32<f16>(f16* p, const float (&v)[8]) {
  half8v h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (f16)v[i];
  store_half8(p, h);
}
template <>
__device__ __forceinline__ void store8_from_f32<float>(float* p, const float (&v)[8]) {
  float4v a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[i + 4]; }
  *reinterpret_cast<float4v*>(p) = a;
  *reinterpret_cast<float4v*>(p + 4) = b;
}

}  // namespace kvattn

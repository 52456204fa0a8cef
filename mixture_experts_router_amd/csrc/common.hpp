// Device helpers shared by the layer's HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// activation dtype codes (same values as moe_dtype)
enum { ACT_F16 = 1, ACT_BF16 = 2 };

constexpr int WAVE = 64;

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(f16, (uint16_t)b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ float act_to_f32(uint32_t b, int act) {
  return act == ACT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32)
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (f16)v);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_act_bits(float v, int act) {
  return act == ACT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
}

// two bf16 (packed in a u32) -> two fp16 (packed), via fp32; exact for
// |v| in [2^-14, 65504]
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  f16x2 r;
  r.x = (f16)bf16_bits_to_f32(w & 0xFFFFu);
  r.y = (f16)bf16_bits_to_f32(w >> 16);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 activations (16 bytes) -> 8 fp16 values (16 bytes)
__device__ __forceinline__ u32x4 act8_to_f16(u32x4 v, int act) {
  if (act == ACT_BF16) {
    v.x = bf16x2_to_f16x2(v.x);
    v.y = bf16x2_to_f16x2(v.y);
    v.z = bf16x2_to_f16x2(v.z);
    v.w = bf16x2_to_f16x2(v.w);
  }
  return v;
}

// Reorder 8 fp16 values (k0..k7, packed in pairs) to the order in which a
// packed 4-bit word is unpacked: (k0,k4), (k1,k5), (k2,k6), (k3,k7).
__device__ __forceinline__ u32x4 perm8_nibble_order(u32x4 v) {
  // v.x = (k0,k1) v.y = (k2,k3) v.z = (k4,k5) v.w = (k6,k7); bytes: lo half first
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (k0, k4)
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (k1, k5)
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (k2, k6)
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (k3, k7)
  return r;
}

// ----------------------------------------------------- unpacking codes ---

// 8 packed 4-bit codes (one u32) -> four fp16 pairs holding 1024 + q, in the
// order (q0,q4) (q1,q5) (q2,q6) (q3,q7)
__device__ __forceinline__ void q4_word_to_biased_pairs(uint32_t v, uint32_t out[4]) {
  out[0] = (v & 0x000F000Fu) | 0x64006400u;
  out[1] = ((v >> 4) & 0x000F000Fu) | 0x64006400u;
  out[2] = ((v >> 8) & 0x000F000Fu) | 0x64006400u;
  out[3] = ((v >> 12) & 0x000F000Fu) | 0x64006400u;
}

// 4 bytes of 8-bit codes -> two fp16 pairs holding 1024 + q: (q0,q1) (q2,q3)
__device__ __forceinline__ void q8_word_to_biased_pairs(uint32_t v, uint32_t out[2]) {
  out[0] = __builtin_amdgcn_perm(0x64646464u, v, 0x04010400u);
  out[1] = __builtin_amdgcn_perm(0x64646464u, v, 0x04030402u);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// -------------------------------------------------------------- SwiGLU ---

// The one SwiGLU used by every path (fused epilogues and the standalone
// kernel), so fused and unfused results are bit-identical.
__device__ __forceinline__ float swiglu(float g, float u) {
  float e = expf(-g);
  float s = g / (1.0f + e);
  return s * u;
}

// ---------------------------------------------------------- reductions ---

// butterfly sum over the 64 lanes; every lane ends with the same value
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// non-temporal 16-byte load for streamed weights
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }

}  // namespace moe

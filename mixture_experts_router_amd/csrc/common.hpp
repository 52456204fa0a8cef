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

// ------------------------------------------- bf16 activations in range --
//
// bf16 activations reach the dot products and matrix cores as fp16 operands.
// To keep bf16's range, token t is converted as x * 2^-a_t, a_t >= 0 the
// smallest exponent with max|x_t| * 2^-a_t < 64: exact (powers of two only
// move the exponent) as long as the scaled values stay in fp16's normal
// range, and a_t = 0, the plain conversion, for every token whose largest
// activation is below 64.  The gate and up sums are scaled back by 2^a_t
// before SwiGLU; h and the down outputs are staged in fp16 at 2^-2a_t and
// the combine scales y back by 2^2a_t.

// largest |v| bit pattern of 8 bf16 values (for finite values the order of
// (bits & 0x7FFF) is the order of |v|)
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(u32x4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, w[i] & 0x7FFFu);
    m = max(m, (w[i] >> 16) & 0x7FFFu);
  }
  return m;
}

// a_t from the largest |x| bit pattern of the token: 2^(e-127) <= max|x| <
// 2^(e-126) for biased exponent e, so max|x| * 2^-a < 2^6 needs a >= e - 132
__device__ __forceinline__ int bf16_token_exp(uint32_t absmax_bits) {
  const int e = (int)(absmax_bits >> 7);
  return e > 132 ? e - 132 : 0;
}

__device__ __forceinline__ float ldexp_f(float v, int e) { return __builtin_amdgcn_ldexpf(v, e); }

// 8 activations (16 bytes) -> 8 fp16 values of x * 2^-a (a = 0 for fp16
// activations)
__device__ __forceinline__ u32x4 act8_to_f16_scaled(u32x4 v, int act, int a) {
  if (act != ACT_BF16) return v;
  if (a == 0) return act8_to_f16(v, act);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 r;
    r.x = (f16)ldexp_f(bf16_bits_to_f32(w[i] & 0xFFFFu), -a);
    r.y = (f16)ldexp_f(bf16_bits_to_f32(w[i] >> 16), -a);
    w[i] = __builtin_bit_cast(uint32_t, r);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
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

// The batched path's operand order for 4-bit weights: each 8-element block
// as (k0,k2) (k4,k6) (k1,k3) (k5,k7), the order in which the GEMM turns a
// word of eight codes into fp16 pairs (the low nibbles of its bytes, then
// the high nibbles).  From natural pairs (k0,k1) (k2,k3) (k4,k5) (k6,k7):
__device__ __forceinline__ u32x4 q4g_order(u32x4 v) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);  // (k0, k2)
  r.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);  // (k4, k6)
  r.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);  // (k1, k3)
  r.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);  // (k5, k7)
  return r;
}

// Inverse of q4g_order: (k0,k2) (k4,k6) (k1,k3) (k5,k7) -> k0..k7.
__device__ __forceinline__ u32x4 q4g_natural(u32x4 v) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (k0, k1)
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (k2, k3)
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (k4, k5)
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (k6, k7)
  return r;
}

// Position of element i (0..7) of an 8-element block in q4g order.
__device__ __forceinline__ int q4g_slot(int i) { return (i & 1) * 4 + (i >> 1); }

// ----------------------------------------------------- unpacking codes ---
//
// gfx9 VOP3 instructions cannot encode 32-bit literals, so (v & mask) | magic
// would compile to two instructions; with mask and magic held in registers it
// is one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(mask), "v"(magic));
  return r;
}

// Loop-invariant constants for unpacking 4-bit codes into fp16 numbers:
// exponent bits 0x6400 turn a code q in mantissa bits 0-3 into 1024 + q and a
// code in mantissa bits 4-7 into 1024 + 16 q.
struct Q4Consts {
  uint32_t lo, hi, magic;
};

__device__ __forceinline__ Q4Consts q4_consts() {
  Q4Consts c;
  c.lo = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  c.hi = __builtin_amdgcn_readfirstlane(0x00F000F0u);
  c.magic = __builtin_amdgcn_readfirstlane(0x64006400u);
  // keep them in VGPRs (one v_and_or_b32 may read at most one SGPR on gfx9)
  asm volatile("" : "+v"(c.lo), "+v"(c.hi), "+v"(c.magic));
  return c;
}

// 8 packed 4-bit codes (one u32: codes k0..k7, even k in the low nibble of
// each byte) -> four fp16 pairs: (k0,k4) and (k2,k6) holding 1024 + q, and
// (k1,k5) and (k3,k7) holding 1024 + 16 q.
__device__ __forceinline__ void q4_word_unpack(uint32_t v, const Q4Consts& c, uint32_t& p04, uint32_t& p15,
                                               uint32_t& p26, uint32_t& p37) {
  const uint32_t v8 = v >> 8;
  p04 = and_or(v, c.lo, c.magic);
  p15 = and_or(v, c.hi, c.magic);
  p26 = and_or(v8, c.lo, c.magic);
  p37 = and_or(v8, c.hi, c.magic);
}

// 8 packed 4-bit codes -> four fp16 pairs holding 1024 + q, in the order
// (q0,q4) (q1,q5) (q2,q6) (q3,q7)
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

// --------------------------------------------------------------- NVFP4 ---
//
// The E2M1 codes of a 32-bit word (eight codes, column 2i in the low nibble
// of byte i) as four fp16 pairs (columns 2i, 2i+1), exact: the gfx950
// conversion with a scale of 1 (the instruction takes only the exponent of
// its scale operand, so block scales are applied separately).
__device__ __forceinline__ void e2m1_word_to_pairs(uint32_t w, uint32_t (&p)[4]) {
  p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
  p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
  p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
  p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
}

// FP8 E4M3 byte B of v (OCP "fn" format on gfx950), exact in fp32
template <int B>
__device__ __forceinline__ float e4m3_byte(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, B);
}

// -------------------------------------------------------------- SwiGLU ---

// The one SwiGLU used by every path (fused epilogues and the standalone
// kernel), so fused and unfused results are bit-identical.  silu(g) =
// g / (1 + e^-g) with the hardware exponential and reciprocal (v_exp_f32,
// v_rcp_f32; about 1 ulp each), far inside the fp16 rounding of h.  For
// very negative g, e^-g overflows to inf and the reciprocal gives 0.
__device__ __forceinline__ float swiglu(float g, float u) {
  const float e = __expf(-g);
  const float s = g * __builtin_amdgcn_rcpf(1.0f + e);
  return s * u;
}

// ---------------------------------------------------------- reductions ---
//
// Cross-lane sums use DPP (data-parallel primitives: lane permutations fused
// into the VALU operand, no LDS round trip).  Pairs, quads, 8-lane halves and
// 16-lane rows are combined with the symmetric permutations quad_perm[1,0,3,2],
// quad_perm[2,3,0,1], row_half_mirror and row_mirror, so every lane of a row
// ends with the identical row total (a+b == b+a); the four row totals are then
// read from lanes 0/16/32/48 and added in row order.  The result is the same
// in every lane and independent of timing.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

constexpr int DPP_QUAD_1032 = 0xB1;
constexpr int DPP_QUAD_2301 = 0x4E;
constexpr int DPP_QUAD_2323 = 0xEE;  // lanes 0,1 of a quad read lanes 2,3
constexpr int DPP_QUAD_1111 = 0x55;  // every lane of a quad reads lane 1
constexpr int DPP_ROW_ROR4 = 0x124;  // rotate a 16-lane row by 4 lanes
constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// sum over the 64 lanes; every lane ends with the same value
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<DPP_QUAD_1032>(v);
  v += dpp_f<DPP_QUAD_2301>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f<DPP_ROW_MIRROR>(v);
  const float r0 = readlane_f(v, 0), r1 = readlane_f(v, 16), r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
  return ((r0 + r1) + r2) + r3;
}

// unsigned maximum over the 64 lanes; every lane ends with the same value
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<DPP_QUAD_1032>((int)v));
  v = max(v, (uint32_t)dpp_i<DPP_QUAD_2301>((int)v));
  v = max(v, (uint32_t)dpp_i<DPP_ROW_HALF_MIRROR>((int)v));
  v = max(v, (uint32_t)dpp_i<DPP_ROW_MIRROR>((int)v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  const float r0 = readlane_f(v, 0), r1 = readlane_f(v, 16), r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// value of `v` in lane `src` (ds_bpermute: the LDS crossbar, no LDS memory)
__device__ __forceinline__ float lane_read_f(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

// Sums of R per-lane partials (R = 1, 2 or 4 rows) over the 64 lanes.  On
// return, lane l (l < R) holds the total of row l; every lane holds the total
// of row l % R.  The partials are first transposed between neighbouring lanes
// (each exchange sends the half the partner keeps), so one butterfly reduces
// all R rows at once.  Every row total is formed by the same expression
// (pairs, then quads, then 16-lane rows, then halves; additions commute
// exactly), whatever the row's position among the R, so a row sums to the
// same bits in any kernel that reduces it with this function.
template <int R>
__device__ __forceinline__ float reduce_rows(const float (&p)[R]) {
  static_assert(R == 1 || R == 2 || R == 4, "1, 2 or 4 rows");
  const int lane = lane_id();
  float v;
  if constexpr (R == 4) {
    const bool o1 = lane & 1, o2 = lane & 2;
    const float k01 = o1 ? p[1] : p[0], s01 = o1 ? p[0] : p[1];
    const float k23 = o1 ? p[3] : p[2], s23 = o1 ? p[2] : p[3];
    const float r01 = k01 + dpp_f<DPP_QUAD_1032>(s01);  // rows 0|1 over the lane pair
    const float r23 = k23 + dpp_f<DPP_QUAD_1032>(s23);  // rows 2|3
    const float k = o2 ? r23 : r01, s = o2 ? r01 : r23;
    v = k + dpp_f<DPP_QUAD_2301>(s);  // row lane%4 over the quad
  } else if constexpr (R == 2) {
    const bool o1 = lane & 1;
    const float k = o1 ? p[1] : p[0], s = o1 ? p[0] : p[1];
    v = k + dpp_f<DPP_QUAD_1032>(s);
    v = v + dpp_f<DPP_QUAD_2301>(v);
  } else {
    v = p[0] + dpp_f<DPP_QUAD_1032>(p[0]);
    v = v + dpp_f<DPP_QUAD_2301>(v);
  }
  v = v + dpp_f<DPP_ROW_ROR4>(v);
  v = v + dpp_f<DPP_ROW_ROR8>(v);
  v = v + lane_read_f(v, lane ^ 16);
  v = v + lane_read_f(v, lane ^ 32);
  return v;
}

// Index of the calling wave in its workgroup, marked wave-uniform (so values
// derived from it live in scalar registers and branches on it stay scalar).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE)); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ------------------------------------------------------ buffer loads ----
//
// Streamed weights are read with buffer instructions: the row's base address
// lives in scalar registers (its arithmetic runs on the scalar unit) and
// every lane adds a fixed byte offset.  A resource of size 0 makes a load
// return zeros without touching memory (the hardware range check), which is
// how loads issued past the end of a wave's work stay harmless.

typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 buffer format word: raw 32-bit data
constexpr int AUX_NT = 2;               // cache policy: non-temporal (read once)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_WORD3);
}

__device__ __forceinline__ u32x4 buf_load16_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX_NT);
}

__device__ __forceinline__ uint32_t buf_load_u16_nt(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, AUX_NT);
}

// non-temporal 16-byte load for streamed weights
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }

// The GEMM operand row of token t: the activations as fp16, each 8-element
// block optionally in the 4-bit GEMM order (q4g_order).  bf16 rows are
// converted as x * 2^-a_t (exact) and a_t is written to tokexp[t], raising
// *any_scaled when a_t > 0; fp16 rows are copied.  One 256-thread group of a
// workgroup per token; every thread of the workgroup calls it (the bf16 form
// has a workgroup barrier), `live` false for a group past the last token.
// wmax: four words of LDS for this group.
__device__ __forceinline__ void prep_a_row(const uint16_t* __restrict__ x, uint16_t* __restrict__ a, int64_t t,
                                           bool live, int H, int act, int perm8, int32_t* __restrict__ tokexp,
                                           int32_t* __restrict__ any_scaled, int tid, uint32_t* wmax) {
  const uint16_t* xr = x + t * H;
  uint16_t* ar = a + t * H;
  int e = 0;
  if (act == ACT_BF16) {
    uint32_t m = 0;
    if (live)
      for (int c = tid * 8; c < H; c += 256 * 8) m = max(m, bf16x8_absmax_bits(load16(xr + c)));
    m = wave_max_u32(m);
    if (lane_id() == 0) wmax[tid / WAVE] = m;
    __syncthreads();
    e = bf16_token_exp(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
    if (live && tid == 0) {
      tokexp[t] = e;
      if (e != 0) *any_scaled = 1;  // every writer stores the same value
    }
  }
  if (!live) return;
  for (int c = tid * 8; c < H; c += 256 * 8) {
    u32x4 v = act8_to_f16_scaled(load16(xr + c), act, e);
    if (perm8) v = q4g_order(v);
    *(u32x4*)(ar + c) = v;
  }
}

}  // namespace moe

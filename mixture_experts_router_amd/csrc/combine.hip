// Small element-wise kernels: the routing-weighted combine, the standalone
// SwiGLU of the unfused path, and copies for the optional taps.
//
// Combine: y[t, :] = sum_{s < k} w[t, s] * o[t, s, :], summed in slot order in
// fp32 and rounded once to the activation dtype (page "Qwen3.5 Block在llama.cpp
// 中的映射与优化原理", section 4.2: the routing weight multiplies each selected
// expert's output after its FFN).  One thread owns 8 consecutive output
// elements, so no atomics are needed and the result is deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o, const int32_t* __restrict__ pos,
                                                      const float* __restrict__ wts,
                                                      const int32_t* __restrict__ k_used, int k_static, int kcap,
                                                      int H, void* __restrict__ y, int act,
                                                      const int32_t* __restrict__ tokexp) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  const int ku = k_used ? *k_used : k_static;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int s = 0; s < ku; ++s) {
    const size_t p = (size_t)t * kcap + s;
    if (pos[p] < 0) continue;  // dropped by the expert capacity
    const float ws = wts[p];
    const u32x4 v = load16(o + (size_t)pos[p] * H + c);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = ws * f16_bits_to_f32(w4[i] & 0xFFFFu);
      const float hi = ws * f16_bits_to_f32(w4[i] >> 16);
      acc[2 * i] = acc[2 * i] + lo;
      acc[2 * i + 1] = acc[2 * i + 1] + hi;
    }
  }
  if (tokexp) {  // o was staged at 2^-2a_t (exact scaling back)
    const int e2 = 2 * tokexp[t];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = ldexp_f(acc[i], e2);
  }
  u32x4 out;
  uint32_t* ow = (uint32_t*)&out;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ow[i] = (uint32_t)f32_to_act_bits(acc[2 * i], act) | ((uint32_t)f32_to_act_bits(acc[2 * i + 1], act) << 16);
  *(u32x4*)((uint16_t*)y + (size_t)t * H + c) = out;
}

hipError_t launch_combine(const uint16_t* o, const int32_t* pos, const float* wts, const int32_t* k_used_dev,
                          int k_static, int kcap, int T, int H, void* y, int act, hipStream_t st,
                          const int32_t* tokexp) {
  dim3 grid((H / 8 + 255) / 256, T);
  launch_kernel(combine_kernel, grid, 256, 0, st, o, pos, wts, k_used_dev, k_static, kcap, H, y, act, tokexp);
  return hipGetLastError();
}

// h = 2^-2a silu(g) * u (a: the row's token exponent, 0 without tokexp);
// with perm8 set, each 8-element block of h is stored in the 4-bit GEMM order (q4g_order)
// (the operand order of the batched 4-bit down GEMM).
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                     uint16_t* __restrict__ h, int64_t n, int I, int perm8,
                                                     const int32_t* __restrict__ tokexp,
                                                     const int32_t* __restrict__ perm, int kcap) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t at = perm8 ? (i & ~(int64_t)7) + q4g_slot((int)(i & 7)) : i;
  float hv = swiglu(g[i], u[i]);
  if (tokexp) {
    const int64_t row = i / I;
    const int64_t pair = perm ? perm[row] : row;  // perm is -1 past the sorted pairs (rows never read)
    if (pair >= 0) hv = ldexp_f(hv, -2 * tokexp[pair / kcap]);
  }
  h[at] = f32_to_f16_bits(hv);
}

hipError_t launch_swiglu(const float* g, const float* u, uint16_t* h, int64_t rows, int I, bool perm8,
                         hipStream_t st, const int32_t* tokexp, const int32_t* perm, int kcap) {
  const int64_t n = rows * I;
  launch_kernel(swiglu_kernel, (unsigned)((n + 255) / 256), 256, 0, st, g, u, h, n, I, perm8 ? 1 : 0, tokexp, perm,
                kcap);
  return hipGetLastError();
}

// Rows of h in pair order (taps); perm8 restores the natural element order
// of rows stored in the 4-bit GEMM order.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ pos, int I,
                                                          uint16_t* __restrict__ out, int kcap,
                                                          const int32_t* __restrict__ k_used, int k_static,
                                                          int perm8) {
  const int64_t p = blockIdx.y;
  int64_t r;
  if (pos) {
    r = pos[p];
  } else {
    const int ku = k_used ? *k_used : k_static;
    r = (int)(p % kcap) < ku ? p : -1;
  }
  if (r < 0) return;
  for (int c = (blockIdx.x * 256 + threadIdx.x) * 8; c < I; c += gridDim.x * 256 * 8) {
    u32x4 v = load16(src + (size_t)r * I + c);
    if (perm8) v = q4g_natural(v);
    *(u32x4*)(out + p * I + c) = v;
  }
}

hipError_t launch_gather_rows(const uint16_t* src, const int32_t* pos, int64_t P, int I, uint16_t* out, int kcap,
                              const int32_t* k_used_dev, int k_static, bool perm8, hipStream_t st) {
  dim3 grid((I / 8 + 255) / 256, (unsigned)P);
  launch_kernel(gather_rows_kernel, grid, 256, 0, st, src, pos, I, out, kcap, k_used_dev, k_static, perm8 ? 1 : 0);
  return hipGetLastError();
}

// The fp32 gate and up rows of the unfused paths, side by side in pair order
// (the gate_up_preact tap).
__global__ __launch_bounds__(256) void gather_preact_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                            const int32_t* __restrict__ pos, int I,
                                                            float* __restrict__ pre, int kcap,
                                                            const int32_t* __restrict__ k_used, int k_static) {
  const int64_t p = blockIdx.y;
  int64_t r;
  if (pos) {
    r = pos[p];
  } else {
    const int ku = k_used ? *k_used : k_static;
    r = (int)(p % kcap) < ku ? p : -1;
  }
  if (r < 0) return;
  for (int c = (blockIdx.x * 256 + threadIdx.x) * 4; c < 2 * I; c += gridDim.x * 256 * 4) {
    const float* src = c < I ? g + (size_t)r * I + c : u + (size_t)r * I + (c - I);
    *(f32x4*)(pre + p * 2 * I + c) = *(const f32x4*)src;
  }
}

hipError_t launch_gather_preact(const float* g, const float* u, const int32_t* pos, int64_t P, int I, float* pre,
                                int kcap, const int32_t* k_used_dev, int k_static, hipStream_t st) {
  if (I % 4 != 0) return hipErrorInvalidValue;
  dim3 grid((2 * I / 4 + 255) / 256, (unsigned)P);
  launch_kernel(gather_preact_kernel, grid, 256, 0, st, g, u, pos, I, pre, kcap, k_used_dev, k_static);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy_words_kernel(const uint32_t* __restrict__ s, uint32_t* __restrict__ d,
                                                         int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) d[i] = s[i];
}

hipError_t launch_copy_words(const void* src, void* dst, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  launch_kernel(copy_words_kernel, (unsigned)((n + 255) / 256), 256, 0, st, (const uint32_t*)src, (uint32_t*)dst, n);
  return hipGetLastError();
}

// Scales and biases [rows, ng] (fp16, rows e*src_stride + n) -> the packed
// layout of the batched path: 8 bytes {s[2p], s[2p+1], b[2p], b[2p+1]} per
// (expert e, group pair p, row n) at ((e*NP + p)*dst_stride + dst_row0 + n)*8;
// a group past ng is 0.  One thread per element, rows fastest (coalesced
// stores).
__global__ __launch_bounds__(256) void pack_sb_kernel(const uint16_t* __restrict__ s, const uint16_t* __restrict__ b,
                                                      int N, int ng, int NP, int64_t src_stride, uint8_t* dst,
                                                      int64_t dst_stride, int64_t dst_row0, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int n = (int)(i % N);
  const int64_t ep = i / N;  // e*NP + p
  const int p = (int)(ep % NP);
  const int64_t e = ep / NP;
  const int64_t src = (e * src_stride + n) * ng;
  const int g0 = 2 * p, g1 = 2 * p + 1;
  const uint32_t s0 = s[src + g0], b0 = b[src + g0];
  const uint32_t s1 = g1 < ng ? s[src + g1] : 0u, b1 = g1 < ng ? b[src + g1] : 0u;
  *(u32x2*)(dst + (ep * dst_stride + dst_row0 + n) * 8) = u32x2{s0 | (s1 << 16), b0 | (b1 << 16)};
}

// NVFP4: slot (e, p, n) holds the four E4M3 block scales of group 2p (one
// 32-bit word of the row's scale bytes) and those of group 2p+1 (0 if none)
__global__ __launch_bounds__(256) void pack_sb_f4_kernel(const uint32_t* __restrict__ s, int N, int ng, int NP,
                                                         int64_t src_stride, uint8_t* dst, int64_t dst_stride,
                                                         int64_t dst_row0, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int n = (int)(i % N);
  const int64_t ep = i / N;
  const int p = (int)(ep % NP);
  const int64_t e = ep / NP;
  const int64_t src = (e * src_stride + n) * ng;  // the row's group words
  const int g0 = 2 * p, g1 = 2 * p + 1;
  const uint32_t w0 = s[src + g0], w1 = g1 < ng ? s[src + g1] : 0u;
  *(u32x2*)(dst + (ep * dst_stride + dst_row0 + n) * 8) = u32x2{w0, w1};
}

hipError_t launch_pack_sb(const uint16_t* s, const uint16_t* b, int E, int N, int K, int64_t src_stride, uint8_t* dst,
                          int64_t dst_stride, int64_t dst_row0, hipStream_t st, bool nvfp4) {
  const int ng = K / 64, NP = (ng + 1) / 2;
  const int64_t total = (int64_t)E * NP * N;
  if (total <= 0) return hipSuccess;
  if ((total + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (nvfp4)
    launch_kernel(pack_sb_f4_kernel, (unsigned)((total + 255) / 256), 256, 0, st, (const uint32_t*)s, N, ng, NP,
                  src_stride, dst, dst_stride, dst_row0, total);
  else
    launch_kernel(pack_sb_kernel, (unsigned)((total + 255) / 256), 256, 0, st, s, b, N, ng, NP, src_stride, dst,
                  dst_stride, dst_row0, total);
  return hipGetLastError();
}

// ---------------------------------------------------------- packed_q ---
//
// One thread per 16-byte piece of the packed_q layout (moe.h): piece c of
// row r of 32-row block j, unit p (one or two groups), expert e.  Source rows are read as
// 32-bit words (5-bit rows are only 8-byte aligned); words past the row's
// code bytes (a missing last group) and rows at or past N are zero.
__global__ __launch_bounds__(256) void pack_q_kernel(const uint8_t* __restrict__ q, int N, int rb, int pb, int np,
                                                     int nb_src, int nb_dst, int64_t src_stride,
                                                     uint8_t* __restrict__ dst, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int ppr = pb / 16;
  int64_t rest = i;
  const int c = (int)(rest % ppr);
  rest /= ppr;
  const int r = (int)(rest % 32);
  rest /= 32;
  const int p = (int)(rest % np);
  rest /= np;
  const int j = (int)(rest % nb_src);
  const int64_t e = rest / nb_src;
  const int n = 32 * j + r;
  const int64_t col = (int64_t)p * pb + (int64_t)c * 16;  // byte within the row's codes
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (n < N) {
    const uint32_t* src = (const uint32_t*)(q + (e * src_stride + n) * rb);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (col + 4 * u < rb) w[u] = src[(col >> 2) + u];
  }
  *(u32x4*)(dst + (((e * nb_dst + j) * np + p) * 32 + r) * pb + c * 16) = u32x4{w[0], w[1], w[2], w[3]};
}

hipError_t launch_pack_q(const uint8_t* q, int E, int N, int K, int bits, int64_t src_stride, uint8_t* dst,
                         int64_t dst_stride, hipStream_t st) {
  const int rb = K * code_bits(bits) / 8;
  const int pb = (int)packed_q_unit_bytes(bits);
  const int np = (int)packed_q_units(K, bits);
  const int nb_src = (N + 31) / 32;
  const int nb_dst = (int)((dst_stride + 31) / 32);
  const int64_t total = (int64_t)E * nb_src * np * 32 * (pb / 16);
  if (total <= 0) return hipSuccess;
  if ((total + 255) / 256 > 0x7FFFFFFF || rb % 4 != 0) return hipErrorInvalidValue;
  launch_kernel(pack_q_kernel, (unsigned)((total + 255) / 256), 256, 0, st, q, N, rb, pb, np, nb_src, nb_dst,
                src_stride, dst, total);
  return hipGetLastError();
}

// ------------------------------------------------------- stream read ---
//
// The practical read ceiling for weight-streaming kernels: 16-byte
// non-temporal buffer loads, four per lane in flight, each of 2048
// workgroups streaming its own contiguous segment of the range (measured
// 6.7-7.0 TB/s at 0.3-1 GB, against 5.5-6.1 TB/s when all workgroups sweep
// the range together grid-stride).  Loads past the end go through the
// descriptor's range check and read nothing.
constexpr int STREAM_BLOCKS = 2048;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ src, uint32_t bytes,
                                                          uint32_t* __restrict__ sink) {
  const rsrc_t r = make_rsrc(src, bytes);
  // ceil(bytes / blocks) rounded up to whole 4 KB pieces: the segments cover the range
  const uint64_t seg = (((uint64_t)bytes + STREAM_BLOCKS - 1) / STREAM_BLOCKS + 4095u) & ~(uint64_t)4095u;
  const uint64_t b0 = (uint64_t)blockIdx.x * seg, b1 = b0 + seg;
  uint32_t acc = 0;
  for (uint64_t o0 = b0 + threadIdx.x * 16u; o0 < b1; o0 += 4u * 4096u) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t o = o0 + (uint64_t)u * 4096u;  // 256 lanes x 16 B = one 4 KB piece per load
      v[u] = (o < b1 && o < bytes) ? buf_load16_nt(r, (uint32_t)o) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) acc ^= __shfl_xor(acc, d, WAVE);
  if (lane_id() == 0) sink[blockIdx.x * 4 + wave_id()] = acc;
}

hipError_t launch_stream_read(const void* src, uint32_t bytes, uint32_t* sink, hipStream_t st) {
  launch_kernel(stream_read_kernel, STREAM_BLOCKS, 256, 0, st, (const uint8_t*)src, bytes, sink);
  return hipGetLastError();
}

}  // namespace moe

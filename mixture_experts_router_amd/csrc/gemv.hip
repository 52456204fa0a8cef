// Decode path: grouped GEMV over the selected experts only.
//
// Only the k experts a token selected are read (page "Qwen3.5 Block在llama.cpp
// 中的映射与优化原理", section 4.2: compute the top-k experts, not all 64),
// so the weight bytes streamed per token are those of k experts.
//
// gate+up (fused tensor [E, 2*inter, H], gate rows first; oMLX gate/up page,
// "融合原理") with the SwiGLU epilogue h = silu(g) * u; down projection with
// the routing-weighted combine y = sum_s w_s * o_s in slot order.
//
// Dequantisation happens in registers and is factored out of the dot
// product.  For a 16-byte chunk of codes q with scale s and bias b,
//     sum_k x_k (s q_k + b) = s * sum_k x_k q_k + b * X,     X = sum_k x_k.
// A 32-bit word of eight 4-bit codes becomes four fp16 pairs with one shift
// and four v_and_or_b32: exponent bits 0x6400 make a code in mantissa bits 0-3
// the number 1024 + q and a code in bits 4-7 the number 1024 + 16 q.  So
//     sum_k x_k q_k = (A - 1024 Xa) + (B - 1024 Xb) / 16,
// where A and B are v_dot2_f32_f16 sums (fp32 accumulation) over the two
// kinds of pairs and Xa, Xb the matching activation sums, computed once per
// wave.  8-bit codes use v_perm_b32 to build 1024 + q pairs the same way.
// About 1.4 VALU operations per 4-bit weight.
//
// Lane l of a wave owns the 16-byte chunks c = l + 64*i of every row, so one
// load instruction covers 1 KB of contiguous weights.  The chunk loops have no
// per-lane branches (a lane past the end of a row re-reads the last chunk and
// masks its contribution), so every load is issued ahead of its use.  Each
// row's 64 lane partials are summed with a DPP butterfly; the same row code
// serves the fused (gate+up+SwiGLU) and the single-projection kernels, so both
// round identically.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {

// Route token t inside a decode kernel: with logits given (static k), every
// wave recomputes the token's selection (topk.hpp, identical in all kernels)
// instead of waiting for a separate selection launch.
struct RouteSrc {
  const float* logits;  // [T, E] or NULL: read idx/wts
  int E;
  int32_t* idx;         // [T, kcap]: output when logits is given, else input
  float* wts;
  int32_t* k_used;      // device scalar: output when logits is given, else input (may be NULL)
  float* entropy;
};

template <typename F>
__device__ __forceinline__ void for_slot(int s, F f) {
#pragma unroll
  for (int j = 0; j < MOE_MAX_K_DEV; ++j)
    if (j == s) f(j);
}

template <int BITS>
struct Chunk {
  static constexpr int VALS = BITS == 4 ? 32 : (BITS == 8 ? 16 : 8);  // weights per 16 bytes
  static constexpr int PAIRS = VALS / 2;                               // fp16 pairs of activations
  static constexpr int PER_GROUP = 64 / VALS;                          // chunks per 64-column group
  static constexpr int PIECES = VALS / 8;                              // 16-byte activation pieces
};

int gemv_lanes_chunks(int K, int bits) {
  int vals = bits == 4 ? 32 : (bits == 8 ? 16 : 8);
  return (K / vals + 63) / 64;
}

// Per-chunk activation terms: 1024 * (sum over the 1024+q pairs),
// 1024 * (sum over the 1024+16q pairs), and the plain sum.
struct XSums {
  float ca, cb, x;
};

// Activation sums of one chunk held as fp16 pairs in unpack order.
template <int BITS>
__device__ __forceinline__ XSums chunk_xsums(const uint32_t* xp) {
  XSums r = {0.0f, 0.0f, 0.0f};
  if constexpr (BITS == 4) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int j = 0; j < Chunk<4>::PAIRS; ++j) {
      const f16x2 hp = __builtin_bit_cast(f16x2, xp[j]);
      const float s2 = (float)hp.x + (float)hp.y;
      if ((j & 1) == 0) a += s2;  // pairs (k0,k4), (k2,k6)
      else b += s2;               // pairs (k1,k5), (k3,k7)
    }
    r.ca = 1024.0f * a;
    r.cb = 1024.0f * b;
    r.x = a + b;
  } else if constexpr (BITS == 8) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < Chunk<8>::PAIRS; ++j) {
      const f16x2 hp = __builtin_bit_cast(f16x2, xp[j]);
      a += (float)hp.x + (float)hp.y;
    }
    r.ca = 1024.0f * a;
    r.x = a;
  }
  return r;
}

// Contribution of one 16-byte chunk of weights to its row (affine terms applied).
template <int BITS>
__device__ __forceinline__ float chunk_value(u32x4 w, const uint32_t* xp, const XSums& xs, uint32_t s_bits,
                                             uint32_t b_bits, const Q4Consts& qc) {
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  if constexpr (BITS == 4) {
    float A = 0.0f, B = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p04, p15, p26, p37;
      q4_word_unpack(wv[j], qc, p04, p15, p26, p37);
      A = dot2(p04, xp[4 * j + 0], A);
      B = dot2(p15, xp[4 * j + 1], B);
      A = dot2(p26, xp[4 * j + 2], A);
      B = dot2(p37, xp[4 * j + 3], B);
    }
    const float qa = A - xs.ca;
    const float qb = B - xs.cb;
    const float dq = qa + 0.0625f * qb;
    const float s = f16_bits_to_f32(s_bits), b = f16_bits_to_f32(b_bits);
    return s * dq + b * xs.x;
  } else if constexpr (BITS == 8) {
    float A = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p[2];
      q8_word_to_biased_pairs(wv[j], p);
      A = dot2(p[0], xp[2 * j], A);
      A = dot2(p[1], xp[2 * j + 1], A);
    }
    const float dq = A - xs.ca;
    const float s = f16_bits_to_f32(s_bits), b = f16_bits_to_f32(b_bits);
    return s * dq + b * xs.x;
  } else {
    float A = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) A = dot2(wv[j], xp[j], A);
    return A;
  }
}

// ------------------------------------------------------------- gate + up --

struct GemvUpParams {
  const uint16_t* x;
  int act;
  RouteSrc rt;
  int k_static, kcap;
  int H, N;  // N: output columns (fused: inter) or rows (single)
  WView w0, w1;
  uint16_t* h;
  float* out32;
  int iters;  // row-iterations per pair
  int iters_per_wave;
};

// rows per iteration: 4 for short rows, 2 when a lane holds more chunks
// (keeps two iterations of loads in registers without spilling)
template <int CPL>
struct Rows {
  static constexpr int N = CPL <= 2 ? 4 : 2;
};

// raw bytes of one iteration's rows, as seen by one lane
template <int BITS, int CPL>
struct RowBuf {
  static constexpr int R = Rows<CPL>::N;
  u32x4 q[R][CPL];
  uint32_t s[R][CPL], b[R][CPL];
};

// Row r of iteration `it`.  Fused: the first half of the rows are gate rows
// j, the second half the up rows j of the same output columns.  Single: R
// consecutive rows of one projection.
template <int CPL, bool FUSED>
__device__ __forceinline__ int row_of(int it, int r) {
  constexpr int R = Rows<CPL>::N;
  return FUSED ? (R / 2) * it + (r % (R / 2)) : R * it + r;
}

template <int BITS, int CPL, bool FUSED>
__device__ __forceinline__ void load_rows(RowBuf<BITS, CPL>& buf, const GemvUpParams& prm, int e, int it,
                                          const int* cc, int ng, int64_t row_bytes) {
  using C = Chunk<BITS>;
  constexpr int R = Rows<CPL>::N;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const WView& wv = (FUSED && r >= R / 2) ? prm.w1 : prm.w0;
    const int64_t row = (int64_t)e * wv.stride + row_of<CPL, FUSED>(it, r);
    const uint8_t* rq = wv.q + row * row_bytes;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      buf.q[r][i] = load_stream16(rq + (size_t)cc[i] * 16);
      if constexpr (BITS != 16) {
        buf.s[r][i] = wv.s[row * ng + cc[i] / C::PER_GROUP];
        buf.b[r][i] = wv.b[row * ng + cc[i] / C::PER_GROUP];
      }
    }
  }
}

template <int BITS, int CPL, bool FUSED>
__device__ __forceinline__ void finish_iter(const RowBuf<BITS, CPL>& buf, const GemvUpParams& prm, int p, int it,
                                            const uint32_t (*xr)[Chunk<BITS>::PAIRS], const XSums* xs,
                                            const bool* valid, const Q4Consts& qc) {
  constexpr int R = Rows<CPL>::N;
  float part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float v = chunk_value<BITS>(buf.q[r][i], xr[i], xs[i], buf.s[r][i], buf.b[r][i], qc);
      acc += valid[i] ? v : 0.0f;
    }
    part[r] = wave_sum(acc);
  }
  if (lane_id() == 0) {
    if constexpr (FUSED) {
      if constexpr (R == 4) {
        const int j = 2 * it;
        const uint32_t h0 = f32_to_f16_bits(swiglu(part[0], part[2]));
        const uint32_t h1 = f32_to_f16_bits(swiglu(part[1], part[3]));
        *(uint32_t*)(prm.h + (size_t)p * prm.N + j) = h0 | (h1 << 16);
      } else {
        prm.h[(size_t)p * prm.N + it] = f32_to_f16_bits(swiglu(part[0], part[1]));
      }
    } else {
      if constexpr (R == 4) {
        const f32x4 o = {part[0], part[1], part[2], part[3]};
        *(f32x4*)(prm.out32 + (size_t)p * prm.N + R * it) = o;
      } else {
        prm.out32[(size_t)p * prm.N + R * it] = part[0];
        prm.out32[(size_t)p * prm.N + R * it + 1] = part[1];
      }
    }
  }
}

template <int BITS, int CPL, bool FUSED>
__global__ __launch_bounds__(256) void gemv_up_kernel(GemvUpParams prm) {
  using C = Chunk<BITS>;
  const int lane = lane_id();
  const int p = blockIdx.y;
  const int t = p / prm.kcap, slot = p % prm.kcap;
  const int ku = prm.rt.logits ? prm.k_static : *prm.rt.k_used;
  if (slot >= ku) return;
  // iterations it = gw, gw + W, gw + 2W, ...: at any moment the waves of a
  // pair read one contiguous stretch of rows, so each expert is swept linearly
  const int gw = blockIdx.x * 4 + threadIdx.x / WAVE;
  const int W = gridDim.x * 4;
  if (gw >= prm.iters) return;
  int e;
  if (prm.rt.logits) {
    int si[MOE_MAX_K_DEV];
    float sw[MOE_MAX_K_DEV];
    route_token(prm.rt.logits + (size_t)t * prm.rt.E, prm.rt.E, ku, si, sw);
    float wsel = 0.0f;
    e = 0;
    for_slot(slot, [&](int j) {
      e = si[j];
      wsel = sw[j];
    });
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      prm.rt.idx[p] = e;
      prm.rt.wts[p] = wsel;
      if (p == 0) {
        *prm.rt.k_used = ku;
        *prm.rt.entropy = 0.0f;
      }
    }
  } else {
    e = prm.rt.idx[p];
  }
  e = __builtin_amdgcn_readfirstlane(e);  // uniform: row addressing stays scalar
  const int H = prm.H;
  const int nch = H / C::VALS;
  const int ng = H / 64;
  const int64_t row_bytes = (int64_t)H * BITS / 8;
  const Q4Consts qc = q4_consts();

  int cc[CPL];
  bool valid[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    valid[i] = c < nch;
    cc[i] = valid[i] ? c : nch - 1;
  }

  // first rows in flight before the activations are prepared
  // rows in flight before the activations are prepared; short rows keep two
  // iterations ahead of the one being reduced, long rows one
  constexpr bool DEEP = CPL <= 2;
  RowBuf<BITS, CPL> bufA, bufB, bufC;
  const int it1 = prm.iters;
  load_rows<BITS, CPL, FUSED>(bufA, prm, e, gw, cc, ng, row_bytes);
  if (DEEP && gw + W < it1) load_rows<BITS, CPL, FUSED>(bufB, prm, e, gw + W, cc, ng, row_bytes);

  // activations of this lane's chunks, as fp16 pairs in the unpack order
  uint32_t xr[CPL][C::PAIRS];
  XSums xs[CPL];
  const uint16_t* xrow = prm.x + (size_t)t * H;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
#pragma unroll
    for (int j = 0; j < C::PIECES; ++j) {
      u32x4 v = act8_to_f16(load16(xrow + (size_t)cc[i] * C::VALS + 8 * j), prm.act);
      if constexpr (BITS == 4) v = perm8_nibble_order(v);
      xr[i][4 * j + 0] = v.x;
      xr[i][4 * j + 1] = v.y;
      xr[i][4 * j + 2] = v.z;
      xr[i][4 * j + 3] = v.w;
    }
    xs[i] = chunk_xsums<BITS>(xr[i]);
  }

  // two row buffers: the next iteration's loads are in flight while the
  // current one is reduced
  if constexpr (DEEP) {
    for (int it = gw; it < it1; it += 3 * W) {
      if (it + 2 * W < it1) load_rows<BITS, CPL, FUSED>(bufC, prm, e, it + 2 * W, cc, ng, row_bytes);
      finish_iter<BITS, CPL, FUSED>(bufA, prm, p, it, xr, xs, valid, qc);
      if (it + W < it1) {
        if (it + 3 * W < it1) load_rows<BITS, CPL, FUSED>(bufA, prm, e, it + 3 * W, cc, ng, row_bytes);
        finish_iter<BITS, CPL, FUSED>(bufB, prm, p, it + W, xr, xs, valid, qc);
      }
      if (it + 2 * W < it1) {
        if (it + 4 * W < it1) load_rows<BITS, CPL, FUSED>(bufB, prm, e, it + 4 * W, cc, ng, row_bytes);
        finish_iter<BITS, CPL, FUSED>(bufC, prm, p, it + 2 * W, xr, xs, valid, qc);
      }
    }
    return;
  }
  for (int it = gw; it < it1; it += 2 * W) {
    if (it + W < it1) load_rows<BITS, CPL, FUSED>(bufB, prm, e, it + W, cc, ng, row_bytes);
    finish_iter<BITS, CPL, FUSED>(bufA, prm, p, it, xr, xs, valid, qc);
    if (it + W < it1) {
      if (it + 2 * W < it1) load_rows<BITS, CPL, FUSED>(bufA, prm, e, it + 2 * W, cc, ng, row_bytes);
      finish_iter<BITS, CPL, FUSED>(bufB, prm, p, it + W, xr, xs, valid, qc);
    }
  }
}

template <int BITS, bool FUSED>
static hipError_t launch_up_cpl(int cpl, const GemvUpParams& prm, dim3 grid, hipStream_t st) {
  switch (cpl) {
    case 1: gemv_up_kernel<BITS, 1, FUSED><<<grid, 256, 0, st>>>(prm); break;
    case 2: gemv_up_kernel<BITS, 2, FUSED><<<grid, 256, 0, st>>>(prm); break;
    case 3: gemv_up_kernel<BITS, 3, FUSED><<<grid, 256, 0, st>>>(prm); break;
    case 4: gemv_up_kernel<BITS, 4, FUSED><<<grid, 256, 0, st>>>(prm); break;
    case 8: gemv_up_kernel<BITS, 8, FUSED><<<grid, 256, 0, st>>>(prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_up(const void* x, int act, const GemvRoute& route, int k_static, int kcap, int T, int H,
                          int N, int bits, bool fused, WView w0, WView w1, uint16_t* h, float* out32, int num_cu,
                          hipStream_t st) {
  GemvUpParams prm;
  prm.x = (const uint16_t*)x;
  prm.act = act;
  prm.rt = RouteSrc{route.logits, route.E, route.idx, route.wts, route.k_used, route.entropy};
  prm.k_static = k_static;
  prm.kcap = kcap;
  prm.H = H;
  prm.N = N;
  prm.w0 = w0;
  prm.w1 = w1;
  prm.h = h;
  prm.out32 = out32;
  int cpl = gemv_lanes_chunks(H, bits);
  if (cpl > 4 && cpl <= 8) cpl = 8;
  const int rows = cpl <= 2 ? 4 : 2;
  prm.iters = fused ? N / (rows / 2) : N / rows;
  // about `waves_per_cu` resident waves per CU, shared by the pairs
  const int64_t want = (int64_t)(num_cu > 0 ? num_cu : 256) * tuning(TUNE_UP_WAVES_PER_CU);
  int64_t per_pair = want / ((int64_t)T * kcap);
  if (per_pair < 4) per_pair = 4;
  if (per_pair > prm.iters) per_pair = prm.iters;
  prm.iters_per_wave = (int)((prm.iters + per_pair - 1) / per_pair);
  dim3 grid((unsigned)((per_pair + 3) / 4), T * kcap);
  if (bits == 4) return fused ? launch_up_cpl<4, true>(cpl, prm, grid, st) : launch_up_cpl<4, false>(cpl, prm, grid, st);
  if (bits == 8) return fused ? launch_up_cpl<8, true>(cpl, prm, grid, st) : launch_up_cpl<8, false>(cpl, prm, grid, st);
  return fused ? launch_up_cpl<16, true>(cpl, prm, grid, st) : launch_up_cpl<16, false>(cpl, prm, grid, st);
}

// ---------------------------------------------------- down + combine ------
//
// Workgroup = kcap waves, wave s handles slot s of token t: it keeps the
// slot's SwiGLU row h in registers (in unpack order, with per-chunk sums) and
// streams R rows m = blockIdx.x + j * gridDim.x of that slot's expert (so all
// workgroups sweep the down weights linearly).  The row values o_s[m] meet in
// LDS and wave 0 combines them in slot order: y = sum_s w_s * o_s.

constexpr int DOWN_MAX_ROWS = 64;

size_t gemv_down_lds_bytes(int kcap, int I, int bits) {
  (void)I;
  (void)bits;
  return (size_t)kcap * DOWN_MAX_ROWS * 4;
}

struct GemvDownParams {
  const uint16_t* h;  // fp16 [T*kcap, I], pair order
  RouteSrc rt;
  int k_static, kcap;
  int H, I;
  int rows;           // rows per workgroup
  WView wd;
  void* y;
  int act;
};

template <int BITS, int DCPL>
struct DownBuf {
  u32x4 q[DCPL];
  uint32_t s[DCPL], b[DCPL];
};

template <int BITS, int DCPL>
__device__ __forceinline__ void load_down_row(DownBuf<BITS, DCPL>& buf, const GemvDownParams& prm, int e, int m,
                                              const int* cc, int ng, int64_t row_bytes) {
  using C = Chunk<BITS>;
  const int64_t row = (int64_t)e * prm.wd.stride + m;
  const uint8_t* rq = prm.wd.q + row * row_bytes;
#pragma unroll
  for (int i = 0; i < DCPL; ++i) {
    buf.q[i] = load_stream16(rq + (size_t)cc[i] * 16);
    if constexpr (BITS != 16) {
      buf.s[i] = prm.wd.s[row * ng + cc[i] / C::PER_GROUP];
      buf.b[i] = prm.wd.b[row * ng + cc[i] / C::PER_GROUP];
    }
  }
}

// KS waves share a slot: wave ks owns lane chunks i in [ks*DC, (ks+1)*DC)
// of every row (DC chunks per lane), halving the registers a long row needs.
template <int BITS, int DC, int KS>
__global__ __launch_bounds__(1024) void gemv_down_kernel(GemvDownParams prm) {
  using C = Chunk<BITS>;
  __shared__ float part[MOE_MAX_K_DEV][KS][DOWN_MAX_ROWS];
  const int t = blockIdx.y;
  const int wv = threadIdx.x / WAVE;
  const int s = wv / KS, ks = wv % KS;
  const int lane = lane_id();
  const int ku = prm.rt.logits ? prm.k_static : *prm.rt.k_used;
  const int I = prm.I;
  const int nch = I / C::VALS;
  const int ng = I / 64;
  const int G = gridDim.x;
  const int R = prm.rows;
  const int64_t row_bytes = (int64_t)I * BITS / 8;
  const Q4Consts qc = q4_consts();

  // the token's experts and routing weights, uniform across the wave
  int si[MOE_MAX_K_DEV];
  float sw[MOE_MAX_K_DEV];
  if (prm.rt.logits) {
    route_token(prm.rt.logits + (size_t)t * prm.rt.E, prm.rt.E, ku, si, sw);
  } else {
#pragma unroll
    for (int j = 0; j < MOE_MAX_K_DEV; ++j) {
      si[j] = j < ku ? prm.rt.idx[(size_t)t * prm.kcap + j] : 0;
      sw[j] = j < ku ? prm.rt.wts[(size_t)t * prm.kcap + j] : 0.0f;
    }
  }

  if (s < ku) {
    int e = 0;
    for_slot(s, [&](int j) { e = si[j]; });
    e = __builtin_amdgcn_readfirstlane(e);
    int cc[DC];
    bool valid[DC];
#pragma unroll
    for (int i = 0; i < DC; ++i) {
      const int c = lane + 64 * (ks * DC + i);
      valid[i] = c < nch;
      cc[i] = valid[i] ? c : nch - 1;
    }
    DownBuf<BITS, DC> bufA, bufB;
    const int m0 = blockIdx.x;
    load_down_row<BITS, DC>(bufA, prm, e, m0, cc, ng, row_bytes);

    // this slot's SwiGLU row (the wave's chunks), as fp16 pairs in unpack order
    uint32_t hr[DC][C::PAIRS];
    XSums hs[DC];
    const uint16_t* hrow = prm.h + ((size_t)t * prm.kcap + s) * I;
#pragma unroll
    for (int i = 0; i < DC; ++i) {
#pragma unroll
      for (int j = 0; j < C::PIECES; ++j) {
        u32x4 v = load16(hrow + (size_t)cc[i] * C::VALS + 8 * j);
        if constexpr (BITS == 4) v = perm8_nibble_order(v);
        hr[i][4 * j + 0] = v.x;
        hr[i][4 * j + 1] = v.y;
        hr[i][4 * j + 2] = v.z;
        hr[i][4 * j + 3] = v.w;
      }
      hs[i] = chunk_xsums<BITS>(hr[i]);
    }

    auto row_value = [&](const DownBuf<BITS, DC>& buf) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < DC; ++i) {
        const float v = chunk_value<BITS>(buf.q[i], hr[i], hs[i], buf.s[i], buf.b[i], qc);
        acc += valid[i] ? v : 0.0f;
      }
      return wave_sum(acc);
    };

    for (int j = 0; j < R; j += 2) {
      const int ma = m0 + j * G, mb = m0 + (j + 1) * G;
      const bool hb = j + 1 < R && mb < prm.H;
      if (hb) load_down_row<BITS, DC>(bufB, prm, e, mb, cc, ng, row_bytes);
      if (ma < prm.H) {
        const float o = row_value(bufA);
        if (lane == 0) part[s][ks][j] = o;
      }
      if (hb) {
        const int mc = m0 + (j + 2) * G;
        if (j + 2 < R && mc < prm.H) load_down_row<BITS, DC>(bufA, prm, e, mc, cc, ng, row_bytes);
        const float o = row_value(bufB);
        if (lane == 0) part[s][ks][j + 1] = o;
      }
    }
  }
  __syncthreads();
  if (wv == 0 && lane < R) {
    const int m = blockIdx.x + lane * G;
    if (m < prm.H) {
      float y = 0.0f;
      for (int q = 0; q < ku; ++q) {
        float w = 0.0f;
        for_slot(q, [&](int j) { w = sw[j]; });
        float o = part[q][0][lane];
#pragma unroll
        for (int k2 = 1; k2 < KS; ++k2) o = o + part[q][k2][lane];
        const float c = w * o;
        y = y + c;
      }
      ((uint16_t*)prm.y)[(size_t)t * prm.H + m] = f32_to_act_bits(y, prm.act);
    }
  }
}

hipError_t gemv_down_set_max_lds(int bytes) {
  (void)bytes;
  return hipSuccess;
}

int gemv_down_max_chunks_per_lane() { return 6; }

hipError_t launch_gemv_down(const uint16_t* h, const GemvRoute& route, int k_static, int kcap, int T, int H, int I,
                            int bits, WView wd, void* y, int act, int num_cu, hipStream_t st) {
  GemvDownParams prm;
  prm.h = h;
  prm.rt = RouteSrc{route.logits, route.E, route.idx, route.wts, route.k_used, route.entropy};
  prm.k_static = k_static;
  prm.kcap = kcap;
  prm.H = H;
  prm.I = I;
  prm.wd = wd;
  prm.y = y;
  prm.act = act;
  const int dcpl = gemv_lanes_chunks(I, bits);
  const int ks = dcpl >= 4 ? 2 : 1;            // waves per slot
  const int dc = (dcpl + ks - 1) / ks;          // chunks per lane per wave
  // rows per workgroup so that about `waves_per_cu` waves per CU are resident
  const int64_t want = (int64_t)(num_cu > 0 ? num_cu : 256) * tuning(TUNE_DOWN_WAVES_PER_CU);
  int64_t groups = want / ((int64_t)T * kcap * ks);
  if (groups < 1) groups = 1;
  int rows = (int)((H + groups - 1) / groups);
  if (rows < 2) rows = 2;
  if (rows > DOWN_MAX_ROWS) rows = DOWN_MAX_ROWS;
  prm.rows = rows;
  const int G = (H + rows - 1) / rows;
  dim3 grid(G, T);
  dim3 block(64 * kcap * ks);
#define X(B, D, K) \
  if (bits == B && dc == D && ks == K) gemv_down_kernel<B, D, K><<<grid, block, 0, st>>>(prm); else
#define CASES(B) X(B, 1, 1) X(B, 2, 1) X(B, 3, 1) X(B, 2, 2) X(B, 3, 2)
  CASES(4) CASES(8) CASES(16) return hipErrorInvalidValue;
#undef CASES
#undef X
  return hipGetLastError();
}

}  // namespace moe

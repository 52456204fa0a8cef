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
// product: for a 16-byte chunk of codes q with scale s and bias b,
//     sum_k x_k (s q_k + b) = s * (sum_k x_k (1024 + q_k) - 1024 * X) + b * X,
// X = sum_k x_k.  The codes become the fp16 numbers 1024 + q with one
// AND-OR per pair (exponent bits 0x6400), and v_dot2_f32_f16 multiplies two
// code/activation pairs with fp32 accumulation, so the inner loop costs
// about 1.4 VALU operations per 4-bit weight.
//
// Lane l of a wave owns the 16-byte chunks c = l + 64*i of every row, so one
// load instruction covers 1 KB of contiguous weights.  Each row's 64 lane
// partials are summed with a butterfly; the same row code serves the fused
// (gate+up+SwiGLU) and the single-projection kernels, so both round the same.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

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

// dot of one 16-byte weight chunk with its activation pairs (fp32 accumulate)
template <int BITS>
__device__ __forceinline__ float chunk_dot(u32x4 w, const uint32_t* xp) {
  float acc = 0.0f;
  uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p[4];
      q4_word_to_biased_pairs(wv[j], p);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = dot2(p[i], xp[4 * j + i], acc);
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p[2];
      q8_word_to_biased_pairs(wv[j], p);
      acc = dot2(p[0], xp[2 * j], acc);
      acc = dot2(p[1], xp[2 * j + 1], acc);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = dot2(wv[j], xp[j], acc);
  }
  return acc;
}

// chunk dot -> contribution of the chunk to the row (affine terms applied)
template <int BITS>
__device__ __forceinline__ float chunk_value(float d, float xsum, uint32_t s_bits, uint32_t b_bits) {
  if constexpr (BITS == 16) {
    return d;
  } else {
    float s = f16_bits_to_f32(s_bits), b = f16_bits_to_f32(b_bits);
    float c = 1024.0f * xsum;
    float a = s * (d - c);
    float bb = b * xsum;
    return a + bb;
  }
}

// ------------------------------------------------------------- gate + up --

struct GemvUpParams {
  const uint16_t* x;
  int act;
  const int32_t* idx;
  const int32_t* k_used;
  int k_static, kcap;
  int H, N;  // N: output columns (fused: inter) or rows (single)
  WView w0, w1;
  uint16_t* h;
  float* out32;
  int iters;            // row-iterations per pair
  int iters_per_wave;
};

constexpr int GEMV_ROWS = 4;  // rows per iteration

template <int BITS, int CPL, bool FUSED>
__global__ __launch_bounds__(256) void gemv_up_kernel(GemvUpParams prm) {
  using C = Chunk<BITS>;
  const int lane = lane_id();
  const int p = blockIdx.y;
  const int t = p / prm.kcap, slot = p % prm.kcap;
  const int ku = prm.k_used ? *prm.k_used : prm.k_static;
  if (slot >= ku) return;
  const int e = prm.idx[p];
  const int gw = blockIdx.x * 4 + threadIdx.x / WAVE;
  const int it0 = gw * prm.iters_per_wave;
  if (it0 >= prm.iters) return;
  const int it1 = min(it0 + prm.iters_per_wave, prm.iters);
  const int H = prm.H;
  const int nch = H / C::VALS;
  const int ng = H / 64;
  const int64_t row_bytes = (int64_t)H * BITS / 8;

  // activations of this lane's chunks, as fp16 pairs in the unpack order
  uint32_t xr[CPL][C::PAIRS];
  float xs[CPL];
  const uint16_t* xrow = prm.x + (size_t)t * H;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    xs[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < C::PIECES; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < nch) v = act8_to_f16(load16(xrow + (size_t)c * C::VALS + 8 * j), prm.act);
      if constexpr (BITS == 4) v = perm8_nibble_order(v);
      xr[i][4 * j + 0] = v.x;
      xr[i][4 * j + 1] = v.y;
      xr[i][4 * j + 2] = v.z;
      xr[i][4 * j + 3] = v.w;
    }
    if constexpr (BITS != 16) {
#pragma unroll
      for (int j = 0; j < C::PAIRS; ++j) {
        f16x2 hp = __builtin_bit_cast(f16x2, xr[i][j]);
        xs[i] += (float)hp.x;
        xs[i] += (float)hp.y;
      }
    }
  }

  for (int it = it0; it < it1; ++it) {
    // the 4 rows of this iteration
    const uint8_t* rq[GEMV_ROWS];
    const uint16_t* rs[GEMV_ROWS];
    const uint16_t* rb[GEMV_ROWS];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r) {
      const WView& wv = (FUSED && r >= 2) ? prm.w1 : prm.w0;
      const int n = FUSED ? 2 * it + (r & 1) : GEMV_ROWS * it + r;
      const int64_t row = (int64_t)e * wv.stride + n;
      rq[r] = wv.q + row * row_bytes;
      rs[r] = BITS == 16 ? nullptr : wv.s + row * ng;
      rb[r] = BITS == 16 ? nullptr : wv.b + row * ng;
    }
    u32x4 wq[GEMV_ROWS][CPL];
    uint32_t sb[GEMV_ROWS][CPL], bb[GEMV_ROWS][CPL];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
          wq[r][i] = load_stream16(rq[r] + (size_t)c * 16);
          if constexpr (BITS != 16) {
            sb[r][i] = rs[r][c / C::PER_GROUP];
            bb[r][i] = rb[r][c / C::PER_GROUP];
          }
        }
      }
    float part[GEMV_ROWS];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
          float d = chunk_dot<BITS>(wq[r][i], xr[i]);
          float v;
          if constexpr (BITS == 16) v = chunk_value<BITS>(d, 0.0f, 0u, 0u);
          else v = chunk_value<BITS>(d, xs[i], sb[r][i], bb[r][i]);
          acc += v;
        }
      }
      part[r] = wave_sum(acc);
    }
    if (lane == 0) {
      if constexpr (FUSED) {
        const int j = 2 * it;
        uint32_t h0 = f32_to_f16_bits(swiglu(part[0], part[2]));
        uint32_t h1 = f32_to_f16_bits(swiglu(part[1], part[3]));
        *(uint32_t*)(prm.h + (size_t)p * prm.N + j) = h0 | (h1 << 16);
      } else {
        f32x4 o = {part[0], part[1], part[2], part[3]};
        *(f32x4*)(prm.out32 + (size_t)p * prm.N + GEMV_ROWS * it) = o;
      }
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

hipError_t launch_gemv_up(const void* x, int act, const int32_t* idx, const int32_t* k_used_dev, int k_static,
                          int kcap, int T, int H, int N, int bits, bool fused, WView w0, WView w1, uint16_t* h,
                          float* out32, hipStream_t st) {
  GemvUpParams prm;
  prm.x = (const uint16_t*)x;
  prm.act = act;
  prm.idx = idx;
  prm.k_used = k_used_dev;
  prm.k_static = k_static;
  prm.kcap = kcap;
  prm.H = H;
  prm.N = N;
  prm.w0 = w0;
  prm.w1 = w1;
  prm.h = h;
  prm.out32 = out32;
  prm.iters = fused ? N / 2 : N / GEMV_ROWS;
  prm.iters_per_wave = 4;
  int cpl = gemv_lanes_chunks(H, bits);
  if (cpl > 4 && cpl <= 8) cpl = 8;
  const int waves = (prm.iters + prm.iters_per_wave - 1) / prm.iters_per_wave;
  dim3 grid((waves + 3) / 4, T * kcap);
  if (bits == 4) return fused ? launch_up_cpl<4, true>(cpl, prm, grid, st) : launch_up_cpl<4, false>(cpl, prm, grid, st);
  if (bits == 8) return fused ? launch_up_cpl<8, true>(cpl, prm, grid, st) : launch_up_cpl<8, false>(cpl, prm, grid, st);
  return fused ? launch_up_cpl<16, true>(cpl, prm, grid, st) : launch_up_cpl<16, false>(cpl, prm, grid, st);
}

// ---------------------------------------------------- down + combine ------

constexpr int DOWN_WAVES = 16;

size_t gemv_down_lds_bytes(int kcap, int I, int bits) {
  int vals = bits == 4 ? 32 : (bits == 8 ? 16 : 8);
  size_t nch = (size_t)I / vals;
  return (size_t)kcap * I * 2 + (bits == 16 ? 0 : (size_t)kcap * nch * 4);
}

struct GemvDownParams {
  const uint16_t* h;  // fp16 [T*kcap, I], pair order
  const int32_t* idx;
  const float* wts;
  const int32_t* k_used;
  int k_static, kcap;
  int H, I;
  WView wd;
  void* y;
  int act;
};

// Workgroup = 16 waves = 16 output rows of one token.  The token's SwiGLU
// rows are staged in LDS once (piece-major so lanes read consecutive 16-byte
// words), with per-chunk sums for the affine terms.
template <int BITS>
__global__ __launch_bounds__(1024) void gemv_down_kernel(GemvDownParams prm) {
  using C = Chunk<BITS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int t = blockIdx.y;
  const int ku = prm.k_used ? *prm.k_used : prm.k_static;
  const int I = prm.I;
  const int nch = I / C::VALS;
  const int ng = I / 64;
  u32x4* hl = (u32x4*)lds;                                   // [kcap][PIECES][nch]
  float* hsum = (float*)(lds + (size_t)prm.kcap * I * 2);   // [kcap][nch]

  for (int s = 0; s < ku; ++s) {
    const uint16_t* hrow = prm.h + ((size_t)t * prm.kcap + s) * I;
    for (int q = threadIdx.x; q < nch * C::PIECES; q += blockDim.x) {
      const int c = q / C::PIECES, j = q % C::PIECES;
      u32x4 v = load16(hrow + (size_t)q * 8);
      if constexpr (BITS == 4) v = perm8_nibble_order(v);
      hl[((size_t)s * C::PIECES + j) * nch + c] = v;
    }
  }
  __syncthreads();
  if constexpr (BITS != 16) {
    for (int q = threadIdx.x; q < ku * nch; q += blockDim.x) {
      const int s = q / nch, c = q % nch;
      float a = 0.0f;
      for (int j = 0; j < C::PIECES; ++j) {
        u32x4 v = hl[((size_t)s * C::PIECES + j) * nch + c];
        uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        for (int i = 0; i < 4; ++i) {
          f16x2 hp = __builtin_bit_cast(f16x2, w4[i]);
          a += (float)hp.x;
          a += (float)hp.y;
        }
      }
      hsum[q] = a;
    }
    __syncthreads();
  }

  const int lane = lane_id();
  const int m = blockIdx.x * DOWN_WAVES + threadIdx.x / WAVE;
  if (m >= prm.H) return;
  const int64_t row_bytes = (int64_t)I * BITS / 8;
  float y = 0.0f;
  for (int s = 0; s < ku; ++s) {
    const int e = prm.idx[(size_t)t * prm.kcap + s];
    const int64_t row = (int64_t)e * prm.wd.stride + m;
    const uint8_t* rq = prm.wd.q + row * row_bytes;
    const uint16_t* rs = BITS == 16 ? nullptr : prm.wd.s + row * ng;
    const uint16_t* rb = BITS == 16 ? nullptr : prm.wd.b + row * ng;
    float acc = 0.0f;
    for (int c = lane; c < nch; c += 64) {
      u32x4 w = load_stream16(rq + (size_t)c * 16);
      uint32_t xp[C::PAIRS];
#pragma unroll
      for (int j = 0; j < C::PIECES; ++j) {
        u32x4 v = hl[((size_t)s * C::PIECES + j) * nch + c];
        xp[4 * j + 0] = v.x;
        xp[4 * j + 1] = v.y;
        xp[4 * j + 2] = v.z;
        xp[4 * j + 3] = v.w;
      }
      float d = chunk_dot<BITS>(w, xp);
      float v;
      if constexpr (BITS == 16) v = chunk_value<BITS>(d, 0.0f, 0u, 0u);
      else v = chunk_value<BITS>(d, hsum[s * nch + c], rs[c / C::PER_GROUP], rb[c / C::PER_GROUP]);
      acc += v;
    }
    const float o = wave_sum(acc);
    const float ws = prm.wts[(size_t)t * prm.kcap + s];
    const float contrib = ws * o;
    y = y + contrib;
  }
  if (lane == 0) ((uint16_t*)prm.y)[(size_t)t * prm.H + m] = f32_to_act_bits(y, prm.act);
}

hipError_t gemv_down_set_max_lds(int bytes) {
  hipError_t e = hipFuncSetAttribute((const void*)gemv_down_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)gemv_down_kernel<8>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)gemv_down_kernel<16>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return e;
}

hipError_t launch_gemv_down(const uint16_t* h, const int32_t* idx, const float* wts, const int32_t* k_used_dev,
                            int k_static, int kcap, int T, int H, int I, int bits, WView wd, void* y, int act,
                            hipStream_t st) {
  GemvDownParams prm;
  prm.h = h;
  prm.idx = idx;
  prm.wts = wts;
  prm.k_used = k_used_dev;
  prm.k_static = k_static;
  prm.kcap = kcap;
  prm.H = H;
  prm.I = I;
  prm.wd = wd;
  prm.y = y;
  prm.act = act;
  const size_t lds = gemv_down_lds_bytes(kcap, I, bits);
  dim3 grid((H + DOWN_WAVES - 1) / DOWN_WAVES, T);
  if (bits == 4) gemv_down_kernel<4><<<grid, 1024, lds, st>>>(prm);
  else if (bits == 8) gemv_down_kernel<8><<<grid, 1024, lds, st>>>(prm);
  else gemv_down_kernel<16><<<grid, 1024, lds, st>>>(prm);
  return hipGetLastError();
}

}  // namespace moe

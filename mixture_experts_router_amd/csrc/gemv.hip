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
// About 1.4 VALU operations per 4-bit weight.  NVFP4 codes have no bias: a
// chunk's two 16-column blocks give two dot sums of exact fp16 E2M1 values
// (one conversion instruction per code pair), weighted by the blocks' E4M3
// scales; the tensor scale multiplies the row's sum.
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
// wave of the gate+up kernel selects its slot's expert from the logits
// (topk.hpp) instead of waiting for a separate selection launch, and block 0
// of each pair writes the selection, which the down kernel then reads.
struct RouteSrc {
  const float* logits;  // [T, E] or NULL: read idx/wts
  int E;
  int32_t* idx;         // [T, kcap]: output when logits is given, else input
  float* wts;
  int32_t* k_used;      // device scalar: output when logits is given, else input (may be NULL)
  float* entropy;
  int gs;               // experts per selection group (1: plain top-k)
};

template <typename F>
__device__ __forceinline__ void for_slot(int s, F f) {
#pragma unroll
  for (int j = 0; j < MOE_MAX_K_DEV; ++j)
    if (j == s) f(j);
}

// A lane's unit of a weight row: 16 bytes (32 4-bit, 16 8-bit or 8 fp16
// weights), 12 bytes of 6-bit codes (16 weights: three whole words) or 20
// bytes of 5-bit codes (32 weights: five whole words)
template <int BITS>
struct Chunk {
  static constexpr int VALS = BITS == 4 || BITS == 5 || BITS == NVF4 ? 32 : (BITS == 6 || BITS == 8 ? 16 : 8);
  static constexpr int BYTES = BITS == 6 ? 12 : (BITS == 5 ? 20 : 16);                          // bytes per chunk
  static constexpr int PAIRS = VALS / 2;       // fp16 pairs of activations
  static constexpr int PER_GROUP = 64 / VALS;  // chunks per 64-column group
  static constexpr int PIECES = VALS / 8;      // 16-byte activation pieces
};

int gemv_lanes_chunks(int K, int bits) {
  int vals = bits == 4 || bits == 5 || bits == NVF4 ? 32 : (bits == 6 || bits == 8 ? 16 : 8);
  return (K / vals + 63) / 64;
}

// a chunk's words in registers: four, or five for 5-bit codes
struct Raw5 {
  u32x4 a;
  uint32_t e;
};
template <int BITS>
struct RawOf {
  typedef u32x4 T;
};
template <>
struct RawOf<5> {
  typedef Raw5 T;
};

// one chunk of codes (a 6-bit chunk is 12 bytes: the fourth word is zero)
template <int BITS>
__device__ __forceinline__ typename RawOf<BITS>::T load_chunk_nt(rsrc_t r, uint32_t off) {
  if constexpr (BITS == 5) {
    return Raw5{buf_load16_nt(r, off), __builtin_amdgcn_raw_buffer_load_b32(r, (int)off + 16, 0, AUX_NT)};
  } else if constexpr (BITS == 6) {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, AUX_NT);
    return u32x4{v.x, v.y, v.z, 0u};
  } else {
    return buf_load16_nt(r, off);
  }
}

// Per-chunk activation terms: k, the amount the biased codes add to the
// chunk's dot sum (1024 Xa + 64 Xb for 4-bit codes, where the 1024+16q pairs
// are scaled by 1/16; 1024 X for 8-bit codes), and the plain sum X.
struct XSums {
  float k, x;
};

// Activation sums of one chunk held as fp16 pairs in unpack order.
template <int BITS>
__device__ __forceinline__ XSums chunk_xsums(const uint32_t* xp) {
  XSums r = {0.0f, 0.0f};
  if constexpr (BITS == 4) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int j = 0; j < Chunk<4>::PAIRS; ++j) {
      const f16x2 hp = __builtin_bit_cast(f16x2, xp[j]);
      const float s2 = (float)hp.x + (float)hp.y;
      if ((j & 1) == 0) a += s2;  // pairs (k0,k4), (k2,k6)
      else b += s2;               // pairs (k1,k5), (k3,k7)
    }
    r.k = 1024.0f * a + 64.0f * b;
    r.x = a + b;
  } else if constexpr (BITS == 5 || BITS == 6 || BITS == 8) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < Chunk<BITS>::PAIRS; ++j) {
      const f16x2 hp = __builtin_bit_cast(f16x2, xp[j]);
      a += (float)hp.x + (float)hp.y;
    }
    r.k = 1024.0f * a;
    r.x = a;
  }
  return r;
}

__device__ __forceinline__ float half_bits_f(uint32_t b) {
  return (float)__builtin_bit_cast(f16, (uint16_t)b);
}

// acc + (contribution of one 16-byte chunk of weights to its row):
//     s * (sum_k x_k q_k) + b * X,  sum_k x_k q_k = A + B/16 - k
// (A, B: dot sums over the two kinds of biased pairs).  The fp16 scale and
// bias enter the fused multiply-adds directly (v_fma_mix_f32).
template <int BITS>
__device__ __forceinline__ float chunk_acc_words(u32x4 w, const uint32_t* xp, const XSums& xs, uint32_t s_bits,
                                                 uint32_t b_bits, const Q4Consts& qc, float acc);

template <int BITS>
__device__ __forceinline__ float chunk_acc(const typename RawOf<BITS>::T& w, const uint32_t* xp, const XSums& xs,
                                           uint32_t s_bits, uint32_t b_bits, const Q4Consts& qc, float acc) {
  if constexpr (BITS == 5) {
    // 32 codes in the 160-bit little-endian value of the five words: code i
    // at bits 5i .. 5i+4; pairs of codes become biased fp16 pairs as for 8 bits
    const uint32_t wv[5] = {w.a.x, w.a.y, w.a.z, w.a.w, w.e};
    auto code = [&](int i) __attribute__((always_inline)) -> uint32_t {
      const int bit = 5 * i, wd = bit >> 5, sh = bit & 31;
      if (sh + 5 <= 32) return (wv[wd] >> sh) & 31u;
      return ((wv[wd] >> sh) | (wv[wd + 1] << (32 - sh))) & 31u;
    };
    float A = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t p = 0x64006400u | code(2 * j) | (code(2 * j + 1) << 16);
      A = dot2(p, xp[j], A);
    }
    const float dq = A - xs.k;
    return __builtin_fmaf(half_bits_f(s_bits), dq, __builtin_fmaf(half_bits_f(b_bits), xs.x, acc));
  } else {
    return chunk_acc_words<BITS>(w, xp, xs, s_bits, b_bits, qc, acc);
  }
}

template <int BITS>
__device__ __forceinline__ float chunk_acc_words(u32x4 w, const uint32_t* xp, const XSums& xs, uint32_t s_bits,
                                                 uint32_t b_bits, const Q4Consts& qc, float acc) {
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
    const float dq = __builtin_fmaf(B, 0.0625f, A) - xs.k;
    return __builtin_fmaf(half_bits_f(s_bits), dq, __builtin_fmaf(half_bits_f(b_bits), xs.x, acc));
  } else if constexpr (BITS == 8) {
    float A = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p[2];
      q8_word_to_biased_pairs(wv[j], p);
      A = dot2(p[0], xp[2 * j], A);
      A = dot2(p[1], xp[2 * j + 1], A);
    }
    const float dq = A - xs.k;
    return __builtin_fmaf(half_bits_f(s_bits), dq, __builtin_fmaf(half_bits_f(b_bits), xs.x, acc));
  } else if constexpr (BITS == 6) {
    // 16 codes in the 96-bit little-endian value w.x | w.y << 32 | w.z << 64:
    // code i at bits 6i .. 6i+5.  Each pair of codes becomes the fp16 pair
    // (1024 + q_2j, 1024 + q_2j+1) (exponent bits 0x6400), as for 8 bits.
    const uint64_t lo = (uint64_t)wv[0] | ((uint64_t)wv[1] << 32);
    auto code = [&](int i) __attribute__((always_inline)) -> uint32_t {
      const int bit = 6 * i;
      if (bit + 6 <= 64) return (uint32_t)(lo >> bit) & 63u;
      if (bit >= 64) return (wv[2] >> (bit - 64)) & 63u;
      return ((uint32_t)(lo >> bit) | (wv[2] << (64 - bit))) & 63u;
    };
    float A = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t p = 0x64006400u | code(2 * j) | (code(2 * j + 1) << 16);
      A = dot2(p, xp[j], A);
    }
    const float dq = A - xs.k;
    return __builtin_fmaf(half_bits_f(s_bits), dq, __builtin_fmaf(half_bits_f(b_bits), xs.x, acc));
  } else if constexpr (BITS == NVF4) {
    // 32 E2M1 codes in column order: words 0-1 are block 0, words 2-3 block
    // 1; s_bits holds the two blocks' E4M3 scales (block 0 in the low byte)
    float A0 = 0.0f, A1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p[4];
      e2m1_word_to_pairs(wv[j], p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (j < 2) A0 = dot2(p[i], xp[4 * j + i], A0);
        else A1 = dot2(p[i], xp[4 * j + i], A1);
      }
    }
    return __builtin_fmaf(e4m3_byte<1>(s_bits), A1, __builtin_fmaf(e4m3_byte<0>(s_bits), A0, acc));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = dot2(wv[j], xp[j], acc);
    return acc;
  }
}

// Byte offset of chunk c's scales in a row's scale bytes: the group's fp16
// scale, or (NVF4) the two E4M3 block scales of the chunk's 32 columns
template <int BITS>
__device__ __forceinline__ uint32_t chunk_scale_off(int c) {
  if constexpr (BITS == NVF4) return (uint32_t)c * 2u;
  else return (uint32_t)(c / Chunk<BITS>::PER_GROUP) * 2u;
}
// scale bytes of one row of K weights
template <int BITS>
__device__ __forceinline__ int64_t scale_row_bytes(int K) {
  return BITS == NVF4 ? K / 16 : (K / 64) * 2;
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
  float* pre;  // fused: fp32 gate and up sums [pairs, 2N] (NULL: not kept)
  int32_t* tokexp;  // bf16 activations: each token's exponent a_t (written); NULL for fp16
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
  typename RawOf<BITS>::T q[R][CPL];
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

// Loads of iteration `it`.  When `live` is false (an iteration past the
// wave's end, issued only to keep the wait counts exact) the loads go through
// empty resources: they return zeros and read no memory.
template <int BITS, int CPL, bool FUSED>
__device__ __forceinline__ void load_rows(RowBuf<BITS, CPL>& buf, const GemvUpParams& prm, int e, int it, bool live,
                                          const uint32_t* qoff, const uint32_t* goff, int ng, int64_t row_bytes) {
  constexpr int R = Rows<CPL>::N;
  const uint32_t nq = live ? (uint32_t)row_bytes : 0u;
  const int64_t srb = scale_row_bytes<BITS>(prm.H);
  const uint32_t ns = live ? (uint32_t)srb : 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const WView& wv = (FUSED && r >= R / 2) ? prm.w1 : prm.w0;
    const int64_t row = (int64_t)e * wv.stride + row_of<CPL, FUSED>(it, r);
    const rsrc_t rq = make_rsrc(wv.q + row * row_bytes, nq);
#pragma unroll
    for (int i = 0; i < CPL; ++i) buf.q[r][i] = load_chunk_nt<BITS>(rq, qoff[i]);
    if constexpr (BITS != 16) {
      const rsrc_t rs = make_rsrc((const uint8_t*)wv.s + row * srb, ns);
#pragma unroll
      for (int i = 0; i < CPL; ++i) buf.s[r][i] = buf_load_u16_nt(rs, goff[i]);
      if constexpr (BITS != NVF4) {
        const rsrc_t rb = make_rsrc((const uint8_t*)wv.b + row * srb, ns);
#pragma unroll
        for (int i = 0; i < CPL; ++i) buf.b[r][i] = buf_load_u16_nt(rb, goff[i]);
      } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) buf.b[r][i] = 0u;
      }
    }
  }
}

// Row sums of one iteration and their store.  After reduce_rows, lane r holds
// row r: fused R = 4 rows are (gate j, gate j+1, up j, up j+1), so lanes 0
// and 1 form h[j] and h[j+1]; fused R = 2 rows are (gate j, up j).
template <int BITS, int CPL, bool FUSED>
__device__ __forceinline__ void finish_iter(const RowBuf<BITS, CPL>& buf, const GemvUpParams& prm, int p, int it,
                                            bool store, const uint32_t (*xr)[Chunk<BITS>::PAIRS], const XSums* xs,
                                            const Q4Consts& qc, int a) {
  constexpr int R = Rows<CPL>::N;
  float part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc = chunk_acc<BITS>(buf.q[r][i], xr[i], xs[i], buf.s[r][i], buf.b[r][i], qc, acc);
    part[r] = acc;
  }
  // the sums of the scaled activations x * 2^-a, scaled back (exact)
  float v = ldexp_f(reduce_rows<R>(part), a);
  const int lane = lane_id();
  // NVFP4: lane r holds row r, whose tensor's scale multiplies its sum
  if constexpr (BITS == NVF4) v *= (FUSED && lane >= R / 2) ? prm.w1.ts : prm.w0.ts;
  if constexpr (FUSED) {
    // the up value of lane 0 (and 1) sits in lane R/2 (and R/2 + 1)
    const float u = R == 4 ? dpp_f<DPP_QUAD_2323>(v) : dpp_f<DPP_QUAD_1111>(v);
    const float hv = ldexp_f(swiglu(v, u), -2 * a);  // staged at 2^-2a
    if (store && lane < R / 2) prm.h[(size_t)p * prm.N + (R / 2) * it + lane] = f32_to_f16_bits(hv);
    if (prm.pre && store && lane < R) {
      // lane r holds row r: gate rows first, then the matching up rows
      const int col = lane < R / 2 ? (R / 2) * it + lane : prm.N + (R / 2) * it + (lane - R / 2);
      prm.pre[(size_t)p * 2 * prm.N + col] = v;
    }
  } else {
    if (store && lane < R) prm.out32[(size_t)p * prm.N + R * it + lane] = v;
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
  const int gw = blockIdx.x * 4 + wave_id();
  const int W = gridDim.x * 4;
  if (gw >= prm.iters) return;
  int e;
  if (prm.rt.logits) {
    float wsel = 0.0f;
    route_slot(prm.rt.logits + (size_t)t * prm.rt.E, prm.rt.E, ku, slot, e, wsel, prm.rt.gs);
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
  const int64_t row_bytes = (int64_t)H * code_bits(BITS) / 8;
  const Q4Consts qc = q4_consts();

  // lane chunks c = lane + 64 i; a lane past the end of the row re-reads the
  // last chunk against zero activations, which adds exactly 0
  int cc[CPL];
  bool valid[CPL];
  uint32_t qoff[CPL], goff[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    valid[i] = c < nch;
    cc[i] = valid[i] ? c : nch - 1;
    qoff[i] = (uint32_t)cc[i] * (uint32_t)C::BYTES;
    goff[i] = chunk_scale_off<BITS>(cc[i]);
  }

  // The wave's iterations are it(k) = gw + k*W, k < n.  Loads are issued
  // unconditionally (past the end through empty resources, results not
  // stored): with loads on every path the wait counts stay exact, so a
  // buffer's loads remain in flight while an older one is reduced.
  const int n = (prm.iters - gw + W - 1) / W;
  auto it_of = [&](int k) { return gw + (k < n ? k : n - 1) * W; };
  // short rows of 8-bit or fp16 weights: two iterations ahead, else one.
  // With one ahead the 4- and 5-bit forms fit three waves per SIMD, not two,
  // which streams faster than the deeper ring at two
  constexpr bool DEEP = CPL <= 2 && BITS != 4 && BITS != 5 && BITS != NVF4;

  // activation loads first: vmcnt retires in issue order, so waiting for
  // them later does not wait for the weight loads issued after them
  u32x4 xraw[CPL][C::PIECES];
  const uint16_t* xrow = prm.x + (size_t)t * H;
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int j = 0; j < C::PIECES; ++j) {
      const u32x4 v = load16(xrow + (size_t)cc[i] * C::VALS + 8 * j);
      xraw[i][j] = valid[i] ? v : u32x4{0u, 0u, 0u, 0u};
    }

  RowBuf<BITS, CPL> bufA, bufB, bufC;
  load_rows<BITS, CPL, FUSED>(bufA, prm, e, it_of(0), 0 < n, qoff, goff, ng, row_bytes);
  if constexpr (DEEP) load_rows<BITS, CPL, FUSED>(bufB, prm, e, it_of(1), 1 < n, qoff, goff, ng, row_bytes);

  // the token's exponent (bf16 activations; 0 for fp16), the same in every
  // wave from the same row
  int a = 0;
  if (prm.act == ACT_BF16) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int j = 0; j < C::PIECES; ++j) m = max(m, bf16x8_absmax_bits(xraw[i][j]));
    a = __builtin_amdgcn_readfirstlane(bf16_token_exp(wave_max_u32(m)));
    if (prm.tokexp && slot == 0 && blockIdx.x == 0 && threadIdx.x == 0) prm.tokexp[t] = a;
  }

  // activations of this lane's chunks, as fp16 pairs in the unpack order
  uint32_t xr[CPL][C::PAIRS];
  XSums xs[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
#pragma unroll
    for (int j = 0; j < C::PIECES; ++j) {
      u32x4 v = act8_to_f16_scaled(xraw[i][j], prm.act, a);
      if constexpr (BITS == 4) v = perm8_nibble_order(v);
      xr[i][4 * j + 0] = v.x;
      xr[i][4 * j + 1] = v.y;
      xr[i][4 * j + 2] = v.z;
      xr[i][4 * j + 3] = v.w;
    }
    xs[i] = chunk_xsums<BITS>(xr[i]);
  }

  if constexpr (DEEP) {
    for (int k = 0; k < n; k += 3) {
      load_rows<BITS, CPL, FUSED>(bufC, prm, e, it_of(k + 2), k + 2 < n, qoff, goff, ng, row_bytes);
      finish_iter<BITS, CPL, FUSED>(bufA, prm, p, it_of(k), k < n, xr, xs, qc, a);
      load_rows<BITS, CPL, FUSED>(bufA, prm, e, it_of(k + 3), k + 3 < n, qoff, goff, ng, row_bytes);
      finish_iter<BITS, CPL, FUSED>(bufB, prm, p, it_of(k + 1), k + 1 < n, xr, xs, qc, a);
      load_rows<BITS, CPL, FUSED>(bufB, prm, e, it_of(k + 4), k + 4 < n, qoff, goff, ng, row_bytes);
      finish_iter<BITS, CPL, FUSED>(bufC, prm, p, it_of(k + 2), k + 2 < n, xr, xs, qc, a);
    }
  } else {
    for (int k = 0; k < n; k += 2) {
      load_rows<BITS, CPL, FUSED>(bufB, prm, e, it_of(k + 1), k + 1 < n, qoff, goff, ng, row_bytes);
      finish_iter<BITS, CPL, FUSED>(bufA, prm, p, it_of(k), k < n, xr, xs, qc, a);
      load_rows<BITS, CPL, FUSED>(bufA, prm, e, it_of(k + 2), k + 2 < n, qoff, goff, ng, row_bytes);
      finish_iter<BITS, CPL, FUSED>(bufB, prm, p, it_of(k + 1), k + 1 < n, xr, xs, qc, a);
    }
  }
}

template <int BITS, bool FUSED>
static hipError_t launch_up_cpl(int cpl, const GemvUpParams& prm, dim3 grid, hipStream_t st) {
  switch (cpl) {
    case 1: launch_kernel(gemv_up_kernel<BITS, 1, FUSED>, grid, 256, 0, st, prm); break;
    case 2: launch_kernel(gemv_up_kernel<BITS, 2, FUSED>, grid, 256, 0, st, prm); break;
    case 3: launch_kernel(gemv_up_kernel<BITS, 3, FUSED>, grid, 256, 0, st, prm); break;
    case 4: launch_kernel(gemv_up_kernel<BITS, 4, FUSED>, grid, 256, 0, st, prm); break;
    case 8: launch_kernel(gemv_up_kernel<BITS, 8, FUSED>, grid, 256, 0, st, prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_up(const void* x, int act, const GemvRoute& route, int k_static, int kcap, int T, int H,
                          int N, int bits, bool fused, WView w0, WView w1, uint16_t* h, float* out32, int num_cu,
                          hipStream_t st, float* pre, int32_t* tokexp) {
  GemvUpParams prm;
  prm.pre = fused ? pre : nullptr;
  prm.tokexp = tokexp;
  prm.x = (const uint16_t*)x;
  prm.act = act;
  prm.rt = RouteSrc{route.logits, route.E, route.idx, route.wts, route.k_used, route.entropy, route.gs};
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
  // (1.5x for 4- and 5-bit codes at up to three chunks per lane, whose
  // kernels fit three or more waves per SIMD rather than two)
  const int upw = (bits == 4 || bits == 5 || bits == NVF4) && cpl <= 3 ? tuning(TUNE_UP_WAVES_PER_CU) * 3 / 2
                                                                        : tuning(TUNE_UP_WAVES_PER_CU);
  const int64_t want = (int64_t)(num_cu > 0 ? num_cu : 256) * upw;
  int64_t per_pair = want / ((int64_t)T * kcap);
  if (per_pair < 4) per_pair = 4;
  if (per_pair > prm.iters) per_pair = prm.iters;
  // as many waves as give every wave the same number of iterations (at most
  // the target): with a few waves one iteration longer than the rest, the
  // last iteration period streams with a fraction of the waves
  if (tuning(TUNE_UP_BALANCE) != 2) {
    const int64_t ipw = (prm.iters + per_pair - 1) / per_pair;
    per_pair = (prm.iters + ipw - 1) / ipw;
  }
  prm.iters_per_wave = (int)((prm.iters + per_pair - 1) / per_pair);
  dim3 grid((unsigned)((per_pair + 3) / 4), T * kcap);
  if (bits == 4) return fused ? launch_up_cpl<4, true>(cpl, prm, grid, st) : launch_up_cpl<4, false>(cpl, prm, grid, st);
  if (bits == 8) return fused ? launch_up_cpl<8, true>(cpl, prm, grid, st) : launch_up_cpl<8, false>(cpl, prm, grid, st);
  if (bits == 6) return fused ? launch_up_cpl<6, true>(cpl, prm, grid, st) : launch_up_cpl<6, false>(cpl, prm, grid, st);
  if (bits == 5) return fused ? launch_up_cpl<5, true>(cpl, prm, grid, st) : launch_up_cpl<5, false>(cpl, prm, grid, st);
  if (bits == NVF4)
    return fused ? launch_up_cpl<NVF4, true>(cpl, prm, grid, st) : launch_up_cpl<NVF4, false>(cpl, prm, grid, st);
  return fused ? launch_up_cpl<16, true>(cpl, prm, grid, st) : launch_up_cpl<16, false>(cpl, prm, grid, st);
}

// ---------------------------------------------------- down + combine ------
//
// Workgroup = kcap waves, wave s handles slot s of token t: it keeps the
// slot's SwiGLU row h in registers (in unpack order, with per-chunk sums) and
// streams R rows m = m0 + j * gridDim.x of that slot's expert, m0 its base row
// (so all workgroups sweep the down weights linearly).  The row values o_s[m] meet in
// LDS and wave 0 combines them in slot order: y = sum_s w_s * o_s.

constexpr int DOWN_MAX_ROWS = 64;

// Base row of workgroup b of G.  Workgroup b runs on XCD b % 8, and each XCD
// has its own L2: when 8 divides G, the workgroups of one XCD take
// consecutive base rows, so the scale/bias bytes two neighbouring rows share
// in a 128-byte line are fetched by one XCD, not two (a bijection of [0, G)).
__device__ __forceinline__ int down_row_base(int b, int G) {
  return (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
}

struct GemvDownParams {
  const uint16_t* h;  // fp16 [T*kcap, I], pair order, at 2^-2a_t
  const int32_t* tokexp;  // each token's exponent a_t (NULL: 0)
  RouteSrc rt;
  int k_static, kcap;
  int H, I;
  int rows;           // rows per workgroup
  WView wd;
  void* y;
  int act;
  int cap;            // expert capacity (0: none)
};

template <int BITS, int DCPL>
struct DownBuf {
  typename RawOf<BITS>::T q[DCPL];
  uint32_t s[DCPL], b[DCPL];
};

// Row m of expert e; a row past the workgroup's end (`live` false) loads
// through empty resources (zeros, no memory access).
template <int BITS, int DCPL>
__device__ __forceinline__ void load_down_row(DownBuf<BITS, DCPL>& buf, const GemvDownParams& prm, int e, int m,
                                              bool live, const uint32_t* qoff, const uint32_t* goff, int ng,
                                              int64_t row_bytes) {
  const int64_t row = (int64_t)e * prm.wd.stride + m;
  const rsrc_t rq = make_rsrc(prm.wd.q + row * row_bytes, live ? (uint32_t)row_bytes : 0u);
#pragma unroll
  for (int i = 0; i < DCPL; ++i) buf.q[i] = load_chunk_nt<BITS>(rq, qoff[i]);
  if constexpr (BITS != 16) {
    const int64_t srb = scale_row_bytes<BITS>(prm.I);
    const uint32_t ns = live ? (uint32_t)srb : 0u;
    const rsrc_t rs = make_rsrc((const uint8_t*)prm.wd.s + row * srb, ns);
#pragma unroll
    for (int i = 0; i < DCPL; ++i) buf.s[i] = buf_load_u16_nt(rs, goff[i]);
    if constexpr (BITS != NVF4) {
      const rsrc_t rb = make_rsrc((const uint8_t*)prm.wd.b + row * srb, ns);
#pragma unroll
      for (int i = 0; i < DCPL; ++i) buf.b[i] = buf_load_u16_nt(rb, goff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < DCPL; ++i) buf.b[i] = 0u;
    }
  }
}

// KS waves share a slot: wave ks owns lane chunks i in [ks*DC, (ks+1)*DC)
// of every row (DC chunks per lane), dividing the registers a long row needs
// by KS.
template <int BITS, int DC, int KS>
__global__ __launch_bounds__(KS == 4 ? 1024 : 512) void gemv_down_kernel(GemvDownParams prm) {
  using C = Chunk<BITS>;
  __shared__ float part[MOE_MAX_K_DEV][KS][DOWN_MAX_ROWS];
  const int t = blockIdx.y;
  const int wv = wave_id();
  const int s = wv / KS, ks = wv % KS;
  const int lane = lane_id();
  const int ku = prm.rt.logits ? prm.k_static : *prm.rt.k_used;
  const int I = prm.I;
  const int nch = I / C::VALS;
  const int ng = I / 64;
  const int G = gridDim.x;
  const int R = prm.rows;
  const int64_t row_bytes = (int64_t)I * code_bits(BITS) / 8;
  const Q4Consts qc = q4_consts();

  // the token's experts and routing weights, uniform across the wave
  int si[MOE_MAX_K_DEV];
  float sw[MOE_MAX_K_DEV];
  if (prm.rt.logits) {
    route_token(prm.rt.logits + (size_t)t * prm.rt.E, prm.rt.E, ku, si, sw, prm.rt.gs);
  } else {
#pragma unroll
    for (int j = 0; j < MOE_MAX_K_DEV; ++j) {
      si[j] = j < ku ? prm.rt.idx[(size_t)t * prm.kcap + j] : 0;
      sw[j] = j < ku ? prm.rt.wts[(size_t)t * prm.kcap + j] : 0.0f;
    }
  }

  // expert capacity: slot q is kept when fewer than cap earlier valid pairs
  // of the call chose its expert (page "Qwen3.5-MoE与Qwen3-MoE架构差异深度
  // 解析", section 5.2); the selection of every pair is in rt.idx
  uint32_t keep = 0xFFFFFFFFu;
  if (prm.cap > 0) {
    keep = 0u;
    for (int q = 0; q < ku; ++q) {
      int eq = 0;
      for_slot(q, [&](int j) { eq = si[j]; });
      const int pq = t * prm.kcap + q;
      int before = 0;
      for (int c0 = 0; c0 < pq; c0 += WAVE) {
        const int pp = c0 + lane;
        const bool hit = pp < pq && (pp % prm.kcap) < ku && prm.rt.idx[pp] == eq;
        before += (int)__popcll(__ballot(hit));
      }
      if (before < prm.cap) keep |= 1u << q;
    }
  }

  if (s < ku && ((keep >> s) & 1u)) {
    int e = 0;
    for_slot(s, [&](int j) { e = si[j]; });
    e = __builtin_amdgcn_readfirstlane(e);
    int cc[DC];
    bool valid[DC];
    uint32_t qoff[DC], goff[DC];
#pragma unroll
    for (int i = 0; i < DC; ++i) {
      const int c = lane + 64 * (ks * DC + i);
      valid[i] = c < nch;
      cc[i] = valid[i] ? c : nch - 1;
      qoff[i] = (uint32_t)cc[i] * (uint32_t)C::BYTES;
      goff[i] = chunk_scale_off<BITS>(cc[i]);
    }
    // rows m(j) = m0 + j*G, j < nr; loads past the end go through empty
    // resources (unconditional loads keep the wait counts exact)
    const int m0 = down_row_base(blockIdx.x, G);
    const int nr = min(R, (prm.H - m0 + G - 1) / G);
    auto m_of = [&](int j) { return m0 + (j < nr ? j : nr - 1) * G; };
    // SwiGLU-row loads first (see the gate+up kernel), then three weight rows;
    // a lane past the end of the row gets zero activations (adds exactly 0)
    u32x4 hraw[DC][C::PIECES];
    const uint16_t* hrow = prm.h + ((size_t)t * prm.kcap + s) * I;
#pragma unroll
    for (int i = 0; i < DC; ++i)
#pragma unroll
      for (int j = 0; j < C::PIECES; ++j) {
        const u32x4 v = load16(hrow + (size_t)cc[i] * C::VALS + 8 * j);
        hraw[i][j] = valid[i] ? v : u32x4{0u, 0u, 0u, 0u};
      }
    DownBuf<BITS, DC> b0, b1, b2, b3;
    load_down_row<BITS, DC>(b0, prm, e, m_of(0), 0 < nr, qoff, goff, ng, row_bytes);
    load_down_row<BITS, DC>(b1, prm, e, m_of(1), 1 < nr, qoff, goff, ng, row_bytes);
    load_down_row<BITS, DC>(b2, prm, e, m_of(2), 2 < nr, qoff, goff, ng, row_bytes);

    // this slot's SwiGLU row (the wave's chunks), as fp16 pairs in unpack order
    uint32_t hr[DC][C::PAIRS];
    XSums hs[DC];
#pragma unroll
    for (int i = 0; i < DC; ++i) {
#pragma unroll
      for (int j = 0; j < C::PIECES; ++j) {
        u32x4 v = hraw[i][j];
        if constexpr (BITS == 4) v = perm8_nibble_order(v);
        hr[i][4 * j + 0] = v.x;
        hr[i][4 * j + 1] = v.y;
        hr[i][4 * j + 2] = v.z;
        hr[i][4 * j + 3] = v.w;
      }
      hs[i] = chunk_xsums<BITS>(hr[i]);
    }

    auto row_part = [&](const DownBuf<BITS, DC>& buf) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < DC; ++i) acc = chunk_acc<BITS>(buf.q[i], hr[i], hs[i], buf.s[i], buf.b[i], qc, acc);
      return acc;
    };

    // ring of four row buffers, three rows ahead: b3 is loaded and consumed
    // in the same trip, the other three are refilled right after their use
    // and consumed in the next trip.  (A loop in which no load is consumed
    // in its own trip makes the compiler drain every load at the loop head.)
    // Scheduling barriers keep each load next to the use it follows.
    for (int j = 0; j < nr; j += 4) {
      float pr[4];
      load_down_row<BITS, DC>(b3, prm, e, m_of(j + 3), j + 3 < nr, qoff, goff, ng, row_bytes);
      __builtin_amdgcn_sched_barrier(0);
      pr[0] = row_part(b0);
      __builtin_amdgcn_sched_barrier(0);
      load_down_row<BITS, DC>(b0, prm, e, m_of(j + 4), j + 4 < nr, qoff, goff, ng, row_bytes);
      __builtin_amdgcn_sched_barrier(0);
      pr[1] = row_part(b1);
      __builtin_amdgcn_sched_barrier(0);
      load_down_row<BITS, DC>(b1, prm, e, m_of(j + 5), j + 5 < nr, qoff, goff, ng, row_bytes);
      __builtin_amdgcn_sched_barrier(0);
      pr[2] = row_part(b2);
      __builtin_amdgcn_sched_barrier(0);
      load_down_row<BITS, DC>(b2, prm, e, m_of(j + 6), j + 6 < nr, qoff, goff, ng, row_bytes);
      __builtin_amdgcn_sched_barrier(0);
      pr[3] = row_part(b3);
      const float o = reduce_rows<4>(pr);
      if (lane < 4 && j + lane < nr) part[s][ks][j + lane] = o;
    }
  }
  __syncthreads();
  if (wv == 0 && lane < R) {
    const int m = down_row_base(blockIdx.x, G) + lane * G;  // lanes past this workgroup's rows store nothing
    if (m < prm.H) {
      float y = 0.0f;
      for (int q = 0; q < ku; ++q) {
        if (!((keep >> q) & 1u)) continue;  // dropped by the capacity
        float w = 0.0f;
        for_slot(q, [&](int j) { w = sw[j]; });
        float o = part[q][0][lane];
#pragma unroll
        for (int k2 = 1; k2 < KS; ++k2) o = o + part[q][k2][lane];
        if constexpr (BITS == NVF4) o = o * prm.wd.ts;
        const float c = w * o;
        y = y + c;
      }
      if (prm.tokexp) y = ldexp_f(y, 2 * prm.tokexp[t]);  // h was staged at 2^-2a_t
      ((uint16_t*)prm.y)[(size_t)t * prm.H + m] = f32_to_act_bits(y, prm.act);
    }
  }
}

// Rows of up to 6 chunks per lane run with one wave per slot, or (at most 4
// slots per token) two waves of up to 3 chunks; rows of 7 to 12 chunks per
// lane need four waves of up to 3 chunks, so at most 4 slots per token.
bool gemv_down_fits(int I, int bits, int kcap) {
  const int dcpl = gemv_lanes_chunks(I, bits);
  return dcpl <= 6 || (dcpl <= 12 && kcap <= 4);
}

hipError_t launch_gemv_down(const uint16_t* h, const GemvRoute& route, int k_static, int kcap, int T, int H, int I,
                            int bits, WView wd, void* y, int act, int num_cu, hipStream_t st, int capacity,
                            const int32_t* tokexp) {
  if (capacity > 0 && route.logits) return hipErrorInvalidValue;
  GemvDownParams prm;
  prm.tokexp = tokexp;
  prm.cap = capacity;
  prm.h = h;
  prm.rt = RouteSrc{route.logits, route.E, route.idx, route.wts, route.k_used, route.entropy, route.gs};
  prm.k_static = k_static;
  prm.kcap = kcap;
  prm.H = H;
  prm.I = I;
  prm.wd = wd;
  prm.y = y;
  prm.act = act;
  const int dcpl = gemv_lanes_chunks(I, bits);
  if (!gemv_down_fits(I, bits, kcap)) return hipErrorInvalidValue;
  // waves per slot (blocks of at most 512 threads, 1024 with four waves per slot)
  const int ks = dcpl > 6 ? 4 : (dcpl >= 4 && kcap <= 4 ? 2 : 1);
  const int dc = (dcpl + ks - 1) / ks;  // chunks per lane per wave
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
  if (bits == B && dc == D && ks == K) launch_kernel(gemv_down_kernel<B, D, K>, grid, block, 0, st, prm); else
#define CASES(B) \
  X(B, 1, 1) X(B, 2, 1) X(B, 3, 1) X(B, 4, 1) X(B, 5, 1) X(B, 6, 1) X(B, 2, 2) X(B, 3, 2) X(B, 2, 4) X(B, 3, 4)
  CASES(4) CASES(5) CASES(6) CASES(8) CASES(16) CASES(NVF4) return hipErrorInvalidValue;
#undef CASES
#undef X
  return hipGetLastError();
}

}  // namespace moe

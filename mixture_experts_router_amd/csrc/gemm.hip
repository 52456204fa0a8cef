// Batched path: grouped GEMM over the expert-sorted pairs on the matrix cores.
//
// Rows of one M tile are consecutive sorted pairs of one expert (the sorted
// gather branch of the oMLX gate/up fusion page), so every tile multiplies one
// expert's weights.  Three instantiations:
//   GEMM_FUSED_SWIGLU  A = x rows gathered through perm, B = the fused gate_up
//                      tensor; each wave owns 32 gate and the matching 32 up
//                      columns, so the SwiGLU epilogue h = silu(g) * u is local
//                      to a lane (oMLX page, steps 3-4: one matmul over the
//                      [gate, up] concatenation, split, then activation)
//   GEMM_GATHER_F32    the same A, one projection, fp32 output (unfused path)
//   GEMM_ROWS_F16      A = h rows in sorted order, B = down, fp16 output
//
// Tile: BM = 32*MS rows x 256 columns (fused: 128 gate/up column pairs), 4
// waves side by side along N, each 32*MS x 64, K stepped one 64-column
// quantisation group at a time.  A (fp16; bf16 activations are converted,
// exact in range) is staged through LDS, double-buffered, rows padded to
// 144 bytes so 8 lanes of a 16-byte read hit 8 different bank groups.
// B never touches LDS: each lane loads the 16 bytes of codes it needs,
// dequantises them in registers (w = fma(q, s, b) in fp16, one rounding) and
// feeds v_mfma_f32_32x32x16_f16 with fp32 accumulation.  For 4-bit weights the
// k order inside each 8-column block is (0,4,1,5,2,6,3,7) on both operands,
// the order in which a 32-bit word of nibbles unpacks.
//
// Each output element's reduction runs over the same k order whichever
// instantiation, tile or column position computes it, so the fused and
// unfused paths produce identical bits.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct GemmParams {
  const uint16_t* a;
  int act;
  const int32_t* perm;
  const int32_t* counts;
  const int32_t* offsets;
  int kcap, E, K, N;
  WView w0, w1;
  void* out;
};

constexpr int A_STRIDE = 144;  // bytes per staged A row (64 fp16 + 16 bytes padding)

int gemm_block_m(int P, int E) {
  const int avg = E > 0 ? P / E : P;
  if (avg <= 32) return 32;
  if (avg <= 96) return 64;
  return 128;
}

int gemm_max_mtiles(int P, int E, int bm) { return (P + bm - 1) / bm + E; }

template <int BITS>
struct BRaw {
  static constexpr int WORDS = BITS == 4 ? 4 : (BITS == 8 ? 8 : 16);  // u32 of codes per lane per group
  u32x4 q[WORDS / 4];
  uint32_t s, b;
};

template <int BITS>
__device__ __forceinline__ void load_b(BRaw<BITS>& r, const uint8_t* qrow, const uint16_t* srow, const uint16_t* brow,
                                       int g, int hh) {
  constexpr int GROUP_BYTES = 64 * BITS / 8;
  const uint8_t* p = qrow + (size_t)g * GROUP_BYTES + hh * (GROUP_BYTES / 2);
#pragma unroll
  for (int i = 0; i < BRaw<BITS>::WORDS / 4; ++i) r.q[i] = load_stream16(p + 16 * i);
  if constexpr (BITS != 16) {
    r.s = srow[g];
    r.b = brow[g];
  }
}

// one fp16 pair of codes (biased by 1024) -> dequantised fp16 pair
__device__ __forceinline__ uint32_t deq_pair(uint32_t biased, f16x2 s2, f16x2 b2) {
  f16x2 q = __builtin_bit_cast(f16x2, biased) - (f16x2){(f16)1024.0f, (f16)1024.0f};
  f16x2 w = __builtin_elementwise_fma(q, s2, b2);
  return __builtin_bit_cast(uint32_t, w);
}

// dequantised B operands of the 4 MFMA k-steps of one group
template <int BITS>
__device__ __forceinline__ void dequant_b(const BRaw<BITS>& r, f16x8 bf[4]) {
  if constexpr (BITS == 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = __builtin_bit_cast(f16x8, r.q[j]);
  } else {
    const f16 s = __builtin_bit_cast(f16, (uint16_t)r.s), b = __builtin_bit_cast(f16, (uint16_t)r.b);
    const f16x2 s2 = {s, s}, b2 = {b, b};
    if constexpr (BITS == 4) {
      const uint32_t w[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t p[4];
        q4_word_to_biased_pairs(w[j], p);
        u32x4 o = {deq_pair(p[0], s2, b2), deq_pair(p[1], s2, b2), deq_pair(p[2], s2, b2), deq_pair(p[3], s2, b2)};
        bf[j] = __builtin_bit_cast(f16x8, o);
      }
    } else {
      const uint32_t w[8] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w, r.q[1].x, r.q[1].y, r.q[1].z, r.q[1].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t p0[2], p1[2];
        q8_word_to_biased_pairs(w[2 * j], p0);
        q8_word_to_biased_pairs(w[2 * j + 1], p1);
        u32x4 o = {deq_pair(p0[0], s2, b2), deq_pair(p0[1], s2, b2), deq_pair(p1[0], s2, b2),
                   deq_pair(p1[1], s2, b2)};
        bf[j] = __builtin_bit_cast(f16x8, o);
      }
    }
  }
}

template <int BITS, int MODE, int MS>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmParams prm) {
  constexpr int BM = 32 * MS;
  constexpr int APT = BM * 8 / 256;  // 16-byte A pieces per thread per group
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][BM * A_STRIDE];
  __shared__ int s_tile[4];

  const int lane = lane_id();
  const int wave = wave_id();
  const int tid = threadIdx.x;

  // ---- which (expert, M tile) this workgroup owns: tiles are numbered
  // expert by expert, ceil(count/BM) tiles per expert
  if (tid < WAVE) {
    const int y = blockIdx.y;
    int base_tiles = 0, fe = -1, fmt = 0;
    for (int base = 0; base < prm.E; base += WAVE) {
      const int e = base + lane;
      const int c = e < prm.E ? prm.counts[e] : 0;
      const int nt = (c + BM - 1) / BM;
      int incl = nt;
#pragma unroll
      for (int o = 1; o < WAVE; o <<= 1) {
        int v = __shfl_up(incl, o, WAVE);
        if (lane >= o) incl += v;
      }
      const int excl = incl - nt;
      if (nt > 0 && y >= base_tiles + excl && y < base_tiles + incl) {
        fe = e;
        fmt = y - base_tiles - excl;
      }
      base_tiles += __shfl(incl, WAVE - 1, WAVE);
    }
    const uint64_t m = __ballot(fe >= 0);
    if (m == 0) {
      if (lane == 0) s_tile[0] = -1;
    } else {
      const int src = __ffsll((unsigned long long)m) - 1;
      const int e = __shfl(fe, src, WAVE);
      const int mt = __shfl(fmt, src, WAVE);
      if (lane == 0) {
        const int m0 = mt * BM;
        s_tile[0] = e;
        s_tile[1] = min(BM, prm.counts[e] - m0);
        s_tile[2] = prm.offsets[e] + m0;
      }
    }
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;
  const int rows = s_tile[1];
  const int row0 = s_tile[2];
  const int K = prm.K;
  const int ng = K / 64;

  // ---- A sources: APT pieces per thread, fixed across groups
  const uint16_t* a_src[APT];
  int a_off[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int pc = tid + 256 * i;
    const int r = pc / 8, j = pc % 8;
    a_off[i] = r * A_STRIDE + j * 16;
    a_src[i] = nullptr;
    if (r < rows) {
      if constexpr (MODE == GEMM_ROWS_F16) {
        a_src[i] = prm.a + (size_t)(row0 + r) * K + 8 * j;
      } else {
        const int pair = prm.perm[row0 + r];
        a_src[i] = prm.a + (size_t)(pair / prm.kcap) * K + 8 * j;
      }
    }
  }
  const int act = MODE == GEMM_ROWS_F16 ? ACT_F16 : prm.act;

  // ---- B rows of this wave (2 subtiles of 32 columns)
  const int hh = lane / 32;
  const int col_in = lane % 32;
  int col0;
  bool valid[2];
  const uint8_t* bq[2];
  const uint16_t* bs[2];
  const uint16_t* bb[2];
  const int64_t row_bytes = (int64_t)K * BITS / 8;
  if constexpr (MODE == GEMM_FUSED_SWIGLU) {
    col0 = blockIdx.x * 128 + wave * 32;
    valid[0] = valid[1] = col0 < prm.N;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const WView& wv = ni == 0 ? prm.w0 : prm.w1;
      const int64_t row = (int64_t)e * wv.stride + (valid[ni] ? col0 + col_in : 0);
      bq[ni] = wv.q + row * row_bytes;
      bs[ni] = BITS == 16 ? nullptr : wv.s + row * ng;
      bb[ni] = BITS == 16 ? nullptr : wv.b + row * ng;
    }
  } else {
    col0 = blockIdx.x * 256 + wave * 64;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      valid[ni] = col0 + 32 * ni < prm.N;
      const int64_t row = (int64_t)e * prm.w0.stride + (valid[ni] ? col0 + 32 * ni + col_in : 0);
      bq[ni] = prm.w0.q + row * row_bytes;
      bs[ni] = BITS == 16 ? nullptr : prm.w0.s + row * ng;
      bb[ni] = BITS == 16 ? nullptr : prm.w0.b + row * ng;
    }
  }
  const bool wave_live = valid[0];

  f32x16 acc[MS][2];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  u32x4 areg[APT];
  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (a_src[i]) v = act8_to_f16(load16(a_src[i] + (size_t)g * 64), act);
      if constexpr (BITS == 4) v = perm8_nibble_order(v);
      areg[i] = v;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < APT; ++i) *(u32x4*)(&a_lds[buf][a_off[i]]) = areg[i];
  };

  BRaw<BITS> braw[2];
  if (wave_live) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      if (valid[ni]) load_b<BITS>(braw[ni], bq[ni], bs[ni], bb[ni], 0, hh);
  }
  load_a(0);
  store_a(0);
  __syncthreads();

  for (int g = 0; g < ng; ++g) {
    const int cur = g & 1;
    const bool more = g + 1 < ng;
    if (more) load_a(g + 1);
    if (wave_live) {
      f16x8 bf[2][4];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if (valid[ni]) dequant_b<BITS>(braw[ni], bf[ni]);
        else {
#pragma unroll
          for (int j = 0; j < 4; ++j) bf[ni][j] = (f16x8){};
        }
      }
      if (more) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          if (valid[ni]) load_b<BITS>(braw[ni], bq[ni], bs[ni], bb[ni], g + 1, hh);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int mi = 0; mi < MS; ++mi) {
          if (mi * 32 < rows) {
            const f16x8 af = *(const f16x8*)(&a_lds[cur][(mi * 32 + col_in) * A_STRIDE + (32 * hh + 8 * j) * 2]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[ni][j], acc[mi][ni], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_a(cur ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  // ---- epilogue.  32x32 accumulator layout: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) {
    if (mi * 32 >= rows) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mi * 32 + 8 * (r / 4) + 4 * hh + (r % 4);
      if (row >= rows) continue;
      const size_t orow = (size_t)(row0 + row) * prm.N;
      if constexpr (MODE == GEMM_FUSED_SWIGLU) {
        const float hv = swiglu(acc[mi][0][r], acc[mi][1][r]);
        ((uint16_t*)prm.out)[orow + col0 + col_in] = f32_to_f16_bits(hv);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          if (!valid[ni]) continue;
          const int col = col0 + 32 * ni + col_in;
          if constexpr (MODE == GEMM_GATHER_F32) ((float*)prm.out)[orow + col] = acc[mi][ni][r];
          else ((uint16_t*)prm.out)[orow + col] = f32_to_f16_bits(acc[mi][ni][r]);
        }
      }
    }
  }
}

template <int BITS, int MODE>
static hipError_t launch_ms(int bm, const GemmParams& prm, dim3 grid, hipStream_t st) {
  switch (bm) {
    case 32: launch_kernel(gemm_kernel<BITS, MODE, 1>, grid, 256, 0, st, prm); break;
    case 64: launch_kernel(gemm_kernel<BITS, MODE, 2>, grid, 256, 0, st, prm); break;
    case 128: launch_kernel(gemm_kernel<BITS, MODE, 4>, grid, 256, 0, st, prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_bits(GemmMode mode, int bm, const GemmParams& prm, dim3 grid, hipStream_t st) {
  switch (mode) {
    case GEMM_FUSED_SWIGLU: return launch_ms<BITS, GEMM_FUSED_SWIGLU>(bm, prm, grid, st);
    case GEMM_GATHER_F32: return launch_ms<BITS, GEMM_GATHER_F32>(bm, prm, grid, st);
    case GEMM_ROWS_F16: return launch_ms<BITS, GEMM_ROWS_F16>(bm, prm, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(GemmMode mode, const void* a, int act, const int32_t* perm, const int32_t* counts,
                       const int32_t* offsets, int kcap, int E, int K, int N, int bits, WView w0, WView w1,
                       void* out, int bm, int max_mtiles, hipStream_t st) {
  GemmParams prm;
  prm.a = (const uint16_t*)a;
  prm.act = act;
  prm.perm = perm;
  prm.counts = counts;
  prm.offsets = offsets;
  prm.kcap = kcap;
  prm.E = E;
  prm.K = K;
  prm.N = N;
  prm.w0 = w0;
  prm.w1 = w1;
  prm.out = out;
  const int ncols = mode == GEMM_FUSED_SWIGLU ? 128 : 256;
  dim3 grid((N + ncols - 1) / ncols, max_mtiles);
  if (bits == 4) return launch_bits<4>(mode, bm, prm, grid, st);
  if (bits == 8) return launch_bits<8>(mode, bm, prm, grid, st);
  return launch_bits<16>(mode, bm, prm, grid, st);
}

}  // namespace moe

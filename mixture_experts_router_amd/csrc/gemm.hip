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
  // tile order (see tile_of): n_tiles column tiles x m_tiles row tiles, in
  // groups of group_m row tiles; per_xcd consecutive tiles per XCD
  int n_tiles, m_tiles, group_m, per_xcd;
};

constexpr int NUM_XCD = 8;  // MI355X: workgroups go round-robin over 8 XCDs, each with its own L2

// Logical tile of workgroup `bid`.  The dispatcher places workgroup b on XCD
// b % 8, so XCD x is given the contiguous logical range [x*per_xcd,
// (x+1)*per_xcd).  Logical tiles run over groups of group_m row tiles, then
// column tiles, then the row tiles of the group: the workgroups of one XCD
// share a column tile's weights across the row tiles of a group and the
// group's activation rows across column tiles, in the same L2.  Returns false
// for indices past the last tile.
__device__ __forceinline__ bool tile_of(const GemmParams& prm, int bid, int& n, int& mt) {
  const int logical = (bid % NUM_XCD) * prm.per_xcd + bid / NUM_XCD;
  const int per_group = prm.n_tiles * prm.group_m;
  const int mg = logical / per_group;
  const int rem = logical - mg * per_group;
  const int gsz = min(prm.group_m, prm.m_tiles - mg * prm.group_m);
  if (gsz <= 0) return false;
  n = rem / gsz;
  if (n >= prm.n_tiles) return false;
  mt = mg * prm.group_m + rem % gsz;
  return true;
}

constexpr int A_STRIDE = 144;  // bytes per staged A row (64 fp16 + 16 bytes padding)

int gemm_block_m(int P, int E) {
  const int forced = tuning(TUNE_GEMM_BM);
  if (forced == 32 || forced == 64 || forced == 128) return forced;
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
  // cached loads: a lane reads part of a 128-byte line per group and the next
  // groups read the rest of it from L2
  for (int i = 0; i < BRaw<BITS>::WORDS / 4; ++i) r.q[i] = load16(p + 16 * i);
  if constexpr (BITS != 16) {
    r.s = srow[g];
    r.b = brow[g];
  }
}

// Dequantised B operand of MFMA k-step j (8 weights of this lane's column)
// of one group.  Every weight is w = fp16(fma(q, s, b)) (one rounding):
// codes become 1024 + q (or 1024 + 16q for the high nibble of a 4-bit byte)
// with v_and_or_b32 / v_perm_b32, an exact packed fp16 operation recovers q,
// and a packed fma applies the group's scale and bias.
template <int BITS>
__device__ __forceinline__ f16x8 dequant_b(const BRaw<BITS>& r, int j, const Q4Consts& qc) {
  if constexpr (BITS == 16) {
    return __builtin_bit_cast(f16x8, r.q[j]);
  } else {
    const f16 s = __builtin_bit_cast(f16, (uint16_t)r.s), b = __builtin_bit_cast(f16, (uint16_t)r.b);
    const f16x2 s2 = {s, s}, b2 = {b, b};
    const f16x2 m1024 = {(f16)-1024.0f, (f16)-1024.0f};
    auto lo = [&](uint32_t p) {  // 1024 + q  ->  s q + b
      const f16x2 q = __builtin_bit_cast(f16x2, p) + m1024;
      return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
    };
    if constexpr (BITS == 4) {
      const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f}, m64 = {(f16)-64.0f, (f16)-64.0f};
      auto hi = [&](uint32_t p) {  // 1024 + 16q  ->  q (exact)  ->  s q + b
        const f16x2 q = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, p), sixteenth, m64);
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
      };
      const uint32_t w = j == 0 ? r.q[0].x : j == 1 ? r.q[0].y : j == 2 ? r.q[0].z : r.q[0].w;
      uint32_t p04, p15, p26, p37;
      q4_word_unpack(w, qc, p04, p15, p26, p37);
      const u32x4 o = {lo(p04), hi(p15), lo(p26), hi(p37)};
      return __builtin_bit_cast(f16x8, o);
    } else {
      const u32x4 q = r.q[j / 2];
      const uint32_t w0 = (j & 1) ? q.z : q.x, w1 = (j & 1) ? q.w : q.y;
      uint32_t p0[2], p1[2];
      q8_word_to_biased_pairs(w0, p0);
      q8_word_to_biased_pairs(w1, p1);
      const u32x4 o = {lo(p0[0]), lo(p0[1]), lo(p1[0]), lo(p1[1])};
      return __builtin_bit_cast(f16x8, o);
    }
  }
}

// One workgroup = one (expert, row tile, column tile).  4 waves side by side
// along N, each 32*MS rows x 64 columns (two 32-column subtiles; fused: 32
// gate and the matching 32 up columns).  K advances one 64-column group per
// step.  Software pipeline, one barrier per group:
//   A (activation rows): global loads two groups ahead into a 2-deep register
//     ring, converted to fp16 and written to a double-buffered LDS tile one
//     group ahead;
//   B (weights): loads two groups ahead into a 2-deep register ring,
//     dequantised right before use.
// Every load is issued on every path (rows past the tile re-read the tile's
// first row, groups past the end re-read the last group, columns past N
// re-read column 0; none of those results is stored), so the compiler's wait
// counts stay exact and loads stay in flight across the MFMAs.
template <int BITS, int MODE, int MS, int ACT>
__global__ __launch_bounds__(256, MS == 4 ? 1 : 2) void gemm_kernel(GemmParams prm) {
  constexpr int BM = 32 * MS;
  constexpr int APT = BM * 8 / 256;  // 16-byte A pieces per thread per group
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][BM * A_STRIDE];
  __shared__ int s_tile[4];

  const int lane = lane_id();
  const int wave = wave_id();
  const int tid = threadIdx.x;

  // ---- which (expert, M tile) this workgroup owns: tiles are numbered
  // expert by expert, ceil(count/BM) tiles per expert
  int n_tile = 0, y = 0;
  if (!tile_of(prm, blockIdx.x, n_tile, y)) return;
  if (tid < WAVE) {
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
  const Q4Consts qc = q4_consts();

  // ---- A sources: APT pieces per thread, fixed across groups
  const uint16_t* a_src[APT];
  int a_off[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int pc = tid + 256 * i;
    const int r = pc / 8, j = pc % 8;
    const int rr = r < rows ? r : 0;  // past the tile: the tile's first row (never stored)
    a_off[i] = r * A_STRIDE + j * 16;
    if constexpr (MODE == GEMM_ROWS_F16) {
      a_src[i] = prm.a + (size_t)(row0 + rr) * K + 8 * j;
    } else {
      const int pair = prm.perm[row0 + rr];
      a_src[i] = prm.a + (size_t)(pair / prm.kcap) * K + 8 * j;
    }
  }

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
    col0 = n_tile * 128 + wave * 32;
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
    col0 = n_tile * 256 + wave * 64;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      valid[ni] = col0 + 32 * ni < prm.N;
      const int64_t row = (int64_t)e * prm.w0.stride + (valid[ni] ? col0 + 32 * ni + col_in : 0);
      bq[ni] = prm.w0.q + row * row_bytes;
      bs[ni] = BITS == 16 ? nullptr : prm.w0.s + row * ng;
      bb[ni] = BITS == 16 ? nullptr : prm.w0.b + row * ng;
    }
  }

  f32x16 acc[MS][2];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  u32x4 areg[2][APT];
  BRaw<BITS> braw[2][2];
  auto load_a = [&](u32x4 (&dst)[APT], int g) {
#pragma unroll
    for (int i = 0; i < APT; ++i) dst[i] = load16(a_src[i] + (size_t)g * 64);
  };
  auto store_a = [&](const u32x4 (&src)[APT], int buf) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      u32x4 v = src[i];
      if constexpr (ACT == ACT_BF16) v = act8_to_f16(v, ACT_BF16);
      if constexpr (BITS == 4) v = perm8_nibble_order(v);
      *(u32x4*)(&a_lds[buf][a_off[i]]) = v;
    }
  };
  auto load_bg = [&](BRaw<BITS> (&dst)[2], int g) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) load_b<BITS>(dst[ni], bq[ni], bs[ni], bb[ni], g, hh);
  };
  auto mma = [&](const BRaw<BITS> (&src)[2], int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x8 b0 = dequant_b<BITS>(src[0], j, qc), b1 = dequant_b<BITS>(src[1], j, qc);
#pragma unroll
      for (int mi = 0; mi < MS; ++mi) {
        const f16x8 af = *(const f16x8*)(&a_lds[buf][(mi * 32 + col_in) * A_STRIDE + (32 * hh + 8 * j) * 2]);
        acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b0, acc[mi][0], 0, 0, 0);
        acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b1, acc[mi][1], 0, 0, 0);
      }
    }
  };
  const int last = ng - 1;
  auto gi = [&](int g) { return g < last ? g : last; };

  // prologue: A(0) in LDS, A(1) and B(0), B(1) in flight
  load_a(areg[0], 0);
  load_a(areg[1], gi(1));
  load_bg(braw[0], 0);
  load_bg(braw[1], gi(1));
  store_a(areg[0], 0);
  __syncthreads();

  // group g: A(g) in LDS buffer g%2, A(g+1) in areg[(g+1)%2], B(g) in braw[g%2]
  for (int g = 0; g < ng; g += 2) {
    load_a(areg[0], gi(g + 2));
    mma(braw[0], 0);
    load_bg(braw[0], gi(g + 2));
    store_a(areg[1], 1);
    __syncthreads();
    if (g + 1 >= ng) break;
    load_a(areg[1], gi(g + 3));
    mma(braw[1], 1);
    load_bg(braw[1], gi(g + 3));
    store_a(areg[0], 0);
    __syncthreads();
  }

  if (!valid[0]) return;
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

template <int BITS, int MODE, int ACT>
static hipError_t launch_act(int bm, const GemmParams& prm, dim3 grid, hipStream_t st) {
  switch (bm) {
    case 32: return launch_kernel(gemm_kernel<BITS, MODE, 1, ACT>, grid, 256, 0, st, prm);
    case 64: return launch_kernel(gemm_kernel<BITS, MODE, 2, ACT>, grid, 256, 0, st, prm);
    case 128: return launch_kernel(gemm_kernel<BITS, MODE, 4, ACT>, grid, 256, 0, st, prm);
    default: return hipErrorInvalidValue;
  }
}

// the down projection reads fp16 SwiGLU rows whatever the activation dtype
template <int BITS, int MODE>
static hipError_t launch_ms(int bm, const GemmParams& prm, dim3 grid, hipStream_t st) {
  if (MODE != GEMM_ROWS_F16 && prm.act == ACT_BF16) return launch_act<BITS, MODE, ACT_BF16>(bm, prm, grid, st);
  return launch_act<BITS, MODE, ACT_F16>(bm, prm, grid, st);
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
  prm.n_tiles = (N + ncols - 1) / ncols;
  prm.m_tiles = max_mtiles;
  prm.group_m = tuning(TUNE_GEMM_GROUP_M);
  const int64_t total = (int64_t)prm.n_tiles * prm.m_tiles;
  prm.per_xcd = (int)((total + NUM_XCD - 1) / NUM_XCD);
  dim3 grid((unsigned)(prm.per_xcd * NUM_XCD));
  if (bits == 4) return launch_bits<4>(mode, bm, prm, grid, st);
  if (bits == 8) return launch_bits<8>(mode, bm, prm, grid, st);
  return launch_bits<16>(mode, bm, prm, grid, st);
}

}  // namespace moe

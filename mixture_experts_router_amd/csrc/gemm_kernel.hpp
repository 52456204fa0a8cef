// Batched path: grouped GEMM over the expert-sorted pairs on the matrix cores.
//
// Rows of one M tile are consecutive sorted pairs of one expert (the sorted
// gather branch of the oMLX gate/up fusion page), so every tile multiplies one
// expert's weights.  Three instantiations:
//   GEMM_FUSED_SWIGLU  A = activation rows gathered through perm, B = the
//                      fused gate_up tensor; each wave owns 32 gate and the
//                      matching 32 up columns, so the SwiGLU epilogue
//                      h = silu(g) * u is local to a lane (oMLX page, steps 3-4:
//                      one matmul over the [gate, up] concatenation, split,
//                      then activation)
//   GEMM_GATHER_F32    the same A, one projection, fp32 output (unfused path)
//   GEMM_ROWS_F16      A = h rows in sorted order, B = down, fp16 output
//
// The A operand is fp16 in HBM, each 8-element block in the order in which
// the weights unpack (4-bit: 0,2,4,6,1,3,5,7; otherwise natural): the
// activations are converted once by sort_prep_kernel and the fused epilogue
// writes h that way.  Tile: BM = 32*MS rows x 256 columns (fused: 128
// gate/up column pairs), 4 waves side by side along N, each 32*MS x 64; K
// advances one 64-column quantisation group per step.
//
// Both operands stream HBM -> LDS with global_load_lds_dwordx4 (no register
// staging) through NS stages sized to the LDS: A rows with a 16-byte-chunk XOR
// swizzle (see piece_swizzle) so the MFMA operand reads are conflict free;
// each wave's 64 weight rows into its own LDS region; the stage's scales and
// biases (KG fp16 values of a column per lane) beside them.  One wait (this wave's loads of the
// stage) and one barrier (every wave's loads; the oldest stage free) per
// group, then the next group's loads are issued and the stage is consumed:
// B codes read once per group, dequantised per MFMA k-step in registers
// (w = fma(q, s, b) in fp16, one rounding), v_mfma_f32_32x32x16_f16 with fp32
// accumulation.  NVFP4 weights stage like 4-bit codes; each code pair becomes
// an exact fp16 E2M1 pair (one conversion instruction) times its block's
// E4M3 scale (exact in fp16: at most six significant bits), and the tensor
// scale multiplies the fp32 sums in the epilogue.
//
// Each output element's reduction runs over the same k order whichever
// instantiation, tile or column position computes it, so the fused and
// unfused paths produce identical bits.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct GemmParams {
  const uint16_t* a;  // fp16 operand rows, 8-element blocks in the weights' unpack order
  const int32_t* perm;
  const int32_t* counts;
  const int32_t* offsets;
  int kcap, E, K, N;
  WView w0, w1;
  void* out;
  float* pre;  // fused: fp32 gate and up sums [pairs, 2N] in pair order (NULL: not kept)
  const int32_t* tokexp;  // gather modes, bf16 activations: each token's exponent a_t (NULL: 0)
  const int32_t* any_scaled;  // nonzero when some a_t > 0 (tokexp is read only then)
  uint32_t a_bytes;  // extent of the A rows (offsets at or past it read nothing)
  int32_t sb_up_delta;  // fused: bytes from a gate column's packed scales to its up column's
  int perm8_out;  // fused: store h blocks in the 4-bit order (q4g_order)
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

// Geometry of one pipeline stage (KG quantisation groups of 64 k columns) of
// a wave's weight rows in LDS.  Each 32-row subtile is loaded by IPS whole
// load instructions: instruction i of a subtile moves its 16-byte pieces
// 64i .. 64i+63 in row-major (row, piece) order, so the subtile sits
// row-major [32 rows][SEG bytes] at the start of its SUBB-byte region.  For
// 4-, 8- and 16-bit codes a row is a power-of-two number of pieces and an
// instruction covers whole rows (DRAM streams rows in segments of at least 64
// bytes far better than in 32); 5- and 6-bit group rows are 40 and 48 bytes,
// so rows straddle instructions and the last instruction of a subtile has
// spare lanes, which re-read the subtile's first piece into the padding.  No
// instruction spans two subtiles, whose rows may lie in different tensors
// (gate and up).
template <int BITS, int KG, int NSUB>
struct BGeo {
  static constexpr int ROW = 64 * code_bits(BITS) / 8;  // code bytes of one row per group: 32 / 40 / 48 / 64 / 128
  static constexpr int SEG = KG * ROW;               // bytes of one row per stage
  static constexpr int LPR = SEG / 16;               // 16-byte pieces per row
  static constexpr bool WHOLE = 64 % LPR == 0;       // an instruction covers whole rows
  static constexpr int IPS = (32 * LPR + 63) / 64;   // load instructions per 32-row subtile
  static constexpr int SUBB = IPS * 1024;            // LDS bytes per subtile (32 * SEG, then padding)
  static constexpr int ROWS = 32 * NSUB;             // weight rows (output columns) per wave
  static constexpr int NI = NSUB * IPS;              // load instructions per wave
  static constexpr int WB = NSUB * SUBB;             // LDS bytes of a wave's weight rows
  static constexpr int HALF = ROW / 2;               // bytes a lane feeds per group (its half of the group's k)
  static constexpr int READS = HALF / 16;            // (4, 8, 16 bits) 16-byte LDS reads per lane, subtile, group
  static_assert(SEG % 16 == 0, "a stage row is whole 16-byte pieces");
};

// WPC: workgroups per CU the LDS budget allows (1: 156 KB, 2: 78 KB, 3: 52 KB each)
template <int BITS, int MS, int KG, int NSUB, int KS, int WPC>
struct GemmCfg {
  static constexpr int BM = 32 * MS;
  static constexpr int A_SUB = BM * 128;  // A of one group: BM rows x 64 fp16
  static constexpr int A_BYTES = KG * A_SUB;
  static constexpr int B_BYTES = 4 * BGeo<BITS, KG, NSUB>::WB;
  // scales and biases: per column block one 1 KB region (one 64-lane load of
  // its 32*NSUB columns' packed group pair, repeated over the spare lanes)
  static constexpr int SC_BYTES = BITS != 16 ? 4 * 1024 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  static constexpr int BUDGET = WPC == 1 ? 156 * 1024 : WPC == 2 ? 78 * 1024 : 52 * 1024;
  static constexpr int NS_FIT = BUDGET / STAGE;
  static constexpr int NS = NS_FIT < 2 ? 2 : (NS_FIT > 6 ? 6 : NS_FIT);
  // vector memory instructions per wave per stage: A, B, scales and biases
  // (the KS waves of a column block split its loads evenly; A instructions
  // per wave and group: MS / KS, or at 32-row tiles with two waves per column
  // block one each, both waves loading the same rows into the same LDS bytes)
  static_assert((MS % KS == 0 || MS == 1) && BGeo<BITS, KG, NSUB>::NI % KS == 0, "loads split over the K waves");
  static constexpr int NA = (MS + KS - 1) / KS;
  static constexpr int LOADS = KG * NA + BGeo<BITS, KG, NSUB>::NI / KS + (BITS != 16 ? 1 : 0);
  static_assert((NS - 2) * LOADS <= 63, "vmcnt range");
  static_assert(NS * STAGE <= 159 * 1024, "LDS");
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS layout swizzles.  A 16-byte read by a wave is served in phases over
// bank rows of LDS_BANK_ROW bytes; rows of a tile that start in the same
// bank row would collide on the same banks.  Each tile row's 16-byte pieces
// are XOR-permuted by the row's index in units of the rows that share a bank
// row, so the lanes of a phase (consecutive rows, same logical piece) hit
// distinct banks.
#ifndef MOE_LDS_BANK_ROW
#define MOE_LDS_BANK_ROW 256
#endif
template <int ROW_BYTES>
__device__ __forceinline__ int piece_swizzle(int row) {
  constexpr int PIECES = ROW_BYTES / 16;
  constexpr int SHARE = MOE_LDS_BANK_ROW / ROW_BYTES > 1 ? MOE_LDS_BANK_ROW / ROW_BYTES : 1;
  return (row / SHARE) % PIECES;
}

// 16 bytes per lane from buffer r at voff + soff into LDS (lane i at dst + 16 i)
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, soff, 0, 0);
}

// wait until at most N vector memory instructions of this wave are pending
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int V>
struct IC {
  static constexpr int value = V;
};

// f(IC<0>), f(IC<1>), ... while f returns true
template <int S, int N, typename F>
__device__ __forceinline__ void for_stages(F&& f) {
  if constexpr (S < N) {
    if (f(IC<S>{})) for_stages<S + 1, N>(f);
  }
}

// Dequantised B operand of MFMA k-step j (8 weights of this lane's column)
// of one group, from the lane's code bytes c (4-bit: c[0]; 8-bit: c[0..1];
// fp16: c[0..3]).  Every weight is w = fp16(fma(q, s, b)) (one rounding):
// 4-bit codes become exact fp16 pairs through the fp8 conversion below;
// 8-bit codes become 1024 + q with v_perm_b32 and an exact packed fp16
// subtraction recovers q; a packed fma applies the group's scale and bias.
template <int BITS>
__device__ __forceinline__ f16x8 dequant_b(const u32x4* c, int j, uint32_t s_bits, uint32_t b_bits,
                                           const Q4Consts& qc) {
  if constexpr (BITS == 16) {
    return __builtin_bit_cast(f16x8, c[j]);
  } else {
    const f16 s = __builtin_bit_cast(f16, (uint16_t)s_bits), b = __builtin_bit_cast(f16, (uint16_t)b_bits);
    const f16x2 s2 = {s, s}, b2 = {b, b};
    const f16x2 m1024 = {(f16)-1024.0f, (f16)-1024.0f};
    auto lo = [&](uint32_t p) {  // 1024 + q  ->  s q + b
      const f16x2 q = __builtin_bit_cast(f16x2, p) + m1024;
      return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
    };
    if constexpr (BITS == 4) {
      // the low nibbles of the word's bytes are codes (0, 2, 4, 6), the high
      // nibbles (1, 3, 5, 7), one per byte after two masks.  A byte holding
      // q in 0..15 is the FP8 E4M3 pattern of q * 2^-9 (subnormal below 8,
      // exponent field 1 from 8 on), so the scaled conversion with 2^9 gives
      // a pair of codes exactly, one instruction per pair; the operand rows
      // are in the matching order (q4g_order)
      const uint32_t w = j == 0 ? c[0].x : j == 1 ? c[0].y : j == 2 ? c[0].z : c[0].w;
      const uint32_t lo4 = w & 0x0F0F0F0Fu, hi4 = (w >> 4) & 0x0F0F0F0Fu;
      auto fq = [&](f16x2 q) { return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2)); };
      const u32x4 o = {fq(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo4, 512.0f, false)),   // (k0, k2)
                       fq(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo4, 512.0f, true)),    // (k4, k6)
                       fq(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi4, 512.0f, false)),   // (k1, k3)
                       fq(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi4, 512.0f, true))};   // (k5, k7)
      (void)qc;
      return __builtin_bit_cast(f16x8, o);
    } else {
      const u32x4 q = c[j / 2];
      const uint32_t w0 = (j & 1) ? q.z : q.x, w1 = (j & 1) ? q.w : q.y;
      uint32_t p0[2], p1[2];
      q8_word_to_biased_pairs(w0, p0);
      q8_word_to_biased_pairs(w1, p1);
      const u32x4 o = {lo(p0[0]), lo(p0[1]), lo(p1[0]), lo(p1[1])};
      return __builtin_bit_cast(f16x8, o);
    }
  }
}

// The same for 5- and 6-bit codes: w holds the lane's half of a group row,
// 32 codes as a little-endian bit stream (code c at bits BITS*c); k-step j
// takes codes 8j .. 8j+7 in natural order.  Each pair of codes becomes the
// fp16 pair (1024 + q, 1024 + q') with exponent bits 0x6400, then
// w = fp16(fma(q, s, b)) as for 8-bit codes.
template <int BITS>
__device__ __forceinline__ f16x8 dequant_b_odd(const uint32_t* w, int j, uint32_t s_bits, uint32_t b_bits) {
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  auto code = [&](int c) __attribute__((always_inline)) -> uint32_t {
    const int bit = BITS * c, wd = bit >> 5, sh = bit & 31;
    if (sh + BITS <= 32) return (w[wd] >> sh) & MASK;
    return ((w[wd] >> sh) | (w[wd + 1] << (32 - sh))) & MASK;
  };
  const f16 s = __builtin_bit_cast(f16, (uint16_t)s_bits), b = __builtin_bit_cast(f16, (uint16_t)b_bits);
  const f16x2 s2 = {s, s}, b2 = {b, b};
  const f16x2 m1024 = {(f16)-1024.0f, (f16)-1024.0f};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = 0x64006400u | code(8 * j + 2 * i) | (code(8 * j + 2 * i + 1) << 16);
    const f16x2 q = __builtin_bit_cast(f16x2, p) + m1024;
    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  const u32x4 v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(f16x8, v);
}

// NVFP4: k-step J of the lane's share of a group, 8 codes in column order
// in one word of c; sv holds the E4M3 scales of the lane's two 16-column
// blocks (low byte first), k-steps 2i and 2i+1 using block i.
// w = fp16(e2m1) * fp16(e4m3), exact.
template <int J>
__device__ __forceinline__ f16x8 dequant_b_f4(const u32x4* c, uint32_t sv) {
  const uint32_t w = J == 0 ? c[0].x : J == 1 ? c[0].y : J == 2 ? c[0].z : c[0].w;
  const f16 s = (f16)e4m3_byte<J / 2>(sv);
  const f16x2 s2 = {s, s};
  uint32_t p[4];
  e2m1_word_to_pairs(w, p);
  u32x4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p[0]) * s2);
  o.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p[1]) * s2);
  o.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p[2]) * s2);
  o.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p[3]) * s2);
  return __builtin_bit_cast(f16x8, o);
}

template <bool C, typename A, typename B>
struct Pick {
  typedef A T;
};
template <typename A, typename B>
struct Pick<false, A, B> {
  typedef B T;
};

template <int BITS, int MODE, int MS, int KG, int NSUB, int KS, int WPC>
__global__ __launch_bounds__(256 * KS, WPC) void gemm_kernel(GemmParams prm) {
  using G = BGeo<BITS, KG, NSUB>;
  using C = GemmCfg<BITS, MS, KG, NSUB, KS, WPC>;
  constexpr int HALFSUB = NSUB / 2;  // fused: subtiles [0, HALFSUB) gate, the rest the matching up
  constexpr int BM = C::BM, NS = C::NS;
  // one array per stage: distinct objects let the compiler see that reading
  // a stage does not wait on loads still landing in the others
  __shared__ __attribute__((aligned(16))) uint8_t st0[C::STAGE], st1[C::STAGE], st2[NS > 2 ? C::STAGE : 16],
      st3[NS > 3 ? C::STAGE : 16], st4[NS > 4 ? C::STAGE : 16], st5[NS > 5 ? C::STAGE : 16];
  auto stage = [&](auto S_) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(S_)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2;
    else if constexpr (S == 3) return st3;
    else if constexpr (S == 4) return st4;
    else return st5;
  };

  const int lane = lane_id();
  const int wave = wave_id();                 // 0 .. 4*KS-1
  const int wn = wave % 4;                    // column block of this wave
  const int kh = KS == 1 ? 0 : wave / 4;      // which share of each group's k-steps
  constexpr int JW = 4 / KS;                  // MFMA k-steps per group and wave

  // ---- which (expert, M tile) this workgroup owns: tiles are numbered
  // expert by expert, ceil(count/BM) tiles per expert.  Every wave finds it
  // itself from one round of loads (counts and offsets together): no LDS
  // hand-off, no barrier, one memory latency.
  int n_tile = 0, y = 0;
  if (!tile_of(prm, blockIdx.x, n_tile, y)) return;
  int e = -1, rows = 0, row0 = 0;
  {
    int base_tiles = 0, fe = -1, fmt = 0, fc = 0, fo = 0;
    for (int base = 0; base < prm.E; base += WAVE) {
      const int ee = base + lane;
      const int c = ee < prm.E ? prm.counts[ee] : 0;
      const int o = ee < prm.E ? prm.offsets[ee] : 0;
      const int nt = (c + BM - 1) / BM;
      int incl = nt;
#pragma unroll
      for (int d = 1; d < WAVE; d <<= 1) {
        int v = __shfl_up(incl, d, WAVE);
        if (lane >= d) incl += v;
      }
      const int excl = incl - nt;
      if (nt > 0 && y >= base_tiles + excl && y < base_tiles + incl) {
        fe = ee;
        fmt = y - base_tiles - excl;
        fc = c;
        fo = o;
      }
      base_tiles += __shfl(incl, WAVE - 1, WAVE);
    }
    const uint64_t m = __ballot(fe >= 0);
    if (m != 0) {
      const int src = __ffsll((unsigned long long)m) - 1;
      e = __builtin_amdgcn_readlane(fe, src);
      const int m0 = __builtin_amdgcn_readlane(fmt, src) * BM;
      rows = min(BM, __builtin_amdgcn_readlane(fc, src) - m0);
      row0 = __builtin_amdgcn_readlane(fo, src) + m0;
    }
  }
  if (e < 0) return;  // the same in every wave of the workgroup
  const int K = prm.K;
  const int ng = K / 64;
  const Q4Consts qc = q4_consts();
  const int hh = lane / 32;
  const int col_in = lane % 32;

  // All loads are buffer loads: base addresses in scalar registers, a fixed
  // 32-bit byte offset per lane, the group's offset as the scalar offset.
  //
  // ---- A: the tile's 4*MS load instructions per group, MS/KS per wave;
  // instruction q covers tile rows r0 = 8*q .. r0+7; lane i writes LDS chunk
  // i%8 of row r0 + i/8, which holds the row's logical 16-byte chunk
  // (i%8) ^ piece_swizzle(row).  Lanes of rows past the tile point past the
  // descriptor's range: no memory access (their LDS rows are never used).
  constexpr int NA = C::NA;
  const int qa0 = MS >= KS ? wn * MS + kh * NA : wn * MS;  // this wave's first A instruction
  const rsrc_t ra = make_rsrc(prm.a, prm.a_bytes);
  uint32_t a_off[NA];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    const int r = 8 * (qa0 + q) + lane / 8;
    const int rr = r < rows ? r : 0;
    uint32_t arow;
    if constexpr (MODE == GEMM_ROWS_F16) arow = (uint32_t)(row0 + rr);
    else arow = (uint32_t)(prm.perm[row0 + rr] / prm.kcap);
    const int chunk = (lane & 7) ^ piece_swizzle<128>(r);
    a_off[q] = r < rows ? arow * (uint32_t)K * 2u + (uint32_t)chunk * 16u : 0x80000000u;
  }

  // ---- B: this wave's 32*NSUB weight rows; rows [32 ni, 32 ni + 32) are
  // subtile ni (fused: NSUB/2 subtiles of gate columns, then the matching up
  // columns).  Columns past N re-read column 0 (never stored).
  int col0;  // first output column of this wave (fused: first gate / h column)
  bool valid[NSUB];
  const WView* view[NSUB];
#pragma unroll
  for (int ni = 0; ni < NSUB; ++ni) {
    if constexpr (MODE == GEMM_FUSED_SWIGLU) {
      col0 = n_tile * (4 * 32 * HALFSUB) + wn * 32 * HALFSUB;
      valid[ni] = col0 + 32 * (ni % HALFSUB) < prm.N;
      view[ni] = ni < HALFSUB ? &prm.w0 : &prm.w1;
    } else {
      col0 = n_tile * (4 * 32 * NSUB) + wn * 32 * NSUB;
      valid[ni] = col0 + 32 * ni < prm.N;
      view[ni] = &prm.w0;
    }
  }
  auto column = [&](int ni, int rin) __attribute__((always_inline)) {
    const int c = col0 + 32 * (MODE == GEMM_FUSED_SWIGLU ? ni % HALFSUB : ni) + rin;
    return valid[ni] ? c : 0;
  };
  const int64_t row_bytes = (int64_t)K * code_bits(BITS) / 8;
  // packed_q: each 32-row block's units (UG groups, PB bytes per row)
  // contiguous, so a step streams 32*PB contiguous bytes per block
  const bool tiled = prm.w0.pq != nullptr;
  constexpr int UG = BITS == 6 || BITS == 16 ? 1 : 2;
  constexpr int PB = UG * G::ROW;
  static_assert(UG == 2 || KG == 1, "one-group units are read one group per step");
  const int nu = (ng + UG - 1) / UG;
  const int np = (ng + 1) / 2;
  const uint8_t* qbase[NSUB];
#pragma unroll
  for (int ni = 0; ni < NSUB; ++ni) {
    const WView& v = *view[ni];
    qbase[ni] = tiled ? v.pq + (int64_t)e * v.pq_expert : v.q + (int64_t)e * v.stride * row_bytes;  // the expert's start
  }
  // ---- scales and biases (packed_sb layout: 8 bytes per column and group
  // pair, columns contiguous): one load per step, lane l takes the 16 bytes
  // of columns 2(c%16), 2(c%16)+1 of subtile c/16, c = l % (16 NSUB); the up
  // columns of the fused tensor lie sb_up_delta bytes after the gate columns
  const int64_t sb_expert = (int64_t)np * prm.w0.sb_stride * 8;
  const rsrc_t rsb = make_rsrc(prm.w0.sb + (BITS != 16 ? e * sb_expert : 0), (uint32_t)sb_expert);
  uint32_t sb_off;
  {
    const int c = lane % (16 * NSUB), ni = c / 16;
    uint32_t off = 0;
#pragma unroll
    for (int n2 = 0; n2 < NSUB; ++n2)
      if (n2 == ni) off = (uint32_t)column(n2, 2 * (c % 16)) * 8u;
    if (MODE == GEMM_FUSED_SWIGLU && ni >= HALFSUB) off += (uint32_t)prm.sb_up_delta;
    sb_off = off;
  }
  // this wave's weight load instructions: q = q0 + qq, qq < NI / KS (the K
  // waves of a column block split its loads); q0 and the subtile of an
  // instruction are wave-uniform, so the descriptors stay in scalar registers
  constexpr int NQ = G::NI / KS;
  const int q0 = kh * NQ;
  rsrc_t rq[NQ];
  uint32_t b_off[NQ];
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int q = q0 + qq;
    const int sub = q / G::IPS;  // the instruction's subtile
    const uint8_t* base = qbase[0];
#pragma unroll
    for (int ni = 1; ni < NSUB; ++ni) base = sub == ni ? qbase[ni] : base;
    rq[qq] = make_rsrc(base, 0xFFFFFFFFu);
    const int item = (q % G::IPS) * 64 + lane;  // (row, piece) of the subtile, row-major
    const bool live = item < 32 * G::LPR;       // spare lanes re-read the first piece (into the padding)
    const int r_in = live ? item / G::LPR : 0;
    const int pl = live ? item % G::LPR : 0;
    const int piece = G::WHOLE ? pl ^ piece_swizzle<G::SEG>(sub * 32 + r_in) : pl;
    const int c = column(sub, r_in);
    b_off[qq] = (tiled ? (uint32_t)((((int64_t)(c >> 5) * nu) * 32 + (c & 31)) * PB) : (uint32_t)(c * row_bytes)) +
                (uint32_t)piece * 16u;
  }
  const int nst = ng / KG;  // pipeline steps (the launcher makes KG divide ng)

  f32x16 acc[MS][NSUB];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int ni = 0; ni < NSUB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // this column block's scale region (both waves of a K split load it, alike)
  const int sc_wave = C::A_BYTES + C::B_BYTES + wn * 1024;
  const int b_wave = C::A_BYTES + wn * G::WB;  // this wave's B codes
  const int last = nst - 1;
  // step k (groups KG k .. KG k + KG - 1; clamped to the last step) into stage S
  auto issue = [&](auto S_, int k) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value;
    k = k < last ? k : last;
    uint8_t* st = stage(S_);
#pragma unroll
    for (int gi = 0; gi < KG; ++gi)
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        const int lds_off = gi * C::A_SUB + 8 * (qa0 + q) * 128;
        dma16(ra, a_off[q], (uint32_t)(k * KG + gi) * 128u, st + lds_off);
      }
    // the step's bytes of each row: stage k of the row-major rows, or (packed
    // layout) unit k (a unit per stage) or half k%2 of two-group unit k/2
    const uint32_t b_soff = !tiled ? (uint32_t)k * G::SEG
                            : KG == UG ? (uint32_t)k * 32u * PB
                                       : (uint32_t)(k >> 1) * 32u * PB + (uint32_t)(k & 1) * G::ROW;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const int lds_off = C::A_BYTES + wn * G::WB + (q0 + qq) * 1024;
      dma16(rq[qq], b_off[qq], b_soff, st + lds_off);
    }
    if constexpr (BITS != 16) {
      const uint32_t pair = KG == 2 ? (uint32_t)k : (uint32_t)k >> 1;  // group pair of the step
      dma16(rsb, sb_off, pair * (uint32_t)prm.w0.sb_stride * 8u, st + sc_wave);
    }
  };
  // ---- reading a stage.  LDS addresses are formed as one integer offset
  // from the stage array: the compiler attributes an access to its array (and
  // so knows it does not wait on loads landing in other stages) only through
  // a short chain of address arithmetic on the array itself.
  //
  // This wave's share of a lane's code bytes of a group: RB bytes (its JW
  // k-steps) at byte kh*RB of the lane's half of the group.
  constexpr int RB = G::HALF / KS;
  constexpr int RT = RB >= 16 ? RB / 16 : 1;
  constexpr bool ODD = BITS == 5 || BITS == 6;  // 5- and 6-bit codes: 20 or 24 bytes per lane and group
  static_assert(!ODD || KS == 1, "5- and 6-bit codes: one wave per column block");
  struct CodesPow2 {
    u32x4 v[NSUB][RT];
  };
  struct CodesOdd {
    uint32_t w[NSUB][6];
  };
  typedef typename Pick<ODD, CodesOdd, CodesPow2>::T Codes;
  // kodd: odd step (one-group stages take the second group of the pair)
  auto read_codes = [&](const uint8_t* st, auto GI_, Codes& bc, uint32_t (&sv)[NSUB], uint32_t (&bv)[NSUB],
                        bool kodd) __attribute__((always_inline)) {
    constexpr int gi = decltype(GI_)::value;
#pragma unroll
    for (int ni = 0; ni < NSUB; ++ni) {
      const int r = ni * 32 + col_in;
      if constexpr (ODD) {
        // the lane's half of the group row: 20 bytes (five words) or 24 (three pairs)
        const int at = b_wave + ni * G::SUBB + col_in * G::SEG + gi * G::ROW + hh * G::HALF;
        if constexpr (BITS == 5) {
#pragma unroll
          for (int w = 0; w < 5; ++w) bc.w[ni][w] = *(const uint32_t*)(st + (at + 4 * w));
          bc.w[ni][5] = 0u;
        } else {
#pragma unroll
          for (int w = 0; w < 3; ++w) {
            const u32x2 v = *(const u32x2*)(st + (at + 8 * w));
            bc.w[ni][2 * w] = v.x;
            bc.w[ni][2 * w + 1] = v.y;
          }
        }
      } else if constexpr (RB >= 16) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int piece = (gi * (G::ROW / 16) + hh * G::READS + kh * RT + t) ^ piece_swizzle<G::SEG>(r);
          bc.v[ni][t] = *(const u32x4*)(st + (b_wave + r * G::SEG + piece * 16));
        }
      } else {  // 8 bytes inside one piece
        const int piece = (gi * (G::ROW / 16) + hh * G::READS) ^ piece_swizzle<G::SEG>(r);
        const u32x2 v = *(const u32x2*)(st + (b_wave + r * G::SEG + piece * 16 + kh * 8));
        bc.v[ni][0] = u32x4{v.x, v.y, 0u, 0u};
      }
      if constexpr (BITS == NVF4) {
        // the slot's two words are the block scales of the pair's groups;
        // this lane's k-steps cover blocks 2hh + kh*JW/2 onward
        const u32x2 sb = *(const u32x2*)(st + (sc_wave + (ni * 16 + col_in / 2) * 16 + (col_in & 1) * 8));
        const bool hi = KG == 2 ? gi == 1 : kodd;
        sv[ni] = ((hi ? sb.y : sb.x) >> (16 * hh + 8 * (kh * JW / 2))) & 0xFFFFu;
        bv[ni] = 0u;
      } else if constexpr (BITS != 16) {
        const u32x2 sb = *(const u32x2*)(st + (sc_wave + (ni * 16 + col_in / 2) * 16 + (col_in & 1) * 8));
        const bool hi = KG == 2 ? gi == 1 : kodd;
        sv[ni] = hi ? sb.x >> 16 : sb.x & 0xFFFFu;
        bv[ni] = hi ? sb.y >> 16 : sb.y & 0xFFFFu;
      } else {
        sv[ni] = bv[ni] = 0;
      }
    }
  };
  // A fragments of group gi, k-step kh*JW + jj of the group
  // msv: 32-row subtiles holding rows of the tile (wave-uniform); the
  // eight-wave loop skips the others' reads and MFMAs
  const int msv = __builtin_amdgcn_readfirstlane(min(MS, (rows + 31) / 32));
  auto read_a = [&](const uint8_t* st, auto GI_, auto JJ_, f16x8 (&af)[MS], bool skip = false)
                    __attribute__((always_inline)) {
    constexpr int gi = decltype(GI_)::value, jj = decltype(JJ_)::value;
#pragma unroll
    for (int mi = 0; mi < MS; ++mi) {
      if (skip && mi > 0 && mi >= msv) break;
      const int row = mi * 32 + col_in;
      const int piece = (4 * hh + kh * JW + jj) ^ piece_swizzle<128>(row);
      af[mi] = *(const f16x8*)(st + (gi * C::A_SUB + row * 128 + (piece << 4)));
    }
  };
  auto deq = [&](const Codes& bc, const uint32_t (&sv)[NSUB], const uint32_t (&bv)[NSUB], auto JJ_,
                 f16x8 (&bf)[NSUB]) __attribute__((always_inline)) {
    constexpr int jj = decltype(JJ_)::value;
#pragma unroll
    for (int ni = 0; ni < NSUB; ++ni) {
      if constexpr (ODD) bf[ni] = dequant_b_odd<BITS>(bc.w[ni], jj, sv[ni], bv[ni]);
      else if constexpr (BITS == NVF4) bf[ni] = dequant_b_f4<jj>(bc.v[ni], sv[ni]);
      else bf[ni] = dequant_b<BITS>(bc.v[ni], jj, sv[ni], bv[ni], qc);
    }
  };
  auto mma = [&](const f16x8 (&af)[MS], const f16x8 (&bf)[NSUB], bool skip = false) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < MS; ++mi) {
      if (skip && mi > 0 && mi >= msv) break;
#pragma unroll
      for (int ni = 0; ni < NSUB; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
  };

  // One stage, one wave per column block: 4 KG MFMA k-steps.  A fragments
  // are read two k-steps ahead and weights dequantised one ahead of the
  // MFMAs, so LDS latency and the dequantisation overlap the matrix cores;
  // each group's weight codes and scales are read one group ahead.
  auto compute = [&](auto S_, int k) __attribute__((always_inline)) {
    const bool kodd = (k & 1) != 0;
    const uint8_t* st = stage(S_);
    constexpr int NJ = JW * KG;
    constexpr int PD = 2;
    Codes bc[KG];
    uint32_t sv[KG][NSUB], bv[KG][NSUB];
    f16x8 af[PD + 1][MS], bf[2][NSUB];
    read_codes(st, IC<0>{}, bc[0], sv[0], bv[0], kodd);
    for_stages<0, (PD < NJ ? PD : NJ)>([&](auto P_) __attribute__((always_inline)) {
      constexpr int p = decltype(P_)::value;
      read_a(st, IC<p / JW>{}, IC<p % JW>{}, af[p]);
      return true;
    });
    deq(bc[0], sv[0], bv[0], IC<0>{}, bf[0]);
    for_stages<0, NJ>([&](auto S2_) __attribute__((always_inline)) {
      constexpr int s2 = decltype(S2_)::value;
      constexpr int c = s2 & 1;
      // the reads go out before this k-step's MFMAs (the scheduler would
      // otherwise sink each read to just before its use)
      if constexpr (s2 % JW == 0 && s2 / JW + 1 < KG)
        read_codes(st, IC<s2 / JW + 1>{}, bc[s2 / JW + 1], sv[s2 / JW + 1], bv[s2 / JW + 1], kodd);
      if constexpr (s2 + PD < NJ) read_a(st, IC<(s2 + PD) / JW>{}, IC<(s2 + PD) % JW>{}, af[(s2 + PD) % (PD + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (s2 + 1 < NJ) {
        constexpr int n = s2 + 1;
        deq(bc[n / JW], sv[n / JW], bv[n / JW], IC<n % JW>{}, bf[c ^ 1]);
      }
      mma(af[s2 % (PD + 1)], bf[c]);
      __builtin_amdgcn_sched_barrier(0);
      return true;
    });
  };

  // prologue: steps 0 .. NS-2 in flight
  for_stages<0, NS - 1>([&](auto S_) __attribute__((always_inline)) {
    issue(S_, decltype(S_)::value);
    __builtin_amdgcn_sched_barrier(0);  // keep each step's loads together, in step order
    return true;
  });
  const int trips = nst / NS;
  const int rem = nst - trips * NS;
  if constexpr (KS == 1) {
    // step k = NS*trip + S uses stage S
    auto step = [&](auto S_, int k) __attribute__((always_inline)) {
      constexpr int S = decltype(S_)::value;
      wait_vmcnt<(NS - 2) * C::LOADS>();  // this wave's loads of step k have landed
      __builtin_amdgcn_s_barrier();       // every wave's have; stage (S-1) is free
      issue(IC<(S + NS - 1) % NS>{}, k + NS - 1);
      __builtin_amdgcn_sched_barrier(0);  // the next step's loads go out before this step's MFMAs
      compute(S_, k);
    };
    // whole trips with no branch inside (one basic block, so no load is moved
    // away from where it is issued), then the remaining steps
    for (int t = 0; t < trips; ++t) {
      for_stages<0, NS>([&](auto S_) __attribute__((always_inline)) {
        step(S_, t * NS + decltype(S_)::value);
        return true;
      });
    }
    for_stages<0, NS - 1>([&](auto S_) __attribute__((always_inline)) {
      constexpr int S = decltype(S_)::value;
      if (S >= rem) return false;
      step(S_, trips * NS + S);
      return true;
    });
  } else {
    // Ping-pong: the two waves on a SIMD (same column block, k shares kh = 0
    // and 1) alternate between preparing a group's fragments (LDS reads,
    // dequantisation) and multiplying them, and the kh = 1 wave runs one
    // barrier behind, so while one issues MFMAs the other prepares.  Global
    // phase 2g is kh = 0 preparing group g, 2g+1 its MFMAs and kh = 1
    // preparing g, 2g+2 kh = 1's MFMAs.  A stage's loads are waited for one
    // phase before its first group is prepared, and a stage is refilled only
    // after the barrier that ends the last preparation reading it.
    f16x8 paf[JW][MS], pbf[JW][NSUB];
    auto group = [&](auto S_, auto GI_, int k) __attribute__((always_inline)) {
      constexpr int S = decltype(S_)::value, gi = decltype(GI_)::value;
      if constexpr (gi == 0) {
        issue(IC<(S + NS - 1) % NS>{}, k + NS - 1);  // into the stage of step k-1
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint8_t* st = stage(S_);
      Codes bc;
      uint32_t sv[NSUB], bv[NSUB];
      read_codes(st, GI_, bc, sv, bv, (k & 1) != 0);
      for_stages<0, JW>([&](auto J_) __attribute__((always_inline)) {
        read_a(st, GI_, J_, paf[decltype(J_)::value], true);
        return true;
      });
      for_stages<0, JW>([&](auto J_) __attribute__((always_inline)) {
        deq(bc, sv, bv, J_, pbf[decltype(J_)::value]);
        return true;
      });
      // the dequantised weights are complete here: the compiler must not sink
      // their VALU work past the barrier into the MFMA phase
#pragma unroll
      for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int ni = 0; ni < NSUB; ++ni) asm volatile("" ::"v"(pbf[jj][ni]));
      if constexpr (gi == KG - 1) wait_vmcnt<(NS - 2) * C::LOADS>();  // step k+1's loads have landed
      // this wave's reads of the stage are complete before the barrier
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      for_stages<0, JW>([&](auto J_) __attribute__((always_inline)) {
        mma(paf[decltype(J_)::value], pbf[decltype(J_)::value], true);
        return true;
      });
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    wait_vmcnt<(NS - 2) * C::LOADS>();  // step 0's loads have landed
    __builtin_amdgcn_s_barrier();
    if (kh == 1) __builtin_amdgcn_s_barrier();
    for (int t = 0; t < trips; ++t) {
      for_stages<0, NS>([&](auto S_) __attribute__((always_inline)) {
        for_stages<0, KG>([&](auto GI_) __attribute__((always_inline)) {
          group(S_, GI_, t * NS + decltype(S_)::value);
          return true;
        });
        return true;
      });
    }
    for_stages<0, NS - 1>([&](auto S_) __attribute__((always_inline)) {
      constexpr int S = decltype(S_)::value;
      if (S >= rem) return false;
      for_stages<0, KG>([&](auto GI_) __attribute__((always_inline)) {
        group(S_, GI_, trips * NS + S);
        return true;
      });
      return true;
    });
    if (kh == 0) __builtin_amdgcn_s_barrier();  // both waves pass the same number of barriers
  }
  wait_vmcnt<0>();  // no load into LDS may land after the workgroup ends

  if constexpr (KS == 2) {
    // the two waves of a column block hold partial sums over disjoint
    // k-steps: the second passes its accumulators through the stage memory
    // (4 KB per 32x32 tile and wave) and the first adds them, always in the
    // same order.  TPS tiles of all four column blocks fit in one stage.
    constexpr int TPS = C::STAGE / 16384;
    constexpr int CAP = TPS * NS;
    static_assert(TPS >= 1, "stage too small for the pair reduction");
    for_stages<0, (MS * NSUB + CAP - 1) / CAP>([&](auto R_) __attribute__((always_inline)) {
      constexpr int t_lo = decltype(R_)::value * CAP;
      __syncthreads();  // every wave is done with the stage memory (or the last round)
      if (kh == 1) {
        for_stages<t_lo, (t_lo + CAP < MS * NSUB ? t_lo + CAP : MS * NSUB)>([&](auto T_)
                                                                            __attribute__((always_inline)) {
          constexpr int t = decltype(T_)::value, u = t - t_lo;
          uint8_t* dst = stage(IC<u / TPS>{});
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[t / NSUB][t % NSUB];
            const f32x4 v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
            *(f32x4*)(dst + ((u % TPS) * 16384 + wn * 4096 + q * 1024 + lane * 16)) = v;
          }
          return true;
        });
      }
      __syncthreads();
      if (kh == 0) {
        for_stages<t_lo, (t_lo + CAP < MS * NSUB ? t_lo + CAP : MS * NSUB)>([&](auto T_)
                                                                            __attribute__((always_inline)) {
          constexpr int t = decltype(T_)::value, u = t - t_lo;
          const uint8_t* src = stage(IC<u / TPS>{});
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = *(const f32x4*)(src + ((u % TPS) * 16384 + wn * 4096 + q * 1024 + lane * 16));
            f32x16& a = acc[t / NSUB][t % NSUB];
            a[4 * q] += v.x;
            a[4 * q + 1] += v.y;
            a[4 * q + 2] += v.z;
            a[4 * q + 3] += v.w;
          }
          return true;
        });
      }
      return true;
    });
    if (kh == 1) return;
  }

  // ---- epilogue.  32x32 accumulator layout: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  // whether any token's activations were scaled (bf16 beyond 64): only then
  // are the exponents read
  const bool scaled = MODE != GEMM_ROWS_F16 && prm.tokexp && *prm.any_scaled != 0;
  // NVFP4: the tensor scales multiply the sums (fused: gate and up halves)
  if constexpr (BITS == NVF4) {
#pragma unroll
    for (int mi = 0; mi < MS; ++mi)
#pragma unroll
      for (int ni = 0; ni < NSUB; ++ni) {
        const float ts = (MODE == GEMM_FUSED_SWIGLU && ni >= HALFSUB) ? prm.w1.ts : prm.w0.ts;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= ts;
      }
  }
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) {
    if (mi * 32 >= rows) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mi * 32 + 8 * (r / 4) + 4 * hh + (r % 4);
      if (row >= rows) continue;
      const size_t orow = (size_t)(row0 + row) * prm.N;
      // the operand rows hold x * 2^-a: sums scaled back by 2^a, h staged at 2^-2a
      int ea = 0;
      if constexpr (MODE != GEMM_ROWS_F16) {
        if (scaled) ea = prm.tokexp[prm.perm[row0 + row] / prm.kcap];
      }
      if constexpr (MODE == GEMM_FUSED_SWIGLU) {
#pragma unroll
        for (int ni = 0; ni < HALFSUB; ++ni) {
          if (!valid[ni]) continue;
          acc[mi][ni][r] = ldexp_f(acc[mi][ni][r], ea);
          acc[mi][ni + HALFSUB][r] = ldexp_f(acc[mi][ni + HALFSUB][r], ea);
          const float hv = ldexp_f(swiglu(acc[mi][ni][r], acc[mi][ni + HALFSUB][r]), -2 * ea);
          const int col = col0 + 32 * ni + col_in;
          const int at = prm.perm8_out ? (col & ~7) + q4g_slot(col & 7) : col;
          ((uint16_t*)prm.out)[orow + at] = f32_to_f16_bits(hv);
        }
        if (prm.pre) {
          float* pr = prm.pre + (size_t)prm.perm[row0 + row] * 2 * prm.N;
#pragma unroll
          for (int ni = 0; ni < HALFSUB; ++ni) {
            if (!valid[ni]) continue;
            const int col = col0 + 32 * ni + col_in;
            pr[col] = acc[mi][ni][r];
            pr[prm.N + col] = acc[mi][ni + HALFSUB][r];
          }
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NSUB; ++ni) {
          if (!valid[ni]) continue;
          const int col = col0 + 32 * ni + col_in;
          if constexpr (MODE == GEMM_GATHER_F32) ((float*)prm.out)[orow + col] = ldexp_f(acc[mi][ni][r], ea);
          else ((uint16_t*)prm.out)[orow + col] = f32_to_f16_bits(acc[mi][ni][r]);
        }
      }
    }
  }
}

// One instantiation: each wave owns NSUB subtiles of 32 columns.  4-bit
// weights stage two groups per step (64-byte row segments) when K allows,
// unless the tuning knob asks for one.
template <int BITS, int MODE, int MS, int NSUB, int KS, int WPC>
static hipError_t launch_sub(GemmParams prm, hipStream_t st) {
  const int ncols = 4 * 32 * (MODE == GEMM_FUSED_SWIGLU ? NSUB / 2 : NSUB);
  prm.n_tiles = (prm.N + ncols - 1) / ncols;
  const int gm = tuning(TUNE_GEMM_GROUP_M);
  prm.group_m = gm >= 1 && gm < prm.m_tiles ? gm : prm.m_tiles;
  const int64_t total = (int64_t)prm.n_tiles * prm.m_tiles;
  prm.per_xcd = (int)((total + NUM_XCD - 1) / NUM_XCD);
  dim3 grid((unsigned)(prm.per_xcd * NUM_XCD));
  // 5-bit rows: two-group stages (80 bytes, five whole pieces; the caller
  // makes K a multiple of 128); 6-bit rows: one group (48 bytes)
  if constexpr (BITS == 5) {
    return launch_kernel(gemm_kernel<5, MODE, MS, 2, NSUB, KS, WPC>, grid, 256 * KS, 0, st, prm);
  } else {
    // two-group stages: 4-bit rows, or 8-bit rows with the whole LDS
    if constexpr ((BITS == 4 || BITS == NVF4 || (BITS == 8 && WPC == 1 && NSUB == 2 && MS < 4)) && WPC < 3) {
      if ((prm.K / 64) % 2 == 0 && tuning(TUNE_GEMM_KG) != 1)
        return launch_kernel(gemm_kernel<BITS, MODE, MS, 2, NSUB, KS, WPC>, grid, 256 * KS, 0, st, prm);
    }
    return launch_kernel(gemm_kernel<BITS, MODE, MS, 1, NSUB, KS, WPC>, grid, 256 * KS, 0, st, prm);
  }
}

// Row tiles of 64 and 128 run four waves, one per column block, or with the
// tuning knob eight, two per column block splitting each group's k-steps.
template <int BITS, int MODE, int MS>
static hipError_t launch_one(const GemmParams& prm, hipStream_t st) {
  // 5- and 6-bit codes: four waves of two subtiles; 5-bit stages (80-byte row
  // segments) leave room for one workgroup per CU, 6-bit ones for two at 32-
  // and 64-row tiles
  if constexpr (BITS == 5) {
    return launch_sub<BITS, MODE, MS, 2, 1, 1>(prm, st);
  } else if constexpr (BITS == 6) {
    if constexpr (MS < 4) return launch_sub<BITS, MODE, MS, 2, 1, 2>(prm, st);
    else return launch_sub<BITS, MODE, MS, 2, 1, 1>(prm, st);
  } else {
    // fp16 rows: two stages of four subtiles would not fit in LDS
    if constexpr (MS == 4 && BITS != 16) {
      if (tuning(TUNE_GEMM_NSUB) == 4) return launch_sub<BITS, MODE, MS, 4, 1, 1>(prm, st);
    }
    if (tuning(TUNE_GEMM_KSPLIT) == 2) return launch_sub<BITS, MODE, MS, 2, 2, 1>(prm, st);
    if constexpr (MS < 4) {
      // 8-bit weights at 32-row tiles: one workgroup per CU streaming two-group
      // (128-byte) row segments measured faster than two with one-group stages;
      // so did the fp16 down projection (three stages instead of two)
      const int wpc = tuning(TUNE_GEMM_WPC);
      // 4-bit and NVFP4 down projections at 64-row tiles: three workgroups per
      // CU (one-group stages, 40 KB of LDS each) measured 3-10% faster than two
      if constexpr (MS == 2 && (BITS == 4 || BITS == NVF4)) {
        if (wpc == 3 || (wpc != 1 && wpc != 2 && MODE == GEMM_ROWS_F16))
          return launch_sub<BITS, MODE, MS, 2, 1, 3>(prm, st);
      }
      if (wpc == 1 || (wpc != 2 && ((MS == 1 && BITS == 8) || (BITS == 16 && MODE == GEMM_ROWS_F16))))
        return launch_sub<BITS, MODE, MS, 2, 1, 1>(prm, st);
      return launch_sub<BITS, MODE, MS, 2, 1, 2>(prm, st);
    }
    return launch_sub<BITS, MODE, MS, 2, 1, 1>(prm, st);
  }
}

template <int BITS, int MODE>
static hipError_t launch_ms(int bm, const GemmParams& prm, hipStream_t st) {
  switch (bm) {
    case 32: return launch_one<BITS, MODE, 1>(prm, st);
    case 64: return launch_one<BITS, MODE, 2>(prm, st);
    case 128: return launch_one<BITS, MODE, 4>(prm, st);
    default: return hipErrorInvalidValue;
  }
}

// one weight format's launches; each format is instantiated in its own
// translation unit (gemm_w*.hip), so the formats compile in parallel
template <int BITS>
hipError_t launch_bits(GemmMode mode, int bm, const GemmParams& prm, hipStream_t st) {
  switch (mode) {
    case GEMM_FUSED_SWIGLU: return launch_ms<BITS, GEMM_FUSED_SWIGLU>(bm, prm, st);
    case GEMM_GATHER_F32: return launch_ms<BITS, GEMM_GATHER_F32>(bm, prm, st);
    case GEMM_ROWS_F16: return launch_ms<BITS, GEMM_ROWS_F16>(bm, prm, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe

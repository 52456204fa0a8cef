// Batched path, host side: the row tile choice and the launch of the grouped
// MFMA GEMM (gemm_kernel.hpp), whose weight formats are instantiated in
// gemm_w4.hip, gemm_w56.hip, gemm_w8.hip, gemm_w16.hip and gemm_wf4.hip.
#include "gemm_kernel.hpp"

namespace moe {

extern template hipError_t launch_bits<4>(GemmMode, int, const GemmParams&, hipStream_t);
extern template hipError_t launch_bits<5>(GemmMode, int, const GemmParams&, hipStream_t);
extern template hipError_t launch_bits<6>(GemmMode, int, const GemmParams&, hipStream_t);
extern template hipError_t launch_bits<8>(GemmMode, int, const GemmParams&, hipStream_t);
extern template hipError_t launch_bits<16>(GemmMode, int, const GemmParams&, hipStream_t);
extern template hipError_t launch_bits<NVF4>(GemmMode, int, const GemmParams&, hipStream_t);

int gemm_block_m(int P, int E) {
  const int forced = tuning(TUNE_GEMM_BM);
  if (forced == 32 || forced == 64 || forced == 128) return forced;
  // measured on MI355X: 32-row tiles while an average expert fits in one,
  // 64-row tiles (two workgroups per CU) beyond: with ~48 pairs per expert a
  // 32-row tiling reads every expert's weights twice (entropy-adaptive top-3
  // over 512 tokens and 32 experts: 64-row tiles 16-19% faster); 128-row
  // tiles only for very large batches, where the per-tile weight traffic
  // dominates
  const int avg = E > 0 ? P / E : P;
  if (avg <= 32) return 32;
  if (avg <= 1024) return 64;
  return 128;
}

int gemm_max_mtiles(int P, int E, int bm) { return (P + bm - 1) / bm + E; }

hipError_t launch_gemm(GemmMode mode, const uint16_t* a, int64_t a_rows, const int32_t* perm, const int32_t* counts,
                       const int32_t* offsets, int kcap, int E, int K, int N, int bits, WView w0, WView w1,
                       void* out, bool perm8_out, int bm, int max_mtiles, hipStream_t st, float* pre,
                       const int32_t* tokexp, const int32_t* any_scaled) {
  GemmParams prm;
  if (tokexp && !any_scaled) return hipErrorInvalidValue;
  prm.any_scaled = any_scaled;
  prm.pre = mode == GEMM_FUSED_SWIGLU ? pre : nullptr;
  prm.tokexp = mode != GEMM_ROWS_F16 ? tokexp : nullptr;
  prm.a = a;
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
  prm.a_bytes = (uint32_t)(a_rows * K * 2);
  prm.sb_up_delta = 0;
  // both operand views in one layout; one expert's packed codes within 32-bit offsets
  if ((w0.pq == nullptr) != (w1.pq == nullptr)) return hipErrorInvalidValue;
  if (w0.pq && (w0.pq_expert > 0xFFFFFFFFll || w1.pq_expert > 0xFFFFFFFFll)) return hipErrorInvalidValue;
  if (bits != 16) {
    if (!w0.sb || !w1.sb) return hipErrorInvalidValue;
    const int64_t delta = w1.sb - w0.sb;
    if (mode == GEMM_FUSED_SWIGLU) {
      // both halves under one descriptor: the up half after the gate half
      if (delta < 0 || delta > 0x7FFFFFFFll || w0.sb_stride != w1.sb_stride) return hipErrorInvalidValue;
      prm.sb_up_delta = (int32_t)delta;
    }
    if ((int64_t)((K / 64 + 1) / 2) * w0.sb_stride * 8 > 0xFFFFFFFFll) return hipErrorInvalidValue;
  }
  prm.perm8_out = perm8_out ? 1 : 0;
  // per-lane buffer offsets are 32-bit: the operand rows and one expert's weight rows
  // (A below 2 GB, so an offset of 2^31 is past its end)
  if (a_rows * K * 2 > 0x7FFFFFFFll || w0.stride * (int64_t)K * code_bits(bits) / 8 > 0xFFFFFFFFll)
    return hipErrorInvalidValue;
  prm.m_tiles = max_mtiles;
  if (bits == 4) return launch_bits<4>(mode, bm, prm, st);
  if (bits == NVF4) return launch_bits<NVF4>(mode, bm, prm, st);
  if (bits == 5) {
    if ((K / 64) % 2 != 0) return hipErrorInvalidValue;  // two-group stages
    return launch_bits<5>(mode, bm, prm, st);
  }
  if (bits == 6) return launch_bits<6>(mode, bm, prm, st);
  if (bits == 8) return launch_bits<8>(mode, bm, prm, st);
  return launch_bits<16>(mode, bm, prm, st);
}

}  // namespace moe

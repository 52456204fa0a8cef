// Launch functions of the layer's HIP kernels (internal; called by moe_abi.cpp).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_MAX_K_DEV 8
#define MOE_K_ENTROPY_CAP_DEV 3
#define MOE_MAX_EXPERTS_DEV 256

namespace moe {

// Width code of NVFP4 weights inside the library (4-bit E2M1 codes with E4M3
// block scales per 16 columns); code_bits gives the bits per code of a width
// code.
constexpr int NVF4 = 0x104;
__host__ __device__ constexpr int code_bits(int bits) { return bits == NVF4 ? 4 : bits; }

// Debug timing hook (moe_debug_set_events): the start/stop event pair for the
// next kernel launch on this thread, if one is pending.
bool next_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through here.  With a pending
// event pair the launch carries it (hipExtLaunchKernelGGL: the events take the
// kernel's own start/end timestamps); otherwise a plain launch.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                                Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (next_launch_events(&a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, a, b, 0, static_cast<KArgs>(args)...);
  else
    kernel<<<grid, block, lds, st>>>(static_cast<KArgs>(args)...);
  return hipGetLastError();
}


// Launch-shape knobs (resident waves per CU the decode kernels aim for).
// Defaults are the measured best; moe_debug_set_tuning overrides them.
enum TuneKey {
  TUNE_UP_WAVES_PER_CU = 0,
  TUNE_DOWN_WAVES_PER_CU = 1,
  TUNE_GEMM_GROUP_M = 2,
  TUNE_GEMM_BM = 3,  // 32, 64 or 128 forces the GEMM row tile; anything else: chosen from the batch
  TUNE_GEMM_KG = 4,  // 1: 4-bit GEMM stages one quantisation group per step (default: two when K allows)
  TUNE_GEMM_NSUB = 5,  // 4: 128-row GEMM tiles give each wave 128 columns (default 64)
  TUNE_GEMM_KSPLIT = 6,  // 2: GEMM tiles run eight waves, two per column block splitting k (default four)
  TUNE_GEMM_WPC = 7,  // 1 / 2 / 3: workgroups per CU at 32- and 64-row GEMM tiles (3: 4-bit and NVFP4 at 64 rows; other values: by bits, tile and mode)
  TUNE_UP_BALANCE = 8,  // 2: decode gate+up waves per pair from the wave target alone (default: equal iterations)
  TUNE_ROUTER_TOKENS = 9,  // 1 / 4: tokens per small-batch router workgroup at eight experts each (default 2)
  TUNE_KEYS = 10
};
int tuning(TuneKey key);

// One expert weight view: row n of expert e starts at q + (e*stride + n)*row_bytes.
// `bits` arguments below are widths 4/5/6/8/16 or NVF4 (common.hpp).
struct WView {
  const uint8_t* q;
  const uint16_t* s;  // fp16 scales [rows, K/64] (NULL for bits 16); NVF4: E4M3 bytes [rows, K/16]
  const uint16_t* b;  // fp16 biases (NULL for NVF4)
  int64_t stride;     // rows between experts
  const uint8_t* sb;  // scales and biases in the packed_sb layout (batched path)
  int64_t sb_stride;  // rows between experts in sb
  float ts = 1.0f;    // NVF4: the tensor scale, applied to the fp32 sums
  const uint8_t* pq = nullptr;  // codes in the packed_q layout (batched path), or NULL
  int64_t pq_expert = 0;        // bytes between experts in pq
};

// ---------------------------------------------------------------- router
// health (fp32 [E], or NULL): logits[t, e] - alpha * health[e] are stored
hipError_t launch_router_logits(const void* x, const void* wr, float* logits, int T, int H, int E, int act,
                                const float* health, float alpha, hipStream_t st);
// least-used expert and population standard deviation of E counts
hipError_t launch_load_stats(const int32_t* counts, int E, int32_t* least_used, float* stddev, hipStream_t st);
// k > 0: static top-k; k <= 0: entropy-adaptive, kcap = 3 (scratch: T
// floats, or NULL for the single-workgroup pass); gs experts per group
// clear_word (optional): a device word set to 0 before the selection's
// consumers run (the batched path's flag of scaled bf16 tokens)
hipError_t launch_topk(const float* logits, int T, int E, int k, int gs, int32_t* idx, float* w, int32_t* k_used,
                       float* entropy, float* scratch, hipStream_t st, int32_t* clear_word = nullptr);

// ------------------------------------------------------------------ sort
// k_used_dev may be NULL (then k_static is used); capacity > 0 lists only the
// first `capacity` pairs of every expert (the rest get pos -1)
hipError_t launch_sort_pairs(const int32_t* idx, int T, int kcap, const int32_t* k_used_dev, int k_static, int E,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t st,
                             int capacity = 0);
// the same sort, and in the same launch the batched GEMM's operand: x as fp16
// (x * 2^-a_t for bf16, which also writes a_t to tokexp[t] and sets
// *any_scaled to 1 when some a_t > 0; it must be 0 before)
hipError_t launch_sort_prep(const int32_t* idx, int T, int kcap, const int32_t* k_used_dev, int k_static, int E,
                            int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos, hipStream_t st,
                            int capacity, const void* x, int act, uint16_t* a, int H, bool perm8, int32_t* tokexp,
                            int32_t* any_scaled);

// ------------------------------------------------- decode (grouped GEMV)
// chunks of 16 bytes per lane needed for a row of K weights
int gemv_lanes_chunks(int K, int bits);
// Where a decode kernel gets its routing: with `logits` set (static k) it
// selects the experts itself and writes idx/wts/k_used/entropy (from the
// gate+up kernel); with `logits` NULL it reads idx, wts and *k_used.
struct GemvRoute {
  const float* logits;
  int E;
  int32_t* idx;
  float* wts;
  int32_t* k_used;
  float* entropy;
  int gs = 1;  // experts per selection group (1: plain top-k)
};
// fused=true: h[p, j] = fp16(2^-2a_t swiglu(gate_j . x, up_j . x)) for j < I,
// and with pre set also pre[p, j] = gate_j . x, pre[p, N + j] = up_j . x (fp32)
// fused=false: out32[p, n] = w0_n . x for n < N
// bf16 activations: a_t as in common.hpp, written to tokexp[t] (if set); 0 for fp16
hipError_t launch_gemv_up(const void* x, int act, const GemvRoute& route, int k_static, int kcap, int T, int H,
                          int N, int bits, bool fused, WView w0, WView w1, uint16_t* h, float* out32, int num_cu,
                          hipStream_t st, float* pre = nullptr, int32_t* tokexp = nullptr);
// whether the decode down kernels take rows of I weights of `bits` bits with
// kcap slots per token
bool gemv_down_fits(int I, int bits, int kcap);
// y[t, m] = act(sum_s w[t,s] * (Wd[e_s, m, :] . h[t*kcap+s, :]));
// capacity > 0: a pair beyond the first `capacity` pairs of its expert (pair
// order) is left out of y (needs route.logits NULL: the selection is read)
// tokexp (NULL: all 0): h rows staged at 2^-2a_t, y scaled back by 2^2a_t
hipError_t launch_gemv_down(const uint16_t* h, const GemvRoute& route, int k_static, int kcap, int T, int H, int I,
                            int bits, WView wd, void* y, int act, int num_cu, hipStream_t st, int capacity = 0,
                            const int32_t* tokexp = nullptr);
// whether the router uses one workgroup per (expert, token) logit rather
// than the 32 x 32 tiled matrix-core kernel
bool router_use_small(int T, int E);

// -------------------------------------------------- batched (MFMA GEMM)
enum GemmMode { GEMM_FUSED_SWIGLU = 0, GEMM_GATHER_F32 = 1, GEMM_ROWS_F16 = 2 };
// rows of one M tile for a dispatch (32, 64 or 128)
int gemm_block_m(int P, int E);
// upper bound on M tiles for P pairs over E experts
int gemm_max_mtiles(int P, int E, int bm);
// a: fp16 rows, 8-element blocks in the weights' unpack order (sort_prep / the
// fused epilogue); GATHER modes read a[perm[row]/kcap], ROWS mode a[row];
// K = reduction dim.  FUSED: out = h fp16 [rows, N=I] (blocks in 4-bit unpack
// order if perm8_out); GATHER_F32: out fp32 [rows, N]; ROWS_F16: out fp16
// a_rows: rows of a (T or P); a and one expert's weight rows must each stay
// below 4 GB (32-bit buffer offsets), else hipErrorInvalidValue
// FUSED with pre set: also the fp32 gate and up sums of pair perm[row] at
// pre[pair, col] and pre[pair, N + col].  tokexp (GATHER modes; NULL: all 0):
// the operand rows hold x * 2^-a_t, so the sums are scaled back by 2^a_t and
// h is stored at 2^-2a_t; read only when *any_scaled is nonzero
hipError_t launch_gemm(GemmMode mode, const uint16_t* a, int64_t a_rows, const int32_t* perm, const int32_t* counts,
                       const int32_t* offsets, int kcap, int E, int K, int N, int bits, WView w0, WView w1,
                       void* out, bool perm8_out, int bm, int max_mtiles, hipStream_t st, float* pre = nullptr,
                       const int32_t* tokexp = nullptr, const int32_t* any_scaled = nullptr);

// --------------------------------------------------------- small kernels
// h[i, j] = fp16(2^-2a swiglu(g[i, j], u[i, j])) for i < rows, a the
// exponent of row i's token: tokexp[pair / kcap], pair = perm ? perm[i] : i
// (tokexp NULL: a = 0)
hipError_t launch_swiglu(const float* g, const float* u, uint16_t* h, int64_t rows, int I, bool perm8,
                         hipStream_t st, const int32_t* tokexp = nullptr, const int32_t* perm = nullptr,
                         int kcap = 1);
// y[t] = act(2^2a_t sum_{s<k} w[t,s] * o[pos[t*kcap+s]]) (tokexp NULL: a_t = 0)
hipError_t launch_combine(const uint16_t* o, const int32_t* pos, const float* wts, const int32_t* k_used_dev,
                          int k_static, int kcap, int T, int H, void* y, int act, hipStream_t st,
                          const int32_t* tokexp = nullptr);
// out[p, :] = src[r, :] (fp16 rows of width I) with r = pos[p] for pos[p] >= 0,
// or, when pos is NULL, r = p for the pairs whose slot p % kcap < k_used
hipError_t launch_gather_rows(const uint16_t* src, const int32_t* pos, int64_t P, int I, uint16_t* out, int kcap,
                              const int32_t* k_used_dev, int k_static, bool perm8, hipStream_t st);
// pre[p, 0:I] = g[r, :], pre[p, I:2I] = u[r, :] (fp32 rows) with r chosen
// as in launch_gather_rows
hipError_t launch_gather_preact(const float* g, const float* u, const int32_t* pos, int64_t P, int I, float* pre,
                                int kcap, const int32_t* k_used_dev, int k_static, hipStream_t st);
// copy n int32/fp32 words
hipError_t launch_copy_words(const void* src, void* dst, int64_t n, hipStream_t st);
// streaming read of `bytes` (multiple of 16, < 4 GiB) at src, a contiguous
// segment per workgroup; sink[w] = XOR of the words wave w read (2048
// workgroups of 256 threads: 8192 waves)
hipError_t launch_stream_read(const void* src, uint32_t bytes, uint32_t* sink, hipStream_t st);
// scales/biases of rows [0, N) of E experts -> packed_sb layout (see moe.h);
// nvfp4: s holds E4M3 block-scale bytes [rows, K/16] and b is unused
hipError_t launch_pack_sb(const uint16_t* s, const uint16_t* b, int E, int N, int K, int64_t src_stride, uint8_t* dst,
                          int64_t dst_stride, int64_t dst_row0, hipStream_t st, bool nvfp4 = false);
inline int64_t packed_sb_bytes(int E, int64_t stride, int K) { return (int64_t)E * ((K / 64 + 1) / 2) * stride * 8; }
// packed_q: a unit is the groups one pipeline step of the batched GEMM reads
// (two for 4-, 5- and 8-bit codes and NVFP4, one for 6-bit codes and fp16);
// bytes of one row's unit, units per row, and bytes of one expert
inline int packed_q_unit_groups(int bits) { return bits == 6 || bits == 16 ? 1 : 2; }
inline int64_t packed_q_unit_bytes(int bits) { return 8 * (int64_t)code_bits(bits) * packed_q_unit_groups(bits); }
inline int64_t packed_q_units(int K, int bits) {
  const int u = 64 * packed_q_unit_groups(bits);
  return (K + u - 1) / u;
}
inline int64_t packed_q_expert_bytes(int64_t stride, int K, int bits) {
  return (stride + 31) / 32 * packed_q_units(K, bits) * 32 * packed_q_unit_bytes(bits);
}
// codes of rows [0, N) of E experts (row-major, src_stride rows apart) ->
// packed_q layout with dst_stride rows per expert (N, strides multiples of 32)
hipError_t launch_pack_q(const uint8_t* q, int E, int N, int K, int bits, int64_t src_stride, uint8_t* dst,
                         int64_t dst_stride, hipStream_t st);

}  // namespace moe

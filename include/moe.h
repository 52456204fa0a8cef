/*
 * moe.h — C ABI of one sparse Mixture-of-Experts FFN layer on AMD Instinct
 * MI355X (gfx950).
 *
 * The layer, in the order it runs:
 *   1. router projection  logits[t, e] = sum_h x[t, h] * Wr[e, h]   (fp32 accumulation)
 *   2. selection          the k largest logits per token, larger logit first and
 *                         the lower expert index first among equal logits; the
 *                         weights are the softmax probabilities of the selected
 *                         experts renormalised to sum to one
 *                         (page "Qwen3.5 Block在llama.cpp中的映射与优化原理",
 *                         section 4.1: linear -> softmax -> top-k)
 *      or the entropy-adaptive variant: k = 1, 2 or 3 from the mean Shannon
 *                         entropy H (nats) of the call's routing distributions,
 *                         k = 1 if H < 1.2, 2 if 1.2 <= H < 2.5, else 3
 *                         (page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析",
 *                         section 2.2, Entropy-Aware Routing)
 *   3. token->expert sort  (token, slot) pairs grouped by expert, stable
 *   4. gate+up projection  over affine group-quantised weights, w = scale*q + bias,
 *                         gate and up concatenated along the output axis
 *                         [E, 2*inter, hidden], gate rows first
 *                         (oMLX gate/up fusion page, "融合原理" and steps 3-4)
 *   5. SwiGLU              h = silu(g) * u,  silu(g) = g / (1 + exp(-g))
 *   6. down projection     o = W_down . h
 *   7. combine             y[t] = sum over slots s of w[t, s] * o[t, s], in slot
 *                         order, rounded to the activation dtype (page
 *                         "Qwen3.5 Block…", section 4.2, the weighted sum after
 *                         the expert FFN)
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer unless stated otherwise.  The caller
 *     owns and allocates every buffer, including the workspace.  The library
 *     never allocates or frees device memory and never synchronises: work is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs
 *     asynchronously.  Faults during execution surface at the caller's next
 *     synchronisation, as with any asynchronous library.
 *   - Arguments are validated completely on the host before anything is
 *     enqueued; an error return means nothing was enqueued.  Validation makes
 *     no HIP call, so it can be exercised without a GPU.
 *   - Layouts are row-major.  Activations and router weights share one dtype.
 *   - Arithmetic: the expert projections run on fp16 operands (dequantised
 *     weights, activations, SwiGLU rows) with fp32 accumulation; routing and
 *     the combine are fp32.  bf16 activations keep bf16's range: token t is
 *     converted as x * 2^-a_t, a_t >= 0 the smallest exponent with
 *     max|x_t| * 2^-a_t < 64 (exact while the scaled values stay in fp16's
 *     normal range; a_t = 0 whenever max|x_t| < 64), its gate and up sums
 *     are scaled back by 2^a_t, its SwiGLU rows and down outputs are staged
 *     at 2^-2a_t and y is scaled back by 2^2a_t.  Only values beyond the
 *     output dtype's range become infinite.
 *   - T == 0 is a no-op returning MOE_OK; buffers whose size is proportional
 *     to T (activations, outputs, routing results) may then be NULL.
 *   - Calls on different streams are independent; the library keeps no
 *     mutable state besides a once-per-device cache of device properties and
 *     the optional per-thread profiling hooks at the end of this header.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,         /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,        /* a size is out of range or inconsistent */
  MOE_ERR_DTYPE = -3,        /* unknown activation dtype */
  MOE_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned */
  MOE_ERR_K = -5,            /* k out of range */
  MOE_ERR_QUANT = -6,        /* unsupported bits / group size / scale presence */
  MOE_ERR_INCOMPATIBLE = -7, /* gate and up cannot be fused (different bits, group
                                size, shape or scale presence); keep them separate */
  MOE_ERR_WORKSPACE = -8,    /* workspace NULL or smaller than required */
  MOE_ERR_DEVICE = -9,       /* no usable gfx950 device is current */
  MOE_ERR_HIP = -10,         /* a HIP launch or query failed */
  MOE_ERR_INTERNAL = -11,    /* unexpected internal error */
  MOE_ERR_OPTION = -12,      /* a routing option is out of range (moe_route_opts) */
  MOE_ERR_SCRATCH = -13      /* moe_layer_forward_noalloc: the call needs more than
                                MOE_NOALLOC_SCRATCH_BYTES of workspace */
} moe_status;

typedef enum { MOE_F16 = 1, MOE_BF16 = 2 } moe_dtype;

/* k argument value selecting the entropy-adaptive top-1/2/3 routing */
#define MOE_K_ENTROPY (-1)
/* slots kept per token in entropy-adaptive mode */
#define MOE_K_ENTROPY_CAP 3
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_K 8

/*
 * One expert weight tensor, logically [E, N, K]: N output rows per expert,
 * K input columns.  Row n of expert e starts at row index e*expert_stride_rows + n
 * (expert_stride_rows == N for a dense tensor; 2*inter for the gate or up half
 * of a fused gate_up tensor, with `q`/`scales`/`biases` pointing at its first row).
 *
 *   bits == 4:  q      uint8 [rows, K/2], two codes per byte, the even column
 *                      in the low nibble; codes are unsigned 0..15
 *   bits == 5:  q      uint8 [rows, 5K/8], code k at bits 5k .. 5k+4 of the row
 *                      read as a little-endian bit stream (eight codes per five
 *                      bytes); codes 0..31
 *   bits == 6:  q      uint8 [rows, 3K/4], code k at bits 6k .. 6k+5 of the row
 *                      read as a little-endian bit stream (four codes per three
 *                      bytes); codes 0..63
 *               5 and 6 bits (a reading: the oMLX page names these modes
 *                      but gives no layout): both paths.  On the batched
 *                      path 5-bit weights need hidden and inter multiples of
 *                      128 (MOE_ERR_QUANT otherwise)
 *   bits == 8:  q      uint8 [rows, K], codes 0..255
 *   bits 4-8:   scales fp16 [rows, K/group_size], biases fp16 [rows, K/group_size];
 *               w[n, k] = scales[n, k/gs] * q[n, k] + biases[n, k/gs]
 *               (affine group quantisation, one scale/bias per row and group)
 *   bits == 16: q      fp16 [rows, K] weights; scales and biases must be NULL
 *
 * group_size must be 64.  K must be a multiple of 64.  q, scales and biases
 * must be 16-byte aligned.
 *
 * format == MOE_FMT_NVFP4 (a reading: the oMLX page names an nvfp4 weight
 * mode, "如何验证正确性", with no layout; this is NVIDIA's published NVFP4):
 *   bits 4, group_size 16, biases NULL, both paths.
 *               q      uint8 [rows, K/2], two E2M1 codes per byte, the even
 *                      column in the low nibble; code bit 3 is the sign,
 *                      codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6
 *               scales uint8 [rows, K/16], one FP8 E4M3 (OCP "fn": bias 7,
 *                      448 largest, 0x7F/0xFF NaN) block scale per 16 columns
 *               tensor_scale  fp32, one per tensor (finite, > 0)
 *               w[n, k] = tensor_scale * e4m3(scales[n, k/16]) * e2m1(q[n, k])
 *   The kernels form e2m1 * e4m3 exactly in fp16 and apply tensor_scale to
 *   the fp32 sums.  A fused gate_up tensor has one tensor_scale; separate
 *   gate and up tensors may differ.
 * format == MOE_FMT_AFFINE (0): the forms above; tensor_scale is ignored.
 *
 * packed_sb (optional, bits 4 to 8): the same scales and biases repacked for
 * the batched path by moe_pack_sb, pointing at the tensor's (or view's) first
 * row like q.  Layout: for expert e, group pair p (groups 2p and 2p+1; a
 * missing last group is 0) and row n, 8 bytes {scale[2p], scale[2p+1],
 * bias[2p], bias[2p+1]} (fp16) at byte ((e*NP + p)*expert_stride_rows + n)*8,
 * NP = ceil(K/128).  One step of the batched GEMM then reads a column block's
 * scales and biases as a few contiguous 128-byte lines instead of one line
 * per column.  NULL: the batched path repacks them into the workspace on every
 * call.  The gate and up views of a fused tensor share its packed_sb (the up
 * view's pointer is the gate view's plus inter*8 bytes).  Set for fp16
 * weights, it is refused with MOE_ERR_QUANT.  NVFP4 weights use the same
 * 8-byte slots for {the four E4M3 block scales of group 2p, those of group
 * 2p+1} (two little-endian 32-bit words, block 4g+i in byte i).
 */
/*
 * packed_q (optional, any format): the same codes (or fp16 weights) repacked
 * for the batched path by moe_pack_q, pointing at the tensor's (or view's)
 * first 32-row block like q.  A unit is U groups of 64 columns: U = 2 for
 * 4-, 5- and 8-bit codes and NVFP4, U = 1 for 6-bit codes and fp16 weights.
 * Layout: for expert e, 32-row block j (rows 32j .. 32j+31; NB =
 * ceil(expert_stride_rows / 32) blocks per expert), unit p (NU =
 * ceil(K / (64 U)) units, a missing last group zero) and row r of the
 * block, the row's PB bytes of the unit (PB = 8 * U * bits per code: 64,
 * 80, 48, 128, 128; NVFP4 64) at byte (((e*NB + j)*NU + p)*32 + r)*PB.  A
 * pipeline step of the batched GEMM then streams each 32-row block's next
 * 32*PB bytes contiguously instead of PB bytes of 32 rows K*bits/8 bytes
 * apart (a DRAM-friendlier pattern: 6.3 TB/s against 4.5 TB/s for the same
 * loads in a probe).  It is a second copy of the codes; q stays required
 * (the decode path reads q).  The up view of a fused tensor starts
 * (inter/32)*NU*32*PB bytes after the gate view.  Needs N and
 * expert_stride_rows multiples of 32.
 */
typedef enum { MOE_FMT_AFFINE = 0, MOE_FMT_NVFP4 = 1 } moe_weight_format;

typedef struct {
  const void* q;
  const void* scales;
  const void* biases;
  int32_t E;
  int32_t N;
  int32_t K;
  int32_t bits;
  int32_t group_size;
  int64_t expert_stride_rows;
  const void* packed_sb;
  int32_t format;      /* moe_weight_format */
  float tensor_scale;  /* NVFP4 only */
  const void* packed_q;  /* optional, see above */
} moe_weights;

/*
 * Optional copies of intermediates (each pointer may be NULL).  They only copy;
 * they never change results.  kcap = k, or MOE_K_ENTROPY_CAP in entropy mode.
 *   logits     fp32  [T, E]         router logits
 *   topk_idx   int32 [T, kcap]      selected experts (slots >= k_used hold -1)
 *   topk_w     fp32  [T, kcap]      routing weights (slots >= k_used hold 0)
 *   k_used     int32 [1]            k actually used
 *   entropy    fp32  [1]            batch entropy (entropy mode; 0 otherwise)
 *   counts     int32 [E]            pairs routed to each expert
 *   offsets    int32 [E+1]          exclusive prefix sum of counts
 *   perm       int32 [T*kcap]       pair ids t*kcap+s grouped by expert, ascending
 *                                   within an expert; entries past the last pair -1
 *   h          fp16  [T*kcap, inter] SwiGLU output of pair t*kcap+s (unused slots
 *                                   untouched), times 2^-2a_t for bf16
 *                                   activations (see Arithmetic above)
 *   gate_up_preact fp32 [T*kcap, 2*inter] the gate+up projection of pair
 *                                   t*kcap+s before SwiGLU: g in columns
 *                                   [0, inter), u in [inter, 2*inter), the
 *                                   fp32 sums the SwiGLU reads (oMLX gate/up
 *                                   page, "how correctness is verified": the
 *                                   fused output equals the separate
 *                                   projections bit for bit).  Unused slots
 *                                   untouched; rows of pairs a capacity drops
 *                                   are unspecified.  Written by the kernels
 *                                   that form g and u, so it costs HBM
 *                                   writes: a debug tap
 */
typedef struct {
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* k_used;
  float* entropy;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  void* h;
  float* gate_up_preact;
} moe_taps;

/*
 * Routing options of the *_ex entry points (NULL: none of them).
 *
 *   health   fp32 [E] on the device, or NULL.  The logits that every later
 *            routing step uses (entropy, selection, weights, the logits tap)
 *            are logits[t, e] - alpha * health[e], the product and the
 *            difference each rounded to fp32: the load-aware correction of
 *            page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section 3.3, where
 *            an auxiliary head supplies a per-expert load index H and a scale
 *            alpha.  The library only applies it; health holds whatever load
 *            index the caller keeps (e.g. activation frequencies).  4-byte
 *            aligned.
 *   alpha    the scale of the correction (ignored when health is NULL).
 *   groups   0 or 1: plain top-k.  G > 1: the E experts form G groups of E/G
 *            consecutive experts and at most one expert per group is chosen:
 *            the best expert of each group, and of those the k best, in key
 *            order (page "Qwen3.5 Block在llama.cpp中的映射与优化原理", section
 *            1.1: 64 experts in 4 groups of 16, the best of each group, so
 *            4 chosen).  Needs E % G == 0 and k <= G (with MOE_K_ENTROPY:
 *            G >= 3).  The weights stay the softmax over all E experts,
 *            renormalised over the chosen ones.
 *   capacity 0: no limit.  C > 0 (moe_layer_forward_ex only): at most C
 *            (token, slot) pairs per expert, the first C in pair order
 *            t*kcap+s; the others are dropped and add nothing to y (their
 *            routing weight is not handed to the other slots).  Page
 *            "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section 5.2: a per-
 *            expert token capacity (expert_capacity).  The topk taps keep
 *            the routing; counts/offsets/perm list the kept pairs only; the
 *            h rows of dropped pairs are unspecified.
 * MOE_ERR_OPTION: groups < 0, E % groups != 0, k too large for the groups,
 * capacity < 0, capacity given to moe_route_ex / moe_topk_from_logits_ex,
 * or (moe_topk_from_logits_ex) health given.  MOE_ERR_ALIGN: health not
 * 4-byte aligned.
 */
typedef struct {
  const float* health;
  float alpha;
  int32_t groups;
  int32_t capacity;
} moe_route_opts;

/* flags of moe_layer_forward */
#define MOE_FLAG_UNFUSED 0x1u    /* separate gate and up projections, then SwiGLU
                                    (a fused tensor is split into two views);
                                    results are bit-identical to the fused path */
#define MOE_FLAG_FORCE_GEMV 0x2u /* decode path (grouped GEMV) where it applies */
#define MOE_FLAG_FORCE_MFMA 0x4u /* batched path (sorted MFMA grouped GEMM) */

/*
 * Router: logits, then top-k selection and renormalised softmax weights.
 *   x         [T, H] activations (dt); router_w [E, H] (dt)
 *   k         1..min(E, 8), or MOE_K_ENTROPY (needs E >= 3; kcap = 3)
 *   topk_idx  int32 [T, kcap] out; topk_w fp32 [T, kcap] out
 *   k_used    int32 [1] out (may be NULL); entropy fp32 [1] out (may be NULL)
 *   logits_out fp32 [T, E] out (may be NULL)
 *   ws        workspace of at least moe_route_workspace_size(T, E, k) bytes
 *             (may be NULL when logits_out is given; with MOE_K_ENTROPY the
 *             per-token entropies then go through a single-workgroup pass)
 * H % 64 == 0, 1 <= E <= 256.  T == 0 is a no-op returning MOE_OK.
 */
size_t moe_route_workspace_size(int32_t T, int32_t E, int32_t k);
moe_status moe_route(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E, int32_t k,
                     int32_t* topk_idx, float* topk_w, int32_t* k_used, float* entropy, float* logits_out, void* ws,
                     size_t ws_bytes, void* stream);
/* moe_route with routing options (opts may be NULL; see moe_route_opts). */
moe_status moe_route_ex(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E,
                        int32_t k, const moe_route_opts* opts, int32_t* topk_idx, float* topk_w, int32_t* k_used,
                        float* entropy, float* logits_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Selection only, from caller-provided fp32 logits [T, E] (same rules and
 * outputs as moe_route).  Lets two callers that hold identical logits check
 * that they select identical experts.
 */
moe_status moe_topk_from_logits(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                                float* topk_w, int32_t* k_used, float* entropy, void* ws, size_t ws_bytes,
                                void* stream);
/* Selection with routing options; the logits are taken as final, so
 * opts->health must be NULL (MOE_ERR_OPTION otherwise). */
moe_status moe_topk_from_logits_ex(const float* logits, int32_t T, int32_t E, int32_t k, const moe_route_opts* opts,
                                   int32_t* topk_idx, float* topk_w, int32_t* k_used, float* entropy, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * The whole layer.
 *   x         [T, H] activations (dt); router_w [E, H] (dt); y [T, H] out (dt)
 *   gate_up   fused tensor, N = 2*inter, K = H (gate rows first), or NULL to use
 *             `gate` and `up` (each N = inter, K = H).  With gate_up given,
 *             gate/up are ignored.
 *   down      N = H, K = inter
 *   flags     MOE_FLAG_*; taps may be NULL
 *   ws        workspace of at least moe_layer_workspace_size(...) bytes, 256-byte
 *             aligned
 * Limits: H % 64 == 0, inter % 64 == 0, 1 <= E <= 256, k as for moe_route, all
 * weight tensors with the same bits and E.  T == 0 is a no-op.
 * Returns MOE_ERR_INCOMPATIBLE when separate gate/up tensors differ in bits,
 * shape or scale presence.
 */
size_t moe_layer_workspace_size(int32_t T, int32_t H, int32_t E, int32_t k, int32_t inter, uint32_t flags);
moe_status moe_layer_forward(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E,
                             int32_t k, const moe_weights* gate_up, const moe_weights* gate, const moe_weights* up,
                             const moe_weights* down, void* y, uint32_t flags, const moe_taps* taps, void* ws,
                             size_t ws_bytes, void* stream);
/* moe_layer_forward with routing options (opts may be NULL; see
 * moe_route_opts); same workspace size. */
moe_status moe_layer_forward_ex(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w, int32_t E,
                                int32_t k, const moe_route_opts* opts, const moe_weights* gate_up,
                                const moe_weights* gate, const moe_weights* up, const moe_weights* down, void* y,
                                uint32_t flags, const moe_taps* taps, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward_ex without a workspace argument and without allocating:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends; the call makes
 * no hipMalloc, hipFree or other allocating call.  The caller still passes
 * inputs, outputs and taps.  A call needing more workspace than the array
 * (the layout of moe_layer_workspace_size, without the batched path's
 * regions on the decode path and without the scale repacks when the
 * weights carry packed_sb) returns MOE_ERR_SCRATCH with nothing enqueued:
 * decode and batched decode fit; a 4096-token prefill does not.
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents (the layer needs none of it cleared): calls that
 * overlap on one GPU (two streams, two threads) race and must be
 * serialised by the caller.  Results are bit-identical to
 * moe_layer_forward_ex with a caller workspace.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const void* x, moe_dtype dt, int32_t T, int32_t H, const void* router_w,
                                     int32_t E, int32_t k, const moe_route_opts* opts, const moe_weights* gate_up,
                                     const moe_weights* gate, const moe_weights* up, const moe_weights* down,
                                     void* y, uint32_t flags, const moe_taps* taps, void* stream);

/*
 * Health figures of per-expert activation counts (page "Qwen3.5-MoE与Qwen3-MoE
 * 架构差异深度解析", closing advice on monitoring: the least-activated expert
 * and the standard deviation of the activation counts), e.g. of the counts
 * tap of moe_layer_forward or of counts the caller accumulates over a window.
 *   counts      int32 [E] on the device, each >= 0
 *   least_used  int32 [1] out: the lowest expert index among the smallest counts
 *   stddev      fp32 [1] out: sqrt(sum_e (counts[e] - mean)^2 / E) (population)
 * 1 <= E <= 256.  Enqueued on `stream`.
 */
moe_status moe_expert_load_stats(const int32_t* counts, int32_t E, int32_t* least_used, float* stddev,
                                 void* stream);

/*
 * Pack separate gate [E, inter, K] and up [E, inter, K] into a fused tensor
 * [E, 2*inter, K], gate rows first, for weights, scales and biases alike
 * (oMLX page, step 3).  q_out/s_out/b_out are caller-owned with the fused
 * sizes (s_out/b_out NULL when bits == 16).  The caller may free the sources
 * afterwards, so resident bytes never double.  Returns MOE_ERR_INCOMPATIBLE
 * (and enqueues nothing) when the two tensors cannot be fused: different
 * bits, group size, shape or scale presence (oMLX page, step 2).
 */
moe_status moe_fuse_gate_up(const moe_weights* gate, const moe_weights* up, void* q_out, void* s_out, void* b_out,
                            void* stream);

/*
 * Bytes of packed_sb for a tensor of E experts, expert_stride_rows rows per
 * expert and K input columns: E * ceil(K/128) * expert_stride_rows * 8.
 */
size_t moe_packed_sb_bytes(int32_t E, int64_t expert_stride_rows, int32_t K);
/*
 * Write w's scales and biases in the packed_sb layout (see moe_weights) to
 * out (caller-owned, moe_packed_sb_bytes, 16-byte aligned), rows [0, N) of
 * every expert at w->expert_stride_rows rows per expert.  Enqueued on
 * `stream`.  MOE_ERR_QUANT for bits 16 (no scales).
 */
moe_status moe_pack_sb(const moe_weights* w, void* out, void* stream);

/*
 * Bytes of packed_q for a tensor of E experts, expert_stride_rows rows per
 * expert (a multiple of 32), K input columns and the given width code
 * (bits 4, 5, 6, 8 or 16; NVFP4: 4): E * (rows/32) * NU * 32 * PB (see
 * moe_weights).  0 for arguments out of range.
 */
size_t moe_packed_q_bytes(int32_t E, int64_t expert_stride_rows, int32_t K, int32_t bits);
/*
 * Write w's codes in the packed_q layout (see moe_weights) to out
 * (caller-owned, moe_packed_q_bytes, 16-byte aligned): rows [0, N) of every
 * expert at w->expert_stride_rows rows per expert; rows of a block past N
 * and a missing last group are zero.  Enqueued on `stream`.  MOE_ERR_SHAPE
 * when N or expert_stride_rows is not a multiple of 32.
 */
moe_status moe_pack_q(const moe_weights* w, void* out, void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/*
 * Profiling hooks (per calling thread).  When `events` is non-NULL, the i-th
 * kernel of every later entry point on this thread is launched with
 * hipExtLaunchKernelGGL, which stamps events[2i] when the kernel starts and
 * events[2i+1] when it ends (the kernel's own dispatch timestamps, no extra
 * packets in the stream), for 2i + 1 < n.  `events` are caller-created
 * hipEvent_t handles, owned by the caller.  Pass NULL to stop.
 * moe_debug_last_plan writes the names of the kernels the last call on this
 * thread launched, comma-separated, into buf (host memory).
 */
void moe_debug_set_events(void* const* events, int32_t n);
int32_t moe_debug_last_plan(char* buf, size_t buf_bytes);
/*
 * Launch-shape knobs for measurement sweeps (process-wide): key 0 = resident
 * waves per CU targeted by the decode gate+up kernel (1.5 times that for
 * 4- and 5-bit codes with hidden <= 6144, whose kernels fit three or more
 * waves per SIMD), key 1 = by the decode
 * down kernel, key 2 = row tiles per group in the batched GEMM's tile order,
 * key 3 = the batched GEMM's row tile (32, 64 or 128; other values: chosen
 * from the batch), key 4 = K groups of 64 per pipeline stage (1; other
 * values: 2 where the stage fits in LDS), key 5 = 32-column subtiles per wave
 * at the 128-row tile (4; other values: 2), key 6 = waves per column block
 * (2, splitting each group's k-steps; other values: 1), key 7 = workgroups
 * per CU at the 32- and 64-row tiles (1: the whole LDS for one, deeper
 * pipeline and two-group 8-bit stages; 2: two; 3: three, for 4-bit and NVFP4
 * weights at 64-row tiles; other values: one for 8-bit weights at 32-row
 * tiles and for fp16 down projections, three for 4-bit and NVFP4 down
 * projections at 64-row tiles, else two), key 8 = waves per
 * (token, slot) pair of the decode gate+up kernel (2: from the resident-wave
 * target alone; other values: as many as give every wave the same number of
 * row iterations, at most that target), key 9 = tokens per workgroup of the
 * small-batch router where it takes eight experts per workgroup (1 or 4;
 * other values: 2).
 * Values <= 0 are ignored.  Key 6 changes the order of the fp32 sums
 * (results within the layer tolerance of the default); the other keys do not
 * change results.
 */
void moe_debug_set_tuning(int32_t key, int32_t value);

/*
 * Measurement reference: a plain streaming read of `bytes` bytes at `src`
 * (device memory, 16-byte aligned, bytes a multiple of 16 and below 4 GiB)
 * (16-byte non-temporal buffer loads as in the decode kernels, four per
 * lane in flight, each of 2048 workgroups of four waves streaming its own
 * contiguous segment).  It bounds what a weight-streaming kernel can reach
 * on this device.  Each wave writes the XOR of the 32-bit words it read to
 * sink[wave] (device memory, MOE_STREAM_READ_WAVES words; every word of src
 * is read exactly once, so the XOR of the sink equals the XOR of src).
 * Errors: MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_SHAPE (bytes), MOE_ERR_DEVICE.
 */
#define MOE_STREAM_READ_WAVES 8192
moe_status moe_debug_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */

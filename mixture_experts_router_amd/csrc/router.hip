// Router: logits GEMV, top-k selection with renormalised softmax weights, and
// the entropy-adaptive top-1/2/3 variant.
//
// logits[t, e] = sum_h x[t, h] * Wr[e, h], fp32 accumulation (page "Qwen3.5
// Block在llama.cpp中的映射与优化原理", section 4.1: the router is one linear
// layer followed by softmax and top-k).  Selection is made on logits with the
// key (larger logit, lower index); see topk.hpp.  Entropy-adaptive k (page
// "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section 2.2): mean over the call's
// tokens of the Shannon entropy (nats) of the routing distribution; k = 1 if
// H < 1.2, 2 if H < 2.5, else 3.
//
// Products of two fp16 (or two bf16) values are exact in fp32, so fmaf here
// rounds exactly like a separate multiply and add.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {

__device__ __forceinline__ void unpack8(u32x4 r, int act, float* v) {
  const uint32_t w4[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = act_to_f32(w4[i] & 0xFFFFu, act);
    v[2 * i + 1] = act_to_f32(w4[i] >> 16, act);
  }
}

// --------------------------------------------------------- small batches --
//
// One workgroup per TB tokens and EB consecutive experts; its four waves
// take consecutive quarters of H, each lane sums its 8-element slices in
// order (a slice of each token row is loaded once and used for all EB
// experts, a slice of each router row for all TB tokens), the wave sums its
// lanes, and the four wave partials are added in wave order, so every EB and
// TB gives the same bits.  EB = 1 spreads a decode step's router over E
// workgroups (E x 8 KB of router rows at H = 4096); larger EB read each token
// row EB times less often, where many tokens would otherwise make E x T
// workgroups that each fetch a whole token row for one logit, and TB = 2 at
// EB = 8 halves the router-row reads again.
template <int ACT, int EB, int TB>
__global__ __launch_bounds__(256) void router_logits_small_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  float* __restrict__ logits, int T, int H, int E,
                                                                  int act, const float* __restrict__ health,
                                                                  float alpha) {
  __shared__ float part[TB][EB][4];
  const int e0 = blockIdx.x * EB, t0 = blockIdx.y * TB;
  const int lane = lane_id(), wave = wave_id();
  const int q = H / 4;
  const uint16_t* xr[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) xr[b] = x + (size_t)min(t0 + b, T - 1) * H + wave * q;  // past T: re-read
  const uint16_t* wrow[EB];
#pragma unroll
  for (int j = 0; j < EB; ++j) wrow[j] = wr + (size_t)min(e0 + j, E - 1) * H + wave * q;  // past E: re-read
  // up to four slices per lane per round, all loaded before the sums (which
  // run slice by slice in order, as one slice at a time would)
  float acc[TB][EB];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int j = 0; j < EB; ++j) acc[b][j] = 0.0f;
  // one slice of each token row (converted once) against the same slice of
  // every expert row
  auto slice = [&](const u32x4* xr8, const u32x4* wr8) __attribute__((always_inline)) {
    float xv[TB][8];
#pragma unroll
    for (int b = 0; b < TB; ++b) unpack8(xr8[b], ACT, xv[b]);
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      float wv[8];
      unpack8(wr8[j], ACT, wv);
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[b][j] = fmaf(xv[b][i], wv[i], acc[b][j]);
    }
  };
  constexpr int R = EB <= 2 ? 4 : 2;  // slices per round (registers: (TB + EB) * R loads)
  int h = lane * 8;
  for (; h + (R - 1) * 512 < q; h += R * 512) {
    u32x4 xa[R][TB], wa[R][EB];
#pragma unroll
    for (int u = 0; u < R; ++u) {
#pragma unroll
      for (int b = 0; b < TB; ++b) xa[u][b] = load16(xr[b] + h + 512 * u);
#pragma unroll
      for (int j = 0; j < EB; ++j) wa[u][j] = load16(wrow[j] + h + 512 * u);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < R; ++u) slice(xa[u], wa[u]);
  }
  if (h < q) {
    // the remaining one to R-1 slices of this lane, loaded together
    u32x4 xa[R - 1][TB], wa[R - 1][EB];
#pragma unroll
    for (int u = 0; u < R - 1; ++u)
      if (h + 512 * u < q) {
#pragma unroll
        for (int b = 0; b < TB; ++b) xa[u][b] = load16(xr[b] + h + 512 * u);
#pragma unroll
        for (int j = 0; j < EB; ++j) wa[u][j] = load16(wrow[j] + h + 512 * u);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < R - 1; ++u)
      if (h + 512 * u < q) slice(xa[u], wa[u]);
  }
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const float s = wave_sum(acc[b][j]);
      if (lane == 0) part[b][j][wave] = s;
    }
  __syncthreads();
  if (threadIdx.x < TB * EB) {
    const int b = threadIdx.x / EB, j = threadIdx.x % EB, e = e0 + j, t = t0 + b;
    if (e < E && t < T) {
      float l = ((part[b][j][0] + part[b][j][1]) + part[b][j][2]) + part[b][j][3];
      if (health) l = l - alpha * health[e];
      logits[(size_t)t * E + e] = l;
    }
  }
}

// ---------------------------------------------------------- large batches --
//
// One workgroup per 32-token x 32-expert tile on the matrix cores: the NW
// waves take consecutive parts of H (split K), each accumulating a 32x32
// fp32 tile with v_mfma_f32_32x32x16_{f16,bf16} fed straight from memory
// (lane l supplies row l%32 and 8 consecutive k), and the partial tiles are
// added in wave order through LDS.  Products of two fp16 (bf16) values are
// exact in fp32; only the summation order differs from a sequential sum.
// Sixteen waves (H % 256 == 0, fewer tiles than CUs) keep a wave's share of
// H to a few k-steps whose loads all go out at once: the tile count is small
// (16 tiles for 512 tokens and 32 experts), so the kernel is bound by load
// latency.  Four waves take the rest.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int ACT, int NW>
__global__ __launch_bounds__(64 * NW) void router_logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ wr,
                                                                     float* __restrict__ logits, int T, int H, int E,
                                                                     const float* __restrict__ health, float alpha) {
  __shared__ float part[NW - 1][16][WAVE];
  const int lane = lane_id(), wave = wave_id();
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int r32 = lane % 32, half = lane / 32;
  const int t = min(t0 + r32, T - 1), e = min(e0 + r32, E - 1);  // past the end: re-read (not stored)
  const int q = H / NW;
  const uint16_t* xa = x + (size_t)t * H + wave * q + half * 8;
  const uint16_t* wb = wr + (size_t)e * H + wave * q + half * 8;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  // eight k-steps per round: all sixteen loads go out before the MFMAs
  // (the same accumulation order as one step at a time)
  auto mfma = [&](u32x4 av, u32x4 bv) __attribute__((always_inline)) {
    if constexpr (ACT == ACT_BF16)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                    acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), acc,
                                                   0, 0, 0);
  };
  constexpr int KU = 8;
  int k = 0;
  for (; k + 16 * KU <= q; k += 16 * KU) {
    u32x4 av[KU], bv[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      av[u] = load16(xa + k + 16 * u);
      bv[u] = load16(wb + k + 16 * u);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
#pragma unroll
    for (int u = 0; u < KU; ++u) mfma(av[u], bv[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; k < q; k += 16) mfma(load16(xa + k), load16(wb + k));
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) part[wave - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (wave == 0) {
    // register i of lane l: token row 8*(i/4) + 4*(l/32) + i%4, expert column l%32
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = acc[i];
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) v = v + part[w][i][lane];
      const int tt = t0 + 8 * (i / 4) + 4 * half + (i % 4), ee = e0 + r32;
      if (health) v = v - alpha * health[e];  // e = min(ee, E - 1): equal to ee where stored
      if (tt < T && ee < E) logits[(size_t)tt * E + ee] = v;
    }
  }
}

// ------------------------------------------------------------- selection --

__global__ __launch_bounds__(256) void topk_static_kernel(const float* __restrict__ logits, int T, int E, int k, int gs,
                                                          int32_t* __restrict__ idx, float* __restrict__ w,
                                                          int32_t* __restrict__ k_used, float* __restrict__ entropy,
                                                          int32_t* __restrict__ clear_word) {
  const int t = blockIdx.x * 4 + wave_id();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (k_used) *k_used = k;
    if (entropy) *entropy = 0.0f;
    if (clear_word) *clear_word = 0;
  }
  if (t >= T) return;
  int si[MOE_MAX_K_DEV];
  float sw[MOE_MAX_K_DEV];
  route_token(logits + (size_t)t * E, E, k, si, sw, gs);
  if (lane_id() == 0) {
#pragma unroll
    for (int s = 0; s < MOE_MAX_K_DEV; ++s)
      if (s < k) {
        idx[(size_t)t * k + s] = si[s];
        w[(size_t)t * k + s] = sw[s];
      }
  }
}

// E <= 64: one wave selects for four tokens, sixteen lanes each (lane i of
// row r holds experts i, i+16, i+32, i+48 of token 4*wave + r).  A row
// reduction over sixteen lanes needs four DPP steps and no lane reads, so a
// token costs about a quarter of the instructions of wave_topk.  The order of
// the candidates is total, so the same experts are chosen, and the weights
// are formed with the same operations in slot order: the same bits as
// topk_static_kernel.
// The k best of one token's E <= 64 logits over the sixteen lanes of a row
// (lane i holds experts i, i+16, i+32, i+48); every lane of the row receives
// the selected logits and indices in slot order.  No live candidate (a token
// past T) gives index -1.
__device__ __forceinline__ void row16_topk(const float* __restrict__ row, bool tv, int E, int k, int gs, int i16,
                                           float* sv, int* si) {
  float v[4];
  bool live[4];
  int grp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = i16 + 16 * j;
    live[j] = tv && e < E;
    v[j] = live[j] ? row[e] : 0.0f;
    grp[j] = e / gs;
  }
#pragma unroll
  for (int s = 0; s < MOE_MAX_K_DEV; ++s) {
    if (s < k) {
      Cand c = {0.0f, -1};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Cand d = {v[j], live[j] ? i16 + 16 * j : -1};
        c = better(c, d);
      }
      c = better(c, dpp_cand<DPP_QUAD_1032>(c));
      c = better(c, dpp_cand<DPP_QUAD_2301>(c));
      c = better(c, dpp_cand<DPP_ROW_HALF_MIRROR>(c));
      c = better(c, dpp_cand<DPP_ROW_MIRROR>(c));
      sv[s] = c.v;
      si[s] = c.i;
      const int cg = c.i / gs;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (grp[j] == cg) live[j] = false;
    }
  }
}

// slots [0, kc) of token t: the k selected experts with exp(l_s - l_1) / z
// (z summed in slot order, as route_token), then index -1 and weight 0
__device__ __forceinline__ void row16_store(int32_t* __restrict__ idx, float* __restrict__ w, int64_t t, int k, int kc,
                                            const float* sv, const int* si) {
  float ex[MOE_MAX_K_DEV];
  float z = 0.0f;
#pragma unroll
  for (int s = 0; s < MOE_MAX_K_DEV; ++s) {
    if (s < k) {
      ex[s] = expf(sv[s] - sv[0]);
      z += ex[s];
    }
  }
#pragma unroll
  for (int s = 0; s < MOE_MAX_K_DEV; ++s)
    if (s < kc) {
      idx[t * kc + s] = s < k ? si[s] : -1;
      w[t * kc + s] = s < k ? ex[s] / z : 0.0f;
    }
}

__global__ __launch_bounds__(256) void topk_static_rows_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                               int gs, int32_t* __restrict__ idx,
                                                               float* __restrict__ w, int32_t* __restrict__ k_used,
                                                               float* __restrict__ entropy,
                                                               int32_t* __restrict__ clear_word) {
  const int lane = lane_id(), r = lane / 16, i16 = lane % 16;
  const int t = (blockIdx.x * 4 + wave_id()) * 4 + r;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (k_used) *k_used = k;
    if (entropy) *entropy = 0.0f;
    if (clear_word) *clear_word = 0;
  }
  // every lane stays active for the row reductions; tokens past T have no
  // live candidate and store nothing
  const bool tv = t < T;
  float sv[MOE_MAX_K_DEV];
  int si[MOE_MAX_K_DEV];
  row16_topk(logits + (size_t)(tv ? t : 0) * E, tv, E, k, gs, i16, sv, si);
  if (i16 == 0 && tv) row16_store(idx, w, t, k, k, sv, si);
}

// Shannon entropy (nats) of softmax(row): H = ln Z - sum_e p_e (l_e - l_max)
__device__ __forceinline__ float wave_entropy(const float* __restrict__ row, int E) {
  const int lane = lane_id();
  float v[4];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  m = wave_max(m);
  float z = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (lane + 64 * j < E) {
      const float d = v[j] - m;
      const float p = expf(d);
      z += p;
      s1 += p * d;
    }
  }
  z = wave_sum(z);
  s1 = wave_sum(s1);
  return logf(z) - s1 / z;
}

// One workgroup of 16 waves.  Wave w handles tokens w, w+16, ...; its
// entropies are summed in token order, the 16 wave partials in wave order,
// so the batch entropy does not depend on timing.
__global__ __launch_bounds__(1024) void topk_entropy_kernel(const float* __restrict__ logits, int T, int E, int gs,
                                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                                            int32_t* __restrict__ k_used,
                                                            float* __restrict__ entropy,
                                                            int32_t* __restrict__ clear_word) {
  __shared__ float part[16];
  __shared__ int k_sh;
  const int wave = wave_id();
  if (clear_word && threadIdx.x == 0) *clear_word = 0;
  float hs = 0.0f;
  for (int t = wave; t < T; t += 16) hs += wave_entropy(logits + (size_t)t * E, E);
  if (lane_id() == 0) part[wave] = hs;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.0f;
    for (int i = 0; i < 16; ++i) tot += part[i];
    const float h = tot / (float)T;
    const int k = h < 1.2f ? 1 : (h < 2.5f ? 2 : 3);
    k_sh = k;
    if (k_used) *k_used = k;
    if (entropy) *entropy = h;
  }
  __syncthreads();
  const int k = k_sh;
  constexpr int KC = MOE_K_ENTROPY_CAP_DEV;
  for (int t = wave; t < T; t += 16) {
    int si[MOE_MAX_K_DEV];
    float sw[MOE_MAX_K_DEV];
    route_token(logits + (size_t)t * E, E, k, si, sw, gs);
    if (lane_id() == 0) {
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        idx[(size_t)t * KC + s] = si[s];
        w[(size_t)t * KC + s] = sw[s];
      }
    }
  }
}

// Parallel form of the adaptive selection, in two launches.  First one wave
// per token writes the token's entropy to scratch.  Then every workgroup sums
// the T entropies in the same fixed order (lane l takes tokens l, l+64, ...
// in order; the lanes are combined by the DPP butterfly), so all of them
// reach the same batch entropy and k, and selects its own tokens.
__global__ __launch_bounds__(256) void entropy_tokens_kernel(const float* __restrict__ logits, int T, int E,
                                                             float* __restrict__ hent, int32_t* __restrict__ clear_word) {
  if (clear_word && blockIdx.x == 0 && threadIdx.x == 0) *clear_word = 0;
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  const float h = wave_entropy(logits + (size_t)t * E, E);
  if (lane_id() == 0) hent[t] = h;
}

__global__ __launch_bounds__(256) void entropy_select_kernel(const float* __restrict__ logits, int T, int E, int gs,
                                                             const float* __restrict__ hent,
                                                             int32_t* __restrict__ idx, float* __restrict__ w,
                                                             int32_t* __restrict__ k_used,
                                                             float* __restrict__ entropy) {
  __shared__ int k_sh;
  const int wave = wave_id(), lane = lane_id();
  if (wave == 0) {
    // lane l adds hent[l], hent[l + 64], ... in order; eight of them are
    // loaded together (one memory round trip per eight instead of per value)
    float s = 0.0f;
    int i = lane;
    for (; i + 7 * WAVE < T; i += 8 * WAVE) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hent[i + u * WAVE];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; i < T; i += WAVE) s += hent[i];
    const float h = wave_sum(s) / (float)T;
    const int k = h < 1.2f ? 1 : (h < 2.5f ? 2 : 3);
    if (lane == 0) {
      k_sh = k;
      if (blockIdx.x == 0) {
        if (k_used) *k_used = k;
        if (entropy) *entropy = h;
      }
    }
  }
  __syncthreads();
  const int k = k_sh;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  constexpr int KC = MOE_K_ENTROPY_CAP_DEV;
  int si[MOE_MAX_K_DEV];
  float sw[MOE_MAX_K_DEV];
  route_token(logits + (size_t)t * E, E, k, si, sw, gs);
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      idx[(size_t)t * KC + s] = si[s];
      w[(size_t)t * KC + s] = sw[s];
    }
  }
}

// ------------------------------------------------------------- launchers --

// The small-batch kernel up to 16384 logits (measured at H = 4096 with one
// logit per workgroup: 9.4 us against 19.6 us for the tiled kernel at 256
// tokens x 32 experts, 12.2 against 18.8 at 512 x 32, and 10.3 us at 512 x 32
// with eight experts per workgroup; above that the tiled kernel wins).  The
// tiled kernel's loads take 32 B of each of 32 rows per instruction, so its
// sixteen waves' working set outgrows the vector L1 and it settles near 19 us
// whatever the size up to 1024 x 64.
bool router_use_small(int T, int E) { return T <= 128 || (int64_t)T * E <= 16384; }

hipError_t launch_router_logits(const void* x, const void* wr, float* logits, int T, int H, int E, int act,
                                const float* health, float alpha, hipStream_t st) {
  if (!router_use_small(T, E)) {
    dim3 grid((T + 31) / 32, (E + 31) / 32);
    const uint16_t* xs = (const uint16_t*)x;
    const uint16_t* ws = (const uint16_t*)wr;
    // sixteen waves per tile while the tiles are few (each wave's loads then
    // all go out in one or two rounds); four once there is a tile per CU,
    // where the sixteen waves' rows overflow the vector L1 (4096 tokens x 64
    // experts: 23.1-23.4 against 25.2-25.6 us)
    if (H % (16 * 16) == 0 && (int64_t)grid.x * grid.y < 256) {
      if (act == ACT_BF16)
        return launch_kernel(router_logits_mfma_kernel<ACT_BF16, 16>, grid, 1024, 0, st, xs, ws, logits, T, H, E, health,
                             alpha);
      return launch_kernel(router_logits_mfma_kernel<ACT_F16, 16>, grid, 1024, 0, st, xs, ws, logits, T, H, E, health,
                           alpha);
    }
    if (act == ACT_BF16)
      return launch_kernel(router_logits_mfma_kernel<ACT_BF16, 4>, grid, 256, 0, st, xs, ws, logits, T, H, E, health,
                           alpha);
    return launch_kernel(router_logits_mfma_kernel<ACT_F16, 4>, grid, 256, 0, st, xs, ws, logits, T, H, E, health,
                         alpha);
  }
  // experts per workgroup: one while the logits alone give at most 1024
  // workgroups, then enough to keep about a thousand
  const int64_t n = (int64_t)T * E;
  const int eb = n <= 1024 ? 1 : n <= 2048 ? 2 : n <= 4096 ? 4 : 8;
  // two tokens per workgroup at eight experts: each router row is read half
  // as often (512 tokens x 32 experts: 8.7 against 10.4 us; four tokens, 9.7)
  const int tk = tuning(TUNE_ROUTER_TOKENS);
  const int tb = eb < 8 ? 1 : (tk == 1 || tk == 4 ? tk : 2);
  auto go = [&](auto kern, int b, int tbk) {
    launch_kernel(kern, dim3((E + b - 1) / b, (T + tbk - 1) / tbk), 256, 0, st, (const uint16_t*)x,
                  (const uint16_t*)wr, logits, T, H, E, act, health, alpha);
  };
  if (act == ACT_BF16) {
    if (eb == 1) go(router_logits_small_kernel<ACT_BF16, 1, 1>, 1, 1);
    else if (eb == 2) go(router_logits_small_kernel<ACT_BF16, 2, 1>, 2, 1);
    else if (eb == 4) go(router_logits_small_kernel<ACT_BF16, 4, 1>, 4, 1);
    else if (tb == 4) go(router_logits_small_kernel<ACT_BF16, 8, 4>, 8, 4);
    else if (tb == 2) go(router_logits_small_kernel<ACT_BF16, 8, 2>, 8, 2);
    else go(router_logits_small_kernel<ACT_BF16, 8, 1>, 8, 1);
  } else {
    if (eb == 1) go(router_logits_small_kernel<ACT_F16, 1, 1>, 1, 1);
    else if (eb == 2) go(router_logits_small_kernel<ACT_F16, 2, 1>, 2, 1);
    else if (eb == 4) go(router_logits_small_kernel<ACT_F16, 4, 1>, 4, 1);
    else if (tb == 4) go(router_logits_small_kernel<ACT_F16, 8, 4>, 8, 4);
    else if (tb == 2) go(router_logits_small_kernel<ACT_F16, 8, 2>, 8, 2);
    else go(router_logits_small_kernel<ACT_F16, 8, 1>, 8, 1);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int gs, int32_t* idx, float* w, int32_t* k_used,
                       float* entropy, float* scratch, hipStream_t st, int32_t* clear_word) {
  if (k <= 0 && scratch) {
    const unsigned g = (unsigned)((T + 3) / 4);
    hipError_t e = launch_kernel(entropy_tokens_kernel, g, 256, 0, st, logits, T, E, scratch, clear_word);
    if (e != hipSuccess) return e;
    return launch_kernel(entropy_select_kernel, g, 256, 0, st, logits, T, E, gs, (const float*)scratch, idx, w,
                         k_used, entropy);
  }
  if (k > 0) {
    if (E <= 64)
      launch_kernel(topk_static_rows_kernel, (T + 15) / 16, 256, 0, st, logits, T, E, k, gs, idx, w, k_used, entropy,
                    clear_word);
    else
      launch_kernel(topk_static_kernel, (T + 3) / 4, 256, 0, st, logits, T, E, k, gs, idx, w, k_used, entropy,
                    clear_word);
  } else {
    launch_kernel(topk_entropy_kernel, 1, 1024, 0, st, logits, T, E, gs, idx, w, k_used, entropy, clear_word);
  }
  return hipGetLastError();
}

// ------------------------------------------------------- load statistics --
//
// One wave.  Lane l holds the counts of experts l, l+64, l+128, l+192: the
// least-used expert is the smallest (count, index) over the wave; the
// standard deviation is sqrt(sum_e (c_e - mean)^2 / E) with the mean from the
// exact integer total and the squares summed in fp64 (page "Qwen3.5-MoE与
// Qwen3-MoE架构差异深度解析", closing advice: watch the least-activated expert
// and the standard deviation of the activation counts).  E <= 256.
__global__ __launch_bounds__(64) void load_stats_kernel(const int32_t* __restrict__ counts, int E,
                                                         int32_t* __restrict__ least_used, float* __restrict__ sd) {
  const int lane = lane_id();
  int c[4];
  int64_t s1 = 0;
  int best_c = 0, best_e = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + WAVE * j;
    c[j] = e < E ? counts[e] : 0;
    s1 += c[j];
    if (e < E && (best_e < 0 || c[j] < best_c)) {  // e grows with j: a lane keeps its lowest index among equals
      best_c = c[j];
      best_e = e;
    }
  }
  for (int off = 1; off < WAVE; off <<= 1) {
    s1 += __shfl_xor(s1, off);
    const int oc = __shfl_xor(best_c, off), oe = __shfl_xor(best_e, off);
    const bool take = oe >= 0 && (best_e < 0 || oc < best_c || (oc == best_c && oe < best_e));
    best_c = take ? oc : best_c;
    best_e = take ? oe : best_e;
  }
  const double mean = (double)s1 / (double)E;
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane + WAVE * j < E) {
      const double d = (double)c[j] - mean;
      ss += d * d;
    }
  for (int off = 1; off < WAVE; off <<= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) {
    *least_used = best_e;
    *sd = (float)sqrt(ss / (double)E);
  }
}

hipError_t launch_load_stats(const int32_t* counts, int E, int32_t* least_used, float* stddev, hipStream_t st) {
  return launch_kernel(load_stats_kernel, 1, 64, 0, st, counts, E, least_used, stddev);
}

}  // namespace moe

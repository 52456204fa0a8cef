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
// One workgroup per (expert, token); its four waves take consecutive quarters
// of H, each lane sums its 8-element slices in order, the wave sums its lanes,
// and the four wave partials are added in wave order.  Spreads a decode
// step's router over E workgroups (E x 8 KB of router rows at H = 4096).
__global__ __launch_bounds__(256) void router_logits_small_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  float* __restrict__ logits, int H, int E,
                                                                  int act) {
  __shared__ float part[4];
  const int e = blockIdx.x, t = blockIdx.y;
  const int lane = lane_id(), wave = wave_id();
  const int q = H / 4;
  const uint16_t* xr = x + (size_t)t * H + wave * q;
  const uint16_t* wrow = wr + (size_t)e * H + wave * q;
  float acc = 0.0f;
#pragma unroll 4
  for (int h = lane * 8; h < q; h += 512) {
    float xv[8], wv[8];
    unpack8(load16(xr + h), act, xv);
    unpack8(load16(wrow + h), act, wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(xv[i], wv[i], acc);
  }
  const float s = wave_sum(acc);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) logits[(size_t)t * E + e] = ((part[0] + part[1]) + part[2]) + part[3];
}

// ---------------------------------------------------------- large batches --
//
// A wave computes a 4-token x 4-expert tile; lane l owns the 8-element column
// slices h = 8*l + 512*i.
__global__ __launch_bounds__(256) void router_logits_tile_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wr,
                                                                 float* __restrict__ logits, int T, int H, int E,
                                                                 int act) {
  constexpr int TT = 4;
  const int lane = lane_id();
  const int wave = wave_id();
  const int t0 = blockIdx.x * TT;
  const int e0 = blockIdx.y * 16 + wave * 4;
  if (e0 >= E) return;
  float acc[TT][4];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;

  for (int h = lane * 8; h < H; h += 512) {
    float xv[TT][8], wv[4][8];
#pragma unroll
    for (int a = 0; a < TT; ++a) {
      const int t = min(t0 + a, T - 1);
      unpack8(load16(x + (size_t)t * H + h), act, xv[a]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = min(e0 + b, E - 1);
      unpack8(load16(wr + (size_t)e * H + h), act, wv[b]);
    }
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[a][b] = fmaf(xv[a][i], wv[b][i], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float s = wave_sum(acc[a][b]);
      const int t = t0 + a, e = e0 + b;
      if (lane == 0 && t < T && e < E) logits[(size_t)t * E + e] = s;
    }
}

// ------------------------------------------------------------- selection --

__global__ __launch_bounds__(256) void topk_static_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ w,
                                                          int32_t* __restrict__ k_used, float* __restrict__ entropy) {
  const int t = blockIdx.x * 4 + wave_id();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (k_used) *k_used = k;
    if (entropy) *entropy = 0.0f;
  }
  if (t >= T) return;
  int si[MOE_MAX_K_DEV];
  float sw[MOE_MAX_K_DEV];
  route_token(logits + (size_t)t * E, E, k, si, sw);
  if (lane_id() == 0) {
#pragma unroll
    for (int s = 0; s < MOE_MAX_K_DEV; ++s)
      if (s < k) {
        idx[(size_t)t * k + s] = si[s];
        w[(size_t)t * k + s] = sw[s];
      }
  }
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
__global__ __launch_bounds__(1024) void topk_entropy_kernel(const float* __restrict__ logits, int T, int E,
                                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                                            int32_t* __restrict__ k_used,
                                                            float* __restrict__ entropy) {
  __shared__ float part[16];
  __shared__ int k_sh;
  const int wave = wave_id();
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
    route_token(logits + (size_t)t * E, E, k, si, sw);
    if (lane_id() == 0) {
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        idx[(size_t)t * KC + s] = si[s];
        w[(size_t)t * KC + s] = sw[s];
      }
    }
  }
}

// ------------------------------------------------------------- launchers --

int router_small_max_tokens() { return 16; }

hipError_t launch_router_logits(const void* x, const void* wr, float* logits, int T, int H, int E, int act,
                                hipStream_t st) {
  if (T <= router_small_max_tokens()) {
    launch_kernel(router_logits_small_kernel, dim3(E, T), 256, 0, st, (const uint16_t*)x, (const uint16_t*)wr, logits, H, E,
                                                            act);
  } else {
    dim3 grid((T + 3) / 4, (E + 15) / 16);
    launch_kernel(router_logits_tile_kernel, grid, 256, 0, st, (const uint16_t*)x, (const uint16_t*)wr, logits, T, H, E, act);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, int32_t* k_used,
                       float* entropy, hipStream_t st) {
  if (k > 0) {
    launch_kernel(topk_static_kernel, (T + 3) / 4, 256, 0, st, logits, T, E, k, idx, w, k_used, entropy);
  } else {
    launch_kernel(topk_entropy_kernel, 1, 1024, 0, st, logits, T, E, idx, w, k_used, entropy);
  }
  return hipGetLastError();
}

}  // namespace moe
